"""Pure-Python loop versions of the DSA steps for tiny inputs (test infrastructure only).

These cross-check the vectorised oracle in `oracle.dsa` with different code: explicit loops
over heads, dims and keys, top-k by counting for every candidate how many candidates rank above
it (no sorting), and a softmax written with math.exp. Inputs are plain nested lists of floats.
"""
from __future__ import annotations

import math


def indexer_row(qI_r, keys, w_r):
    """qI_r: H_I lists of d_I floats; keys: list of d_I-float lists (the causal prefix)."""
    out = []
    for key in keys:
        acc = 0.0
        for j, qv in enumerate(qI_r):
            dot = 0.0
            for a, b in zip(qv, key):
                dot += a * b
            acc += w_r[j] * (dot if dot > 0.0 else 0.0)
        out.append(acc)
    return out


def topk_by_rank(scores, k):
    """Position s is kept iff fewer than k candidates rank above it, where t ranks above s when
    scores[t] > scores[s], or scores[t] == scores[s] and t < s. Ascending, padded with -1."""
    n = len(scores)
    keep = []
    for s in range(n):
        above = 0
        for t in range(n):
            if scores[t] > scores[s] or (scores[t] == scores[s] and t < s):
                above += 1
        if above < k:
            keep.append(s)
    return keep + [-1] * (k - len(keep))


def attn_row(q_r, rows, scale, d_v):
    """q_r: H lists of d_qk floats; rows: the selected latent rows (lists of d_qk floats)."""
    H = len(q_r)
    if not rows:
        return [[0.0] * d_v for _ in range(H)], [-math.inf] * H
    outs, lses = [], []
    for h in range(H):
        z = []
        for c in rows:
            acc = 0.0
            for a, b in zip(q_r[h], c):
                acc += a * b
            z.append(scale * acc)
        m = max(z)
        e = [math.exp(v - m) for v in z]
        l = sum(e)
        o = [0.0] * d_v
        for p, c in zip(e, rows):
            for d in range(d_v):
                o[d] += (p / l) * c[d]
        outs.append(o)
        lses.append(m + math.log(l))
    return outs, lses


def alignment_row(q_r, rows, scale, scores_sel):
    """Head-averaged attention distribution over the given latent rows and its KL divergence from
    the softmax of the indexer scores of the same rows. Loops and math.exp / math.log only."""
    n = len(rows)
    if n == 0:
        return [], 0.0
    H = len(q_r)
    p = [0.0] * n
    for h in range(H):
        z = []
        for c in rows:
            acc = 0.0
            for a, b in zip(q_r[h], c):
                acc += a * b
            z.append(scale * acc)
        m = max(z)
        e = [math.exp(v - m) for v in z]
        tot = sum(e)
        for i in range(n):
            p[i] += e[i] / tot / H
    mi = max(scores_sel)
    ei = [math.exp(v - mi) for v in scores_sel]
    ti = sum(ei)
    kl = 0.0
    for i in range(n):
        if p[i] > 0.0:
            kl += p[i] * (math.log(p[i]) - math.log(ei[i] / ti))
    return p, kl
