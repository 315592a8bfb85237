"""Vectorised float64 oracle of the DSA forward path (test infrastructure only).

Sources (page titles and sections; the pages print no code and no worked example):
  [digest]  "DeepSeek-V3.2: Pushing the Frontier of Open Large Language Models", paper digest,
            "Key claims" (paper section 2.1, Eq. 1-2 and Fig. 2) and "Method".
  [36kr]    "A paper signed by Liang Wenfeng: The most powerful open-source Agent model of
            DeepSeek has made a big splash" (36kr), section "02. Built on the final version of
            DeepSeek-V3.1, DSA makes model computation smarter".
  [blog]    "DeepSeek-V3.2 Series Open Source, Performance Rivals Gemini-3.0-Pro" (aitoearn),
            "Technical Innovations in V3.2" and "Training Process", Phase 2 (each query token
            selects 2,048 key-value entries).

Conventions (readings where the pages are silent; each is listed with its reason in the design
notes of the repository):
  * Sequence b has m_b query rows and n_b keys; query i of b sits at position pos = n_b - m_b + i
    and its candidates are keys s = 0..pos (inclusive: the tokens before the query are read as
    the causal prefix including the token itself, otherwise position 0 has nothing to attend to).
  * Scores are float64; no scale factors are applied to the FP8 inputs.
  * Top-k: the min(k, pos+1) candidates with the largest score; equal scores prefer the lower
    position (+0 and -0 are equal); the chosen positions are returned in ascending order and the
    list is padded to k with -1.
  * Attention: key = all d_qk dims of the selected latent row, value = its first d_v dims;
    logits = scale * q . key with a natural-base softmax; lse = max + ln(sum of exp).
    Index -1 and indices outside [0, n_b) are skipped; a row with no valid index gives out = 0 and
    lse = -inf. Repeated indices count as many times as they appear.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .numerics import decode


@dataclass
class Seqs:
    """Ragged batch description: cumulative query / key row counts per sequence."""
    cu_seqlens_q: np.ndarray
    cu_seqlens_k: np.ndarray

    def __post_init__(self):
        self.cu_seqlens_q = np.asarray(self.cu_seqlens_q, np.int64)
        self.cu_seqlens_k = np.asarray(self.cu_seqlens_k, np.int64)

    @property
    def num_seqs(self):
        return len(self.cu_seqlens_q) - 1

    @property
    def T(self):
        return int(self.cu_seqlens_q[-1])

    def locate(self, r: int):
        """Query row r -> (sequence b, position pos, first key row of b, n_b)."""
        b = int(np.searchsorted(self.cu_seqlens_q, r, side="right") - 1)
        m = self.cu_seqlens_q[b + 1] - self.cu_seqlens_q[b]
        n = self.cu_seqlens_k[b + 1] - self.cu_seqlens_k[b]
        i = r - self.cu_seqlens_q[b]
        return b, int(n - m + i), int(self.cu_seqlens_k[b]), int(n)


# ------------------------------------------------------------------ step 1: lightning indexer

def indexer_scores_row(seqs: Seqs, qI, kI, w, r: int, q_scale=None, k_scale=None) -> np.ndarray:
    """I[r, s] for s = 0..pos(r) ([digest] Key claims, Eq. 1; [36kr] section 02).

    I[r, s] = sum_j w[r, j] * max(0, sum_d qI[r, j, d] * kI[s, d]).
    qI: [T, H_I, d_I], kI: [Nk, d_I] (stored codes or floats), w: [T, H_I] float.
    Scaled FP8 inputs (a reading: the pages say "FP8" without a scaling scheme): the stored
    query vector of (r, j) stands for q_scale[r, j] times itself and key s for k_scale[s] times
    itself; the scores are those of the scaled vectors (q_scale [T, H_I], k_scale [Nk]).
    """
    _, pos, k0, _ = seqs.locate(r)
    q = decode(qI[r])                              # [H_I, d_I]
    keys = decode(kI[k0:k0 + pos + 1])             # [pos+1, d_I]
    if q_scale is not None:
        q = q * np.asarray(q_scale[r], np.float64)[:, None]
    if k_scale is not None:
        keys = keys * np.asarray(k_scale[k0:k0 + pos + 1], np.float64)[:, None]
    dots = q @ keys.T                              # [H_I, pos+1]
    return decode(w[r]) @ np.maximum(dots, 0.0)    # [pos+1]


def indexer_scores(seqs: Seqs, qI, kI, w, rows=None, q_scale=None, k_scale=None) -> list:
    """List of score rows (one float64 array of length pos+1 per requested row)."""
    rows = range(seqs.T) if rows is None else rows
    return [indexer_scores_row(seqs, qI, kI, w, int(r), q_scale, k_scale) for r in rows]


# ------------------------------------------------------------------ step 2: top-k selection

def topk_row(scores: np.ndarray, k: int) -> np.ndarray:
    """Top-k of one causal score row ([36kr] section 02: keep the key-value entries with the
    top-k index scores; [digest] Key claims, Eq. 2).

    Candidates are ordered by (score descending, position ascending); the first min(k, n)
    positions are returned sorted ascending and padded with -1 to length k.
    """
    scores = np.asarray(scores, np.float64)
    n = scores.shape[0]
    order = np.argsort(-scores, kind="stable")     # stable: equal scores keep position order
    take = np.sort(order[:min(k, n)])
    out = np.full(k, -1, np.int32)
    out[:take.shape[0]] = take
    return out


def topk(score_rows: list, k: int) -> np.ndarray:
    return np.stack([topk_row(s, k) for s in score_rows]) if score_rows else np.zeros((0, k), np.int32)


# ------------------------------------------------------------------ step 3: sparse MLA attention

def attn_row(seqs: Seqs, q, kv, indices_row, scale: float, d_v: int, r: int):
    """Attention of every head of query row r over its selected latent rows.

    MLA in MQA mode ([digest] Key claims, Fig. 2; Method): one latent row per key is shared by
    all query heads of the token; key = the whole row, value = its first d_v dims.
    Returns (out [H, d_v] float64, lse [H] float64).
    """
    _, _, k0, n = seqs.locate(r)
    qr = decode(q[r])                                             # [H, d_qk]
    idx = np.asarray(indices_row, np.int64)
    idx = idx[(idx >= 0) & (idx < n)]
    H = qr.shape[0]
    if idx.shape[0] == 0:
        return np.zeros((H, d_v)), np.full(H, -np.inf)
    c = decode(kv[k0 + idx])                                      # [|S|, d_qk]
    z = scale * (qr @ c.T)                                        # [H, |S|]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    out = (e / l) @ c[:, :d_v]
    lse = (m + np.log(l))[:, 0]
    return out, lse


def sparse_mla_attn(seqs: Seqs, q, kv, indices, scale: float, d_v: int, rows=None):
    """out [R, H, d_v], lse [R, H] for the requested rows (default: all)."""
    rows = list(range(seqs.T)) if rows is None else [int(r) for r in rows]
    outs, lses = [], []
    for i, r in enumerate(rows):
        o, l = attn_row(seqs, q, kv, indices[i], scale, d_v, r)
        outs.append(o)
        lses.append(l)
    if not outs:
        return np.zeros((0, 0, d_v)), np.zeros((0, 0))
    return np.stack(outs), np.stack(lses)


# ------------------------------------------------------------------ composition

def forward_rows(seqs: Seqs, qI, kI, w, q, kv, k: int, scale: float, d_v: int, rows=None,
                 q_scale=None, k_scale=None):
    """Indexer -> top-k -> attention for the requested rows.

    Returns dict(scores=list of rows, indices [R, k], out [R, H, d_v], lse [R, H]).
    """
    rows = list(range(seqs.T)) if rows is None else [int(r) for r in rows]
    sc = indexer_scores(seqs, qI, kI, w, rows, q_scale, k_scale)
    idx = topk(sc, k)
    out, lse = sparse_mla_attn(seqs, q, kv, idx, scale, d_v, rows)
    return dict(scores=sc, indices=idx, out=out, lse=lse)


# ------------------------------------------------------------------ indexer-alignment target

def alignment_row(seqs: Seqs, q, kv, indices_row, scale: float, scores_row, r: int):
    """Training target of the indexer for row r and its KL divergence from the indexer's own
    distribution ([digest] Key claims and Method, paper section 2.1.1, Eq. 3-4: the indexer is
    trained with a KL loss towards the main attention distribution aggregated over the heads --
    over all preceding keys in the dense warm-up, over the selected ones in the sparse stage).

    Readings (the pages print neither equation): the set S is the given index list restricted to
    causal candidates 0..pos (entries -1 or outside are skipped; repeats count as listed); each
    head's attention softmax over S (logits scale * q_h . c_s, natural exp) is averaged over the
    H heads, p[s] = (1/H) sum_h softmax_h[s] (the head sum renormalised); the indexer's
    distribution is softmax over S of I[r, s]; the loss is KL(p || softmax(I)) =
    sum_s p[s] (ln p[s] - ln softmax(I)[s]), with 0 ln 0 = 0.
    Returns (target [len(indices_row)] float64, 0 at skipped entries; kl float).
    """
    _, pos, k0, _ = seqs.locate(r)
    idx = np.asarray(indices_row, np.int64)
    valid = (idx >= 0) & (idx <= pos)
    target = np.zeros(idx.shape[0])
    if not valid.any():
        return target, 0.0
    sel = idx[valid]
    qr = decode(q[r])                                             # [H, d_qk]
    c = decode(kv[k0 + sel])                                      # [|S|, d_qk]
    z = scale * (qr @ c.T)                                        # [H, |S|]
    z = z - z.max(axis=1, keepdims=True)
    ph = np.exp(z)
    ph /= ph.sum(axis=1, keepdims=True)
    p = ph.mean(axis=0)                                           # [|S|]
    i_sel = np.asarray(scores_row, np.float64)[sel]
    lq = i_sel - i_sel.max()
    lq = lq - np.log(np.exp(lq).sum())                            # ln softmax(I) over S
    pos_p = p > 0
    kl = float(np.sum(p[pos_p] * (np.log(p[pos_p]) - lq[pos_p])))
    target[valid] = p
    return target, kl
