"""Comparison helpers for the parity tests (test infrastructure; uses the oracle only).

Floating-point contracts checked here:
  * indexer scores: |I_gpu - I*| <= eps[r, s] with
        eps = 2 * (delta + gamma(H_I + 1)) * sum_j |w_j| sum_d |qI_jd kI_sd|
              + 2^-29 * max_d |u_d| * sum_d |kI_sd|,          u = sum_j w_j qI_j,
    delta = accumulation error of one d_I-term dot product relative to sum_d |q k|:
    gamma(d_I) for sequential fp32, and for the FP8 matrix instruction, whose internal sum of its
    128 products is coarser than fp32, the measured worst rate times a margin (DELTA_FP8_NORMAL
    for the N(0,1)-drawn codes of the workloads, DELTA_FP8_FULL for codes over the whole e4m3
    range). The second term covers the FP8 prefill kernel's 4-piece split of u (it takes the
    score as (sum_j w_j |x_j| + u . k) / 2 with u * 2^-e, max |u| * 2^-e in [128, 256), split into
    four E4M3 pieces, leaving at most 2^-16 |u_d| + 2^-22 * 2^e per component: the relative part
    and the extra roundings fit inside the first term, the absolute part is this one).
    tests/test_score_bound.py checks this bound against a NumPy model of the kernel arithmetic,
    both ways: it covers the model, and the model with one head's term or one of the two leading
    pieces of u left out falls outside it.
    On integer-valued inputs every partial sum is exact, so scores must match bit for bit.
  * top-k: bit-exact on integer inputs; on N(0,1) inputs "eps-valid": ascending, unique,
    in range, min(k, n) entries, and no candidate outside the set beats one inside it by more
    than the two error bounds.
  * attention: against the oracle evaluated on the GPU's own (validated) index set.
"""
from __future__ import annotations

import numpy as np

import oracle
from oracle.dsa import Seqs

U = 2.0 ** -24


def gamma(n):
    return n * U / (1 - n * U)


# The gfx950 FP8 matrix instruction (v_mfma_f32_16x16x128_f8f6f4) adds its 128 products with less
# than fp32 precision. Its worst error rate max |err| / sum |a b| was measured on the box with
# the kernel's instruction and operand layout: 2^-16.1 on codes rounded from N(0,1) draws (the
# workloads' data) and 2^-13.5 on uniformly drawn codes over the whole e4m3 range. The bounds
# keep a margin above each: x4.3 and x5.7.
DELTA_FP8_NORMAL = 2.0 ** -14
DELTA_FP8_FULL = 2.0 ** -11
MFMA_RATE_NORMAL = 2.0 ** -16.1
MFMA_RATE_FULL = 2.0 ** -13.5


def fp8_delta(variant: str) -> float:
    """delta of the FP8 path for an input variant of dsa_datagen."""
    return DELTA_FP8_FULL if variant == "e4m3" else DELTA_FP8_NORMAL


def score_bound_row(sq: Seqs, qI, kI, w, r, delta, q_scale=None, k_scale=None):
    """Bound for one row. With scales, the kernels run on w' = fl(w * q_scale) (one more rounding
    per weight: at most u * S') and multiply each score by k_scale (one more rounding: u |I|)."""
    _, pos, k0, _ = sq.locate(r)
    q = np.abs(oracle.decode(qI[r]))
    keys = np.abs(oracle.decode(kI[k0:k0 + pos + 1]))
    H_I = q.shape[0]
    wr = oracle.decode(w[r])
    if q_scale is not None:
        wr = wr * np.asarray(q_scale[r], np.float64)
    S = np.abs(wr) @ (q @ keys.T)
    u = wr @ oracle.decode(qI[r])
    eps = 2.0 * (delta + gamma(H_I + 1)) * S + 2.0 ** -29 * np.max(np.abs(u)) * keys.sum(axis=1)
    if q_scale is None and k_scale is None:
        return eps
    ks = np.ones(pos + 1) if k_scale is None else np.asarray(k_scale[k0:k0 + pos + 1], np.float64)
    return ks * (eps + 2.0 * U * S) * (1 + 2.0 * U) + 2.0 * U * ks * S


def check_topk_row(got, exact_scores, eps, k, pos):
    """eps-valid check of one GPU top-k row. Returns overlap fraction with the oracle set."""
    n = pos + 1
    want = min(k, n)
    got = np.asarray(got)
    sel = got[:want]
    assert np.all(got[want:] == -1), "padding must be -1"
    assert np.all((sel >= 0) & (sel <= pos)), "index out of causal range"
    assert np.all(np.diff(sel) > 0), "indices must be strictly ascending"
    if want < n:
        inside = np.zeros(n, bool)
        inside[sel] = True
        lo_in = np.min(exact_scores[inside] + eps[inside])
        hi_out = np.max(exact_scores[~inside] - eps[~inside])
        assert lo_in >= hi_out, f"a candidate outside the set beats one inside ({hi_out} > {lo_in})"
    ref = oracle.topk_row(exact_scores, k)[:want]
    return len(np.intersect1d(ref, sel)) / max(1, want)
