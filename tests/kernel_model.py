"""NumPy model of the FP8 prefill indexer kernel's score arithmetic (test infrastructure).

It exists only to check, on the CPU, that the parity bound of tests/dsa_check.py covers what the
kernel computes and is tight enough to catch a kernel that drops part of the work. It models the
kernel; it does not define the score (the oracle does) and nothing outside tests/ uses it.

The kernel evaluates, per query row and key,
    sum_j w_j ReLU(x_j) = 1/2 sum_j w_j |x_j| + 1/2 u . k,   x_j = qI_j . k,  u = sum_j w_j qI_j
with u split into four FP8 E4M3 pieces:
  * u = fma(w_j, qI_j, u) over j = 0..63 in fp32;
  * e from frexp(max_d |u_d|) minus 8 (floored at -112), so that max |u| 2^-e lies in [128, 256);
  * rem_0 = u 2^-e; piece p = round-to-nearest-even E4M3 value of rem_p, rem_{p+1} = 16 (rem_p - piece p);
  * the linear tile of lane group p is 2^(e-1-4p) * (piece p . k) (an E8M0 operand scale);
  * lane group p accumulates its linear tile, then fma(w_j / 2, |x_j|, .) for the heads j = 4 mm + p,
    mm = 0..15, in that order;
  * the score of key kappa of a 16-key block is (A_p + A_{p^2}) + (A_{p^1} + A_{p^3}) with
    p = kappa % 4 (two cross-lane steps inside a quad).
The 128-term FP8 dot products are taken exactly and rounded to fp32, optionally perturbed by
`mfma_rel` * sum_d |a_d b_d| with random signs: the matrix instruction adds its products with
less than fp32 precision, and `mfma_rel` stands for its measured worst error rate.
"""
from __future__ import annotations

import numpy as np

import oracle


def _fma32(a, b, c):
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64)).astype(np.float32)


def round_e4m3(r: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even onto the E4M3 grid (|r| < 448), through torch's own cast."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(r, np.float32)).to(torch.float8_e4m3fn).to(torch.float32).numpy()


def linear_pieces(qI_row_codes, w_row):
    """(pieces [4, d_I] float32 values, e) of the row's linear term, as the kernel splits it."""
    q = oracle.decode(qI_row_codes).astype(np.float32)       # exact: e4m3 values are fp32 values
    w = np.asarray(w_row, np.float32)
    u = np.zeros(q.shape[1], np.float32)
    for j in range(q.shape[0]):
        u = _fma32(w[j], q[j], u)
    mx = float(np.max(np.abs(u)))
    e = 0
    if mx > 0.0:
        _, e = np.frexp(np.float32(mx))
        e = max(int(e) - 8, -112)
    rem = np.ldexp(u, -e).astype(np.float32)
    pieces = []
    for _ in range(4):
        v = round_e4m3(rem)
        pieces.append(v)
        rem = ((rem - v) * np.float32(16.0)).astype(np.float32)
    return np.stack(pieces), e


def prefill_scores(qI_row_codes, kI_codes, w_row, mfma_rel=0.0, rng=None, drop_head=None, drop_piece=None):
    """Model of the kernel's scores of one row against the keys kI_codes [n, d_I] (positions 0..n-1)."""
    q = oracle.decode(qI_row_codes)                          # [H_I, d_I]
    k = oracle.decode(kI_codes)                              # [n, d_I]
    w = np.asarray(w_row, np.float32)
    H_I = q.shape[0]
    pieces, e = linear_pieces(qI_row_codes, w_row)
    n = k.shape[0]

    def mfma(a):
        exact = k @ np.asarray(a, np.float64)
        if mfma_rel:
            exact = exact + rng.choice([-1.0, 1.0], size=n) * mfma_rel * (np.abs(k) @ np.abs(a))
        return exact.astype(np.float32)

    A = []
    for p in range(4):
        lin = (mfma(pieces[p]).astype(np.float64) * 2.0 ** (e - 1 - 4 * p)).astype(np.float32)
        if drop_piece == p:
            lin = np.zeros(n, np.float32)
        acc = lin
        for mm in range(H_I // 4):
            j = 4 * mm + p
            if j == drop_head:
                continue
            acc = _fma32(np.float32(0.5) * w[j], np.abs(mfma(q[j])), acc)
        A.append(acc)
    A = np.stack(A)                                          # [4, n]
    kappa = np.arange(n) % 4
    out = np.empty(n, np.float32)
    for p in range(4):
        sel = kappa == p
        a = (A[p, sel] + A[p ^ 2, sel]).astype(np.float32)
        b = (A[p ^ 1, sel] + A[p ^ 3, sel]).astype(np.float32)
        out[sel] = (a + b).astype(np.float32)
    return out
