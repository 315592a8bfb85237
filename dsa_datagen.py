"""Seeded synthetic inputs for the DSA forward path (indexer -> top-k -> sparse MLA attention).

This module is shared by the oracle-side tests, the GPU tests and the benchmark. It holds
workload shapes and random draws only: none of the method's arithmetic lives here.

Workloads (shapes follow the problem statement of DeepSeek Sparse Attention: an indexer with
H_I heads of dimension d_I, top-k selection, and MLA in MQA mode with H query heads over one
shared latent row of d_qk dims whose first d_v dims are the value):

  tiny      one causal sequence L=512; H_I=4, d_I=32, k=64; H=8, d_qk=80, d_v=64; all fp32.
  prefill8k one causal sequence L=8192; H_I=64, d_I=128 (FP8 e4m3), k=2048; H=128, 576/512 bf16.
  decode32k 64 sequences, one query each at position 32767 over 32768 cached entries.
  chunk128k 4096 query rows at positions 126976..131071 of one sequence of 131072 keys.
  ragged    128 single-query sequences with context lengths ~ U[4096, 131072] (seeded).
  short2k   one causal sequence L=2048 with k=2048 (every row selects all its candidates).

Value recipe: q^I, k^I, q and the latent rows are N(0,1); w is N(0,1)/sqrt(H_I). FP8 and bf16
tensors are produced by rounding the fp32 draws to nearest-even (torch's host cast). The
"int" variant replaces q^I, k^I by integers uniform in [-3, 3] and w by multiples of 1/8 in
[-1, 1], so that every indexer score is exactly representable in fp32. The "e4m3" variant
(FP8 indexer inputs only) draws q^I and k^I as uniformly random non-NaN e4m3fn codes, i.e.
values over the format's whole exponent range (subnormals to +-448), with w as for "normal".

Draws are counter-based: every tensor is generated in chunks of CHUNK leading-dim rows, chunk c
of tensor t of workload/variant/seed uses SeedSequence([seed, workload_id, variant_id, t, c]),
so any slice can be regenerated alone and chunks are drawn in parallel threads.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 4096

# tensor ids for the counter-based streams
T_QI, T_KI, T_W, T_Q, T_KV, T_LEN, T_QS, T_KS = 0, 1, 2, 3, 4, 5, 6, 7
VARIANTS = {"normal": 0, "int": 1, "e4m3": 2}


@dataclass
class Workload:
    name: str
    wid: int
    seqlens_q: list          # m_b per sequence
    seqlens_k: list          # n_b per sequence
    H_I: int
    d_I: int
    k: int
    H: int
    d_qk: int
    d_v: int
    idx_dtype: str           # "fp8" (OCP e4m3fn bytes) or "f32"
    attn_dtype: str          # "bf16" (bit patterns) or "f32"
    scale: float = field(default=0.0)

    def __post_init__(self):
        if not self.scale:
            self.scale = 1.0 / math.sqrt(self.d_qk)

    @property
    def num_seqs(self):
        return len(self.seqlens_q)

    @property
    def T(self):
        return int(sum(self.seqlens_q))

    @property
    def Nk(self):
        return int(sum(self.seqlens_k))

    @property
    def cu_seqlens_q(self):
        return np.concatenate([[0], np.cumsum(self.seqlens_q)]).astype(np.int32)

    @property
    def cu_seqlens_k(self):
        return np.concatenate([[0], np.cumsum(self.seqlens_k)]).astype(np.int32)

    @property
    def max_seqlen_q(self):
        return int(max(self.seqlens_q)) if self.seqlens_q else 0

    @property
    def max_seqlen_k(self):
        return int(max(self.seqlens_k)) if self.seqlens_k else 0

    def row_positions(self):
        """(seq, pos) of every global query row; query i of seq b sits at n_b - m_b + i."""
        seq, pos = [], []
        for b, (m, n) in enumerate(zip(self.seqlens_q, self.seqlens_k)):
            seq.extend([b] * m)
            pos.extend(range(n - m, n))
        return np.asarray(seq, np.int64), np.asarray(pos, np.int64)


def _ragged_lengths(seed, wid, batch, lo, hi):
    rng = np.random.default_rng(np.random.SeedSequence([seed, wid, 0, T_LEN, 0]))
    return rng.integers(lo, hi, endpoint=True, size=batch).astype(np.int64).tolist()


def workload(name: str, seed: int = 0) -> Workload:
    big = dict(H_I=64, d_I=128, k=2048, H=128, d_qk=576, d_v=512, idx_dtype="fp8", attn_dtype="bf16")
    if name == "tiny":
        return Workload(name, 0, [512], [512], H_I=4, d_I=32, k=64, H=8, d_qk=80, d_v=64,
                        idx_dtype="f32", attn_dtype="f32")
    if name == "prefill8k":
        return Workload(name, 1, [8192], [8192], **big)
    if name == "decode32k":
        return Workload(name, 2, [1] * 64, [32768] * 64, **big)
    if name == "chunk128k":
        return Workload(name, 3, [4096], [131072], **big)
    if name == "ragged":
        return Workload(name, 4, [1] * 128, _ragged_lengths(seed, 4, 128, 4096, 131072), **big)
    if name == "short2k":
        return Workload(name, 5, [2048], [2048], **big)
    raise KeyError(name)


WORKLOADS = ("tiny", "prefill8k", "decode32k", "chunk128k", "ragged", "short2k")


def custom(name="custom", seqlens_q=(64,), seqlens_k=(64,), H_I=4, d_I=32, k=16, H=8, d_qk=80,
           d_v=64, idx_dtype="f32", attn_dtype="f32", wid=99, scale=0.0) -> Workload:
    """A small workload of arbitrary shape (tests, edge cases)."""
    return Workload(name, wid, list(seqlens_q), list(seqlens_k), H_I, d_I, k, H, d_qk, d_v,
                    idx_dtype, attn_dtype, scale)


# ---------------------------------------------------------------- draws

def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw(seed, wid, variant, tid, rows, inner, kind, row_lo=0, row_hi=None):
    """Rows [row_lo, row_hi) of a [rows, inner] stream, drawn chunk by chunk."""
    row_hi = rows if row_hi is None else row_hi
    out = np.empty((row_hi - row_lo, inner), np.float32)
    c0, c1 = row_lo // CHUNK, (row_hi + CHUNK - 1) // CHUNK if row_hi > row_lo else row_lo // CHUNK

    def one(c):
        lo, hi = c * CHUNK, min(rows, (c + 1) * CHUNK)
        rng = np.random.default_rng(np.random.SeedSequence([seed, wid, variant, tid, c]))
        if kind == "normal":
            blk = rng.standard_normal((hi - lo, inner), dtype=np.float32)
        elif kind == "int3":
            blk = rng.integers(-3, 3, endpoint=True, size=(hi - lo, inner), dtype=np.int8).astype(np.float32)
        elif kind == "eighths":
            blk = rng.integers(-8, 8, endpoint=True, size=(hi - lo, inner), dtype=np.int8).astype(np.float32) / 8
        elif kind == "pow2":
            blk = np.exp2(rng.integers(-1, 1, endpoint=True, size=(hi - lo, inner))).astype(np.float32)
        elif kind == "logu":
            blk = np.exp2(rng.uniform(-2.0, 2.0, size=(hi - lo, inner))).astype(np.float32)
        elif kind == "e4m3code":   # uniform over the 254 non-NaN codes (0x7F and 0xFF skipped)
            c = rng.integers(0, 253, endpoint=True, size=(hi - lo, inner))
            blk = (c + (c >= 0x7F)).astype(np.float32)
        elif kind == "ternary":
            blk = rng.integers(-1, 1, endpoint=True, size=(hi - lo, inner), dtype=np.int8).astype(np.float32)
        else:
            raise ValueError(kind)
        a, b = max(lo, row_lo), min(hi, row_hi)
        out[a - row_lo:b - row_lo] = blk[a - lo:b - lo]

    chunks = list(range(c0, c1))
    if len(chunks) > 1:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, chunks))
    else:
        for c in chunks:
            one(c)
    return out


def to_fp8_e4m3fn_bytes(x: np.ndarray) -> np.ndarray:
    """Round fp32 to OCP FP8 e4m3fn (nearest-even), returned as uint8 codes."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (nearest-even), returned as uint16 bit patterns."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def gen_inputs(wl: Workload, variant: str = "normal", seed: int = 0, parts=("idx", "attn")) -> dict:
    """All inputs of the forward path for workload `wl`.

    Returns numpy arrays: qI [T,H_I,d_I], kI [Nk,d_I] (uint8 e4m3fn codes or float32),
    w [T,H_I] float32, q [T,H,d_qk], kv [Nk,d_qk] (uint16 bf16 bits or float32), plus
    cu_seqlens_q / cu_seqlens_k int32.
    """
    v = VARIANTS[variant]
    T, Nk = wl.T, wl.Nk
    out = dict(cu_seqlens_q=wl.cu_seqlens_q, cu_seqlens_k=wl.cu_seqlens_k)
    if "idx" in parts:
        if variant == "e4m3" and wl.idx_dtype != "fp8":
            raise ValueError("the e4m3 variant needs FP8 indexer inputs")
        qk_kind = {"int": "int3", "e4m3": "e4m3code"}.get(variant, "normal")
        qI = _draw(seed, wl.wid, v, T_QI, T, wl.H_I * wl.d_I, qk_kind).reshape(T, wl.H_I, wl.d_I)
        kI = _draw(seed, wl.wid, v, T_KI, Nk, wl.d_I, qk_kind)
        if variant == "int":
            w = _draw(seed, wl.wid, v, T_W, T, wl.H_I, "eighths")
        else:
            w = _draw(seed, wl.wid, v, T_W, T, wl.H_I, "normal") / np.float32(math.sqrt(wl.H_I))
        if variant == "e4m3":   # the draws are the codes themselves
            qI, kI = qI.astype(np.uint8), kI.astype(np.uint8)
        elif wl.idx_dtype == "fp8":
            qI, kI = to_fp8_e4m3fn_bytes(qI), to_fp8_e4m3fn_bytes(kI)
        out.update(qI=qI, kI=kI, w=np.ascontiguousarray(w, np.float32))
    if "attn" in parts:
        # the attention inputs are N(0,1) in both variants
        q = _draw(seed, wl.wid, 0, T_Q, T, wl.H * wl.d_qk, "normal").reshape(T, wl.H, wl.d_qk)
        kv = _draw(seed, wl.wid, 0, T_KV, Nk, wl.d_qk, "normal")
        if wl.attn_dtype == "bf16":
            q, kv = to_bf16_bits(q), to_bf16_bits(kv)
        out.update(q=q, kv=kv)
    return out


def gen_ternary(wl: Workload, seed: int = 0) -> dict:
    """Indexer queries and keys with entries in {-1, 0, 1} (FP8 codes for FP8 workloads, else
    float32), for cases whose head weights the caller constructs."""
    qI = _draw(seed, wl.wid, 3, T_QI, wl.T, wl.H_I * wl.d_I, "ternary").reshape(wl.T, wl.H_I, wl.d_I)
    kI = _draw(seed, wl.wid, 3, T_KI, wl.Nk, wl.d_I, "ternary")
    if wl.idx_dtype == "fp8":
        qI, kI = to_fp8_e4m3fn_bytes(qI), to_fp8_e4m3fn_bytes(kI)
    return dict(qI=qI, kI=kI)


# Head weights with 17 to 19 significant bits (c * 128 in [128, 256)): products with integers up to
# 32 stay exact in fp32, and rounding c * 128 to 4 significant bits, then 16 times the remainder,
# and so on, leaves a nonzero part at each of four steps.
SPLIT_WEIGHTS = (133.193359375 / 128, 246.2861328125 / 128, 136.63623046875 / 128)


def gen_linear_split(wl: Workload, seed: int = 0) -> dict:
    """Indexer inputs whose weighted query sum needs many significant bits, with every score
    exact in fp32: q^I, k^I in {-1, 0, 1}; row r weighs a single head j_r = r % H_I by
    +-SPLIT_WEIGHTS[r % 3] * 2^m (m cycling through -6, 0, 3, 9), all other heads 0; that head's
    query keeps at most 32 nonzero entries (so |q^I . k^I| <= 32)."""
    x = gen_ternary(wl, seed)
    qI = x["qI"].copy()
    zero = 0 if wl.idx_dtype != "fp8" else to_fp8_e4m3fn_bytes(np.zeros(1, np.float32))[0]
    w = np.zeros((wl.T, wl.H_I), np.float32)
    ms = (-6, 0, 3, 9)
    for r in range(wl.T):
        j = r % wl.H_I
        qI[r, j, 32:] = zero
        sign = -1.0 if (r // 3) % 2 else 1.0
        w[r, j] = np.float32(sign * SPLIT_WEIGHTS[r % 3] * 2.0 ** ms[(r // 2) % 4])
    return dict(qI=qI, kI=x["kI"], w=w)


def gen_scales(wl: Workload, variant: str = "normal", seed: int = 0) -> dict:
    """Positive scales of the indexer inputs: q_scale [T, H_I] and k_scale [Nk] float32.

    "int" variant: powers of two 1/2, 1, 2 (with the integer inputs every partial sum of a scaled
    score is a multiple of 1/16 below 2^18, exact in fp32);
    "normal": 2^U(-2, 2).
    """
    v = VARIANTS[variant]
    kind = "pow2" if variant == "int" else "logu"
    qs = _draw(seed, wl.wid, v, T_QS, wl.T, wl.H_I, kind)
    ks = _draw(seed, wl.wid, v, T_KS, wl.Nk, 1, kind).reshape(wl.Nk)
    return dict(q_scale=np.ascontiguousarray(qs), k_scale=np.ascontiguousarray(ks))
