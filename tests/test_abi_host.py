"""Host-only checks of the C ABI (no GPU needed): the library loads, exports every symbol that
include/dsa.h declares, and rejects invalid arguments with the documented status codes before
any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")
LIB = os.path.join(ROOT, "sparse_attention_head_amd", "libdsa.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libdsa.so not built")


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_head_amd as m
    return m


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", txt)))


def test_exports_every_declared_symbol(dsa):
    lib = ctypes.CDLL(LIB)
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"{n} declared in dsa.h but not exported"
    assert set(names) == set(dsa.EXPORTS)


def test_abi_version_and_status_strings(dsa):
    assert dsa.abi_version() == 4
    for st in range(8):
        s = dsa._c_status(st)
        assert s and len(s) >= 2
    assert dsa._c_status(99) == b"unknown status"


# ------------------------------------------------------------------ validation without a GPU

class FakeSeqs:
    """Host-side stand-in: device pointers are never dereferenced during validation."""

    def __init__(self, dsa, cu_q, cu_k, max_m=None, max_n=None):
        self.cu_q = np.asarray(cu_q, np.int32)
        self.cu_k = np.asarray(cu_k, np.int32)
        self.s = dsa._Seqs()
        self.s.num_seqs = len(cu_q) - 1
        self.s.cu_seqlens_q = self.cu_q.ctypes.data
        self.s.cu_seqlens_k = self.cu_k.ctypes.data
        self.s.cu_seqlens_q_host = self.cu_q.ctypes.data
        self.s.cu_seqlens_k_host = self.cu_k.ctypes.data
        m = np.diff(self.cu_q)
        n = np.diff(self.cu_k)
        self.s.max_seqlen_q = int(m.max()) if max_m is None else max_m
        self.s.max_seqlen_k = int(n.max()) if max_n is None else max_n

    @property
    def ref(self):
        return ctypes.byref(self.s)


def buf(nbytes, misalign=0):
    a = np.zeros(nbytes + 64, np.uint8)
    p = a.ctypes.data
    p += (-p) % 16 + misalign
    return a, p


def indexer(dsa, sq, H_I=64, d_I=128, dt=2, ptrs=None, ld=None, ws=None, ws_bytes=0):
    keep, p = buf(64)
    q, k, w, s = ptrs if ptrs else (p, p, p, p)
    ld = ld if ld is not None else (sq.s.max_seqlen_k + 3) // 4 * 4
    st = dsa._c_indexer(sq.ref, H_I, d_I, dt, q, k, w, s, ld, ws, ws_bytes, None)
    return st


def test_indexer_validation(dsa):
    sq = FakeSeqs(dsa, [0, 10], [0, 10])
    assert dsa._c_indexer(None, 64, 128, 2, 16, 16, 16, 16, 12, None, 0, None) == dsa.DSA_ERR_NULL
    assert indexer(dsa, sq, ld=8) == dsa.DSA_ERR_SHAPE                 # ld < max_seqlen_k
    assert indexer(dsa, sq, ld=14) == dsa.DSA_ERR_SHAPE                # ld not a multiple of 4
    assert indexer(dsa, sq, H_I=32) == dsa.DSA_ERR_UNSUPPORTED         # FP8 needs 64 x 128
    assert indexer(dsa, sq, dt=1) == dsa.DSA_ERR_DTYPE                 # bf16 indexer inputs
    assert indexer(dsa, sq, H_I=0) == dsa.DSA_ERR_SHAPE
    assert indexer(dsa, sq, dt=0, H_I=200) == dsa.DSA_ERR_UNSUPPORTED  # fp32 path limits
    keep, p = buf(64)
    _, pm = buf(64, misalign=4)
    assert indexer(dsa, sq, ptrs=(p, None, p, p)) == dsa.DSA_ERR_NULL
    assert indexer(dsa, sq, ptrs=(p, p, pm, p)) == dsa.DSA_ERR_ALIGN


def test_indexer_workspace(dsa):
    """The FP8 prefill path needs T * 516 bytes (rounded up) of workspace; decode and fp32 need
    none."""
    sq = FakeSeqs(dsa, [0, 10], [0, 10])
    need = dsa._c_indexer_ws(sq.ref, 64, 128, dsa.DSA_FP8_E4M3)
    assert need >= 10 * 516
    assert dsa._c_indexer_ws(sq.ref, 64, 128, dsa.DSA_F32) == 0
    assert dsa._c_indexer_ws(FakeSeqs(dsa, [0, 1, 2], [0, 5, 9]).ref, 64, 128, dsa.DSA_FP8_E4M3) == 0
    assert indexer(dsa, sq) == dsa.DSA_ERR_WORKSPACE
    keep, p = buf(need)
    assert indexer(dsa, sq, ws=p, ws_bytes=need - 1) == dsa.DSA_ERR_WORKSPACE
    _, pm = buf(need, misalign=4)
    assert indexer(dsa, sq, ws=pm, ws_bytes=need) == dsa.DSA_ERR_ALIGN


def test_seqs_validation(dsa):
    assert indexer(dsa, FakeSeqs(dsa, [0, 10], [0, 5])) == dsa.DSA_ERR_SHAPE             # m > n
    assert indexer(dsa, FakeSeqs(dsa, [0, 3, 2], [0, 5, 9])) == dsa.DSA_ERR_SHAPE        # decreasing
    assert indexer(dsa, FakeSeqs(dsa, [1, 3], [0, 5])) == dsa.DSA_ERR_SHAPE              # not from 0
    assert indexer(dsa, FakeSeqs(dsa, [0, 3], [0, 5], max_n=6)) == dsa.DSA_ERR_SHAPE     # wrong max
    neg = FakeSeqs(dsa, [0, 1], [0, 1])
    neg.s.num_seqs = -1
    assert indexer(dsa, neg) == dsa.DSA_ERR_SHAPE
    nulls = FakeSeqs(dsa, [0, 1], [0, 1])
    nulls.s.cu_seqlens_q_host = None
    assert indexer(dsa, nulls) == dsa.DSA_ERR_NULL
    empty = FakeSeqs(dsa, [0], [0], max_m=0, max_n=0)
    assert indexer(dsa, empty) == dsa.DSA_OK                            # B = 0: no-op


def test_indexer_grid_limits(dsa):
    """More sequences (FP8) or longer rows (fp32) than a launch grid dimension holds are refused
    before any launch (only rejected shapes are tried here: an accepted call would launch on the
    fake pointers)."""
    many = np.arange(65537, dtype=np.int32)   # 65536 decode sequences of one key
    assert indexer(dsa, FakeSeqs(dsa, many, many), ld=4) == dsa.DSA_ERR_UNSUPPORTED
    long_k = 65535 * 256 + 1
    assert indexer(dsa, FakeSeqs(dsa, [0, 1], [0, long_k]), dt=0, H_I=4, d_I=32,
                   ld=(long_k + 3) // 4 * 4) == dsa.DSA_ERR_UNSUPPORTED


def test_topk_and_attention_validation(dsa):
    sq = FakeSeqs(dsa, [0, 10], [0, 10])
    keep, p = buf(64)
    assert dsa._c_topk(sq.ref, p, 12, 0, p, None, 0, None) == dsa.DSA_ERR_UNSUPPORTED
    assert dsa._c_topk(sq.ref, p, 12, 20000, p, None, 0, None) == dsa.DSA_ERR_UNSUPPORTED
    assert dsa._c_topk(sq.ref, p, 8, 4, p, None, 0, None) == dsa.DSA_ERR_SHAPE
    assert dsa._c_topk(sq.ref, None, 12, 4, p, None, 0, None) == dsa.DSA_ERR_NULL
    # attention
    A = dsa._c_attn
    assert A(sq.ref, 128, 576, 512, 2, p, p, p, 64, 1.0, p, p, None, 0, None) == dsa.DSA_ERR_DTYPE
    assert A(sq.ref, 128, 576, 600, 1, p, p, p, 64, 1.0, p, p, None, 0, None) == dsa.DSA_ERR_SHAPE
    assert A(sq.ref, 64, 576, 512, 1, p, p, p, 64, 1.0, p, p, None, 0, None) == dsa.DSA_ERR_UNSUPPORTED
    assert A(sq.ref, 8, 80, 64, 0, p, p, p, 8000, 1.0, p, p, None, 0, None) == dsa.DSA_ERR_UNSUPPORTED
    assert A(sq.ref, 8, 80, 64, 0, p, None, p, 64, 1.0, p, p, None, 0, None) == dsa.DSA_ERR_NULL
    _, pm = buf(64, misalign=8)
    assert A(sq.ref, 8, 80, 64, 0, p, p, p, 64, 1.0, pm, p, None, 0, None) == dsa.DSA_ERR_ALIGN
    for bad_scale in (0.0, -0.5, float("inf"), float("nan")):
        assert A(sq.ref, 8, 80, 64, 0, p, p, p, 64, bad_scale, p, p, None, 0, None) == dsa.DSA_ERR_SHAPE


def test_forward_validation_and_workspace(dsa):
    sq = FakeSeqs(dsa, [0, 100], [0, 100])
    keep, p = buf(64)
    a = dsa._FwdArgs()
    a.H_I, a.d_I, a.qk_dtype = 64, 128, dsa.DSA_FP8_E4M3
    a.q_idx = a.k_idx = a.w = p
    a.k = 16
    a.H, a.d_qk, a.d_v, a.dtype = 128, 576, 512, dsa.DSA_BF16
    a.q = a.kv = a.out = a.lse = p
    a.softmax_scale = 0.04
    need = dsa._c_fwd_ws(sq.ref, ctypes.byref(a))
    # scores [100, 100] fp32 + indices [100, 16] int32, each 256-byte aligned
    assert need >= 100 * 100 * 4 + 100 * 16 * 4
    assert dsa._c_fwd(sq.ref, ctypes.byref(a), None, 0, None) == dsa.DSA_ERR_WORKSPACE
    assert dsa._c_fwd(sq.ref, ctypes.byref(a), p, need - 1, None) == dsa.DSA_ERR_WORKSPACE
    assert dsa._c_fwd(sq.ref, None, p, need, None) == dsa.DSA_ERR_NULL
    a.k = 0
    assert dsa._c_fwd(sq.ref, ctypes.byref(a), p, need, None) == dsa.DSA_ERR_UNSUPPORTED
    a.k = 16
    # caller-provided intermediates shrink the workspace
    a.scores_out, a.ld_scores_out, a.indices_out = p, 100, p
    assert dsa._c_fwd_ws(sq.ref, ctypes.byref(a)) < need
    a.ld_scores_out = 96
    assert dsa._c_fwd(sq.ref, ctypes.byref(a), p, need, None) == dsa.DSA_ERR_SHAPE


def test_forward_short_context_workspace(dsa):
    """With at most k keys per sequence the fused call needs neither scores nor indices: its
    workspace is the attention's alone, and grows by the indexer's when scores are requested."""
    sq = FakeSeqs(dsa, [0, 100], [0, 100])
    keep, p = buf(64)
    a = dsa._FwdArgs()
    a.H_I, a.d_I, a.qk_dtype = 64, 128, dsa.DSA_FP8_E4M3
    a.q_idx = a.k_idx = a.w = p
    a.k = 128
    a.H, a.d_qk, a.d_v, a.dtype = 128, 576, 512, dsa.DSA_BF16
    a.q = a.kv = a.out = a.lse = p
    a.softmax_scale = 0.04
    attn = dsa._c_attn_ws(sq.ref, 128, 576, 512, 128, dsa.DSA_BF16)
    assert dsa._c_fwd_ws(sq.ref, ctypes.byref(a)) == attn
    a.indices_out = p
    assert dsa._c_fwd_ws(sq.ref, ctypes.byref(a)) == attn
    a.scores_out, a.ld_scores_out = p, 100
    idx_ws = dsa._c_indexer_ws(sq.ref, 64, 128, dsa.DSA_FP8_E4M3)
    assert idx_ws > 0
    assert dsa._c_fwd_ws(sq.ref, ctypes.byref(a)) >= attn + idx_ws
    # one key more than k: the full path with its scores and indices
    a.k, a.scores_out, a.indices_out = 99, None, None
    assert dsa._c_fwd_ws(sq.ref, ctypes.byref(a)) >= 100 * 100 * 4 + 100 * 99 * 4


def test_alignment_validation(dsa):
    sq = FakeSeqs(dsa, [0, 10], [0, 20])
    keep, p = buf(64)
    A = dsa._c_align
    assert A(sq.ref, 128, 576, dsa.DSA_FP8_E4M3, p, p, p, 64, 0.04, p, p, 20, p, p, None) == dsa.DSA_ERR_DTYPE
    assert A(sq.ref, 8, 80, dsa.DSA_F32, p, p, p, 64, 0.04, p, p, 20, p, p, None) == dsa.DSA_ERR_UNSUPPORTED
    assert A(sq.ref, 128, 576, dsa.DSA_BF16, p, p, p, 0, 0.04, p, p, 20, p, p, None) == dsa.DSA_ERR_UNSUPPORTED
    assert A(sq.ref, 128, 576, dsa.DSA_BF16, p, p, p, 64, 0.04, p, p, 18, p, p, None) == dsa.DSA_ERR_SHAPE
    assert A(sq.ref, 128, 576, dsa.DSA_BF16, p, p, p, 64, -1.0, p, p, 20, p, p, None) == dsa.DSA_ERR_SHAPE
    assert A(sq.ref, 128, 576, dsa.DSA_BF16, p, p, p, 64, 0.04, None, p, 20, p, p, None) == dsa.DSA_ERR_NULL
    assert A(sq.ref, 128, 576, dsa.DSA_BF16, p, p, p, 64, 0.04, p, p, 20, p, None, None) == dsa.DSA_ERR_NULL
    _, pm = buf(64, misalign=4)
    assert A(sq.ref, 128, 576, dsa.DSA_BF16, p, p, p, 64, 0.04, p, p, 20, pm, p, None) == dsa.DSA_ERR_ALIGN


def test_last_error_is_descriptive(dsa):
    sq = FakeSeqs(dsa, [0, 10], [0, 5])
    indexer(dsa, sq)
    assert b"queries" in dsa._c_last()


# ------------------------------------------------------------------ Python binding argument checks
# The binding checks shapes, storage types, layouts and devices before any library call (the C
# layer sees pointers only). Each case below fails in the binding: CPU tensors never reach the
# library, the valid-shaped ones are stopped by the device check.

def _binding_case(dsa):
    import torch
    seqs = dsa.Seqs([0, 3, 5], [0, 10, 16], device="cpu")       # T = 5, Nk = 16, max_n = 10
    f8 = torch.float8_e4m3fn
    x = dict(
        qI=torch.zeros(5, 64, 128, dtype=f8), kI=torch.zeros(16, 128, dtype=f8),
        w=torch.zeros(5, 64), q=torch.zeros(5, 128, 576, dtype=torch.bfloat16),
        kv=torch.zeros(16, 576, dtype=torch.bfloat16), idx=torch.zeros(5, 64, dtype=torch.int32),
        scores=torch.zeros(5, 12), lse=torch.zeros(5, 128))
    return seqs, x


def test_binding_rejects_bad_indexer_arguments(dsa):
    import torch
    seqs, x = _binding_case(dsa)
    bad = [
        (dict(qI=torch.zeros(4, 64, 128, dtype=torch.float8_e4m3fn)), ValueError, "q_idx"),   # rows != T
        (dict(kI=torch.zeros(15, 128, dtype=torch.float8_e4m3fn)), ValueError, "k_idx"),      # keys != Nk
        (dict(kI=torch.zeros(16, 128)), TypeError, "k_idx"),                                  # fp32 keys, FP8 queries
        (dict(w=torch.zeros(5, 64, dtype=torch.float64)), TypeError, "w"),
        (dict(w=torch.zeros(5, 32)), ValueError, "w"),
        (dict(qI=torch.zeros(5, 64, 256, dtype=torch.float8_e4m3fn)[:, :, :128]), ValueError, "contiguous"),
        (dict(qI=torch.zeros(5, 64, 128, dtype=torch.int16)), TypeError, "q_idx"),
        (dict(scores=torch.zeros(5, 8)), ValueError, "scores"),                             # < max_n columns
        (dict(scores=torch.zeros(5, 12, dtype=torch.float16)), TypeError, "scores"),
        (dict(scores=torch.zeros(12, 5).t()), ValueError, "scores"),                         # column stride 5
    ]
    for change, exc, what in bad:
        y = dict(x, **change)
        with pytest.raises(exc, match=what):
            dsa.indexer_scores(seqs, y["qI"], y["kI"], y["w"], scores=y["scores"])
    with pytest.raises(ValueError, match="GPU"):
        dsa.indexer_scores(seqs, x["qI"], x["kI"], x["w"], scores=x["scores"])
    with pytest.raises(ValueError, match="q_scale"):
        dsa.indexer_scores_scaled(seqs, x["qI"], torch.ones(5, 32), x["kI"], None, x["w"])
    with pytest.raises(ValueError, match="k_scale"):
        dsa.indexer_scores_scaled(seqs, x["qI"], None, x["kI"], torch.ones(10), x["w"])


def test_binding_rejects_bad_topk_and_attention_arguments(dsa):
    import torch
    seqs, x = _binding_case(dsa)
    with pytest.raises(TypeError, match="indices"):
        dsa.topk(seqs, x["scores"], 64, indices=torch.zeros(5, 64, dtype=torch.int64))
    with pytest.raises(ValueError, match="indices"):
        dsa.topk(seqs, x["scores"], 64, indices=torch.zeros(5, 32, dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU"):
        dsa.topk(seqs, x["scores"], 64)
    bad = [
        (dict(kv=torch.zeros(16, 576)), TypeError, "kv"),                                   # fp32 kv, bf16 q
        (dict(kv=torch.zeros(12, 576, dtype=torch.bfloat16)), ValueError, "kv"),            # rows != Nk
        (dict(q=torch.zeros(6, 128, 576, dtype=torch.bfloat16)), ValueError, "q"),
        (dict(idx=torch.zeros(5, 64, dtype=torch.int64)), TypeError, "indices"),
        (dict(idx=torch.zeros(64, 5, dtype=torch.int32).t()), ValueError, "indices"),        # not contiguous
        (dict(lse=torch.zeros(5, 64)), ValueError, "lse"),
    ]
    for change, exc, what in bad:
        y = dict(x, **change)
        with pytest.raises(exc, match=what):
            dsa.sparse_mla_attn(seqs, y["q"], y["kv"], y["idx"], 0.04, lse=y["lse"])
    with pytest.raises(ValueError, match="out"):
        dsa.sparse_mla_attn(seqs, x["q"], x["kv"], x["idx"], 0.04, out=torch.zeros(5, 128, 576, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU"):
        dsa.sparse_mla_attn(seqs, x["q"], x["kv"], x["idx"], 0.04)
    with pytest.raises(ValueError, match="scores"):
        dsa.indexer_alignment(seqs, x["q"], x["kv"], x["idx"], 0.04, x["lse"], torch.zeros(4, 12))
    with pytest.raises(ValueError, match="GPU"):
        dsa.indexer_alignment(seqs, x["q"], x["kv"], x["idx"], 0.04, x["lse"], x["scores"])


def test_binding_rejects_bad_forward_arguments(dsa):
    import torch
    seqs, x = _binding_case(dsa)
    with pytest.raises(ValueError, match="kv"):
        dsa.Forward(seqs, x["qI"], x["kI"], x["w"], x["q"], x["kv"][:8], 64, 0.04)
    with pytest.raises(TypeError, match="w"):
        dsa.Forward(seqs, x["qI"], x["kI"], x["w"].double(), x["q"], x["kv"], 64, 0.04)
    with pytest.raises(ValueError, match="k_idx_scale"):
        dsa.Forward(seqs, x["qI"], x["kI"], x["w"], x["q"], x["kv"], 64, 0.04, k_idx_scale=torch.ones(5))
    with pytest.raises(ValueError, match="GPU"):
        dsa.Forward(seqs, x["qI"], x["kI"], x["w"], x["q"], x["kv"], 64, 0.04)


def test_noalloc_forward_rejects_oversized_batches_without_a_device(dsa):
    """dsa_forward_noalloc checks the batch's workspace against its static scratch before touching
    a device: a 5000-row prefill (scores 100 MB and indices 41 MB, more than the scratch) is rejected
    with DSA_ERR_WORKSPACE, and B = 0 is a no-op."""
    sq = FakeSeqs(dsa, [0, 5000], [0, 5000])
    keep, p = buf(64)
    a = dsa._FwdArgs()
    a.H_I, a.d_I, a.qk_dtype = 64, 128, dsa.DSA_FP8_E4M3
    a.q_idx = a.k_idx = a.w = p
    a.k = 2048
    a.H, a.d_qk, a.d_v, a.dtype = 128, 576, 512, dsa.DSA_BF16
    a.q = a.kv = a.out = a.lse = p
    a.softmax_scale = 0.04
    assert dsa._c_fwd_ws(sq.ref, ctypes.byref(a)) > dsa.NOALLOC_SCRATCH_BYTES
    assert dsa._c_fwd_na(sq.ref, ctypes.byref(a), None) == dsa.DSA_ERR_WORKSPACE
    assert b"scratch" in dsa._c_last()
    assert dsa._c_fwd_na(sq.ref, None, None) == dsa.DSA_ERR_NULL
    empty = FakeSeqs(dsa, [0], [0], max_m=0, max_n=0)
    assert dsa._c_fwd_na(empty.ref, ctypes.byref(a), None) == dsa.DSA_OK


def test_noalloc_forward_checks_arguments_before_sizing(dsa):
    """Arguments are validated before the workspace is planned: on an oversized batch a bad k or
    softmax scale is reported as such (not as a workspace shortfall) by both fused entry points,
    still without touching a device."""
    sq = FakeSeqs(dsa, [0, 5000], [0, 5000])
    keep, p = buf(64)
    a = dsa._FwdArgs()
    a.H_I, a.d_I, a.qk_dtype = 64, 128, dsa.DSA_FP8_E4M3
    a.q_idx = a.k_idx = a.w = p
    a.H, a.d_qk, a.d_v, a.dtype = 128, 576, 512, dsa.DSA_BF16
    a.q = a.kv = a.out = a.lse = p
    a.softmax_scale = 0.04
    for bad_k in (0, -5, 16385):
        a.k = bad_k
        assert dsa._c_fwd_na(sq.ref, ctypes.byref(a), None) == dsa.DSA_ERR_UNSUPPORTED
        assert b"k = " in dsa._c_last()
        assert dsa._c_fwd(sq.ref, ctypes.byref(a), None, 0, None) == dsa.DSA_ERR_UNSUPPORTED
    a.k = 2048
    a.softmax_scale = 0.0
    assert dsa._c_fwd_na(sq.ref, ctypes.byref(a), None) == dsa.DSA_ERR_SHAPE
    assert b"softmax_scale" in dsa._c_last()
    a.softmax_scale = 0.04
    a.H_I = -64
    assert dsa._c_fwd_na(sq.ref, ctypes.byref(a), None) == dsa.DSA_ERR_SHAPE
    a.H_I = 64
    assert dsa._c_fwd_na(sq.ref, ctypes.byref(a), None) == dsa.DSA_ERR_WORKSPACE
