"""Python binding of libdsa.so, the MI355X (gfx950) DeepSeek Sparse Attention forward path.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI of
include/dsa.h. Tensors are torch tensors on the GPU (PyTorch provides device memory and the
current stream); sequence descriptions are cumulative row counts.

    import sparse_attention_head_amd as dsa
    seqs = dsa.Seqs(cu_seqlens_q, cu_seqlens_k)          # int32 lists / arrays
    scores = dsa.indexer_scores(seqs, q_idx, k_idx, w)    # [T, ld] fp32
    idx = dsa.topk(seqs, scores, k)                       # [T, k] int32
    out, lse = dsa.sparse_mla_attn(seqs, q, kv, idx, scale)
    out, lse = dsa.forward(seqs, q_idx, k_idx, w, q, kv, k, scale)

FP8 tensors are passed as torch.float8_e4m3fn (or uint8 codes), bf16 as torch.bfloat16.
If the library has not been built, importing this package raises ImportError: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing; build it with `python sparse_attention_head_amd/build.py`")

_lib = ctypes.CDLL(_LIB_PATH)

# ---------------------------------------------------------------- C types

DSA_OK, DSA_ERR_NULL, DSA_ERR_SHAPE, DSA_ERR_DTYPE, DSA_ERR_ALIGN, DSA_ERR_WORKSPACE, \
    DSA_ERR_UNSUPPORTED, DSA_ERR_HIP = range(8)
DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2

_i32p = ctypes.POINTER(ctypes.c_int32)
_vp = ctypes.c_void_p


class _Seqs(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32),
                ("cu_seqlens_q", _vp), ("cu_seqlens_k", _vp),
                ("cu_seqlens_q_host", _vp), ("cu_seqlens_k_host", _vp),
                ("max_seqlen_q", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32)]


class _FwdArgs(ctypes.Structure):
    _fields_ = [("H_I", ctypes.c_int32), ("d_I", ctypes.c_int32), ("qk_dtype", ctypes.c_int),
                ("q_idx", _vp), ("k_idx", _vp), ("w", _vp),
                ("k", ctypes.c_int32),
                ("H", ctypes.c_int32), ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("dtype", ctypes.c_int), ("q", _vp), ("kv", _vp), ("softmax_scale", ctypes.c_float),
                ("out", _vp), ("lse", _vp),
                ("scores_out", _vp), ("ld_scores_out", ctypes.c_int64), ("indices_out", _vp),
                ("q_idx_scale", _vp), ("k_idx_scale", _vp)]


def _proto(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_c_indexer_ws = _proto("dsa_indexer_workspace_size", ctypes.c_size_t,
                       [ctypes.POINTER(_Seqs), ctypes.c_int32, ctypes.c_int32, ctypes.c_int])
_c_indexer = _proto("dsa_indexer_scores", ctypes.c_int,
                    [ctypes.POINTER(_Seqs), ctypes.c_int32, ctypes.c_int32, ctypes.c_int, _vp, _vp, _vp,
                     _vp, ctypes.c_int64, _vp, ctypes.c_size_t, _vp])
_c_indexer_sws = _proto("dsa_indexer_scaled_workspace_size", ctypes.c_size_t,
                        [ctypes.POINTER(_Seqs), ctypes.c_int32, ctypes.c_int32, ctypes.c_int])
_c_indexer_s = _proto("dsa_indexer_scores_scaled", ctypes.c_int,
                      [ctypes.POINTER(_Seqs), ctypes.c_int32, ctypes.c_int32, ctypes.c_int, _vp, _vp, _vp, _vp,
                       _vp, _vp, ctypes.c_int64, _vp, ctypes.c_size_t, _vp])
_c_topk_ws = _proto("dsa_topk_workspace_size", ctypes.c_size_t, [ctypes.POINTER(_Seqs), ctypes.c_int32])
_c_topk = _proto("dsa_topk", ctypes.c_int,
                 [ctypes.POINTER(_Seqs), _vp, ctypes.c_int64, ctypes.c_int32, _vp, _vp, ctypes.c_size_t, _vp])
_c_itk_ws = _proto("dsa_indexer_topk_workspace_size", ctypes.c_size_t,
                   [ctypes.POINTER(_Seqs), ctypes.c_int32, ctypes.c_int32, ctypes.c_int, ctypes.c_int32])
_c_itk = _proto("dsa_indexer_topk", ctypes.c_int,
                [ctypes.POINTER(_Seqs), ctypes.c_int32, ctypes.c_int32, ctypes.c_int, _vp, _vp, _vp, _vp,
                 ctypes.c_int64, ctypes.c_int32, _vp, _vp, ctypes.c_size_t, _vp])
_c_attn_ws = _proto("dsa_sparse_mla_attn_workspace_size", ctypes.c_size_t,
                    [ctypes.POINTER(_Seqs), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                     ctypes.c_int])
_c_attn = _proto("dsa_sparse_mla_attn", ctypes.c_int,
                 [ctypes.POINTER(_Seqs), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int, _vp, _vp,
                  _vp, ctypes.c_int32, ctypes.c_float, _vp, _vp, _vp, ctypes.c_size_t, _vp])
_c_fwd_ws = _proto("dsa_forward_workspace_size", ctypes.c_size_t, [ctypes.POINTER(_Seqs), ctypes.POINTER(_FwdArgs)])
_c_fwd = _proto("dsa_forward", ctypes.c_int,
                [ctypes.POINTER(_Seqs), ctypes.POINTER(_FwdArgs), _vp, ctypes.c_size_t, _vp])
_c_fwd_na = _proto("dsa_forward_noalloc", ctypes.c_int, [ctypes.POINTER(_Seqs), ctypes.POINTER(_FwdArgs), _vp])
_c_align = _proto("dsa_indexer_alignment", ctypes.c_int,
                  [ctypes.POINTER(_Seqs), ctypes.c_int32, ctypes.c_int32, ctypes.c_int, _vp, _vp, _vp,
                   ctypes.c_int32, ctypes.c_float, _vp, _vp, ctypes.c_int64, _vp, _vp, _vp])
_c_status = _proto("dsa_status_string", ctypes.c_char_p, [ctypes.c_int])
_c_last = _proto("dsa_last_error", ctypes.c_char_p, [])
_c_abi = _proto("dsa_abi_version", ctypes.c_int32, [])

EXPORTS = ("dsa_indexer_workspace_size", "dsa_indexer_scores", "dsa_indexer_scaled_workspace_size",
           "dsa_indexer_scores_scaled", "dsa_topk_workspace_size", "dsa_topk", "dsa_indexer_topk_workspace_size",
           "dsa_indexer_topk", "dsa_sparse_mla_attn_workspace_size",
           "dsa_sparse_mla_attn", "dsa_forward_workspace_size", "dsa_forward", "dsa_forward_noalloc",
           "dsa_indexer_alignment",
           "dsa_status_string",
           "dsa_last_error", "dsa_abi_version")


class DSAError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {_c_status(status).decode()} ({_c_last().decode()})")


def _check(st, call):
    if st != DSA_OK:
        raise DSAError(st, call)


def abi_version() -> int:
    return int(_c_abi())


def library_path() -> str:
    return _LIB_PATH


# ---------------------------------------------------------------- marshalling helpers

def _torch():
    import torch
    return torch


class Seqs:
    """A ragged batch: cu_seqlens_q / cu_seqlens_k (length B+1, starting at 0).

    Keeps host copies (read by the library for validation and planning) and device copies
    (read by the kernels). `device` defaults to the current CUDA device.
    """

    def __init__(self, cu_seqlens_q, cu_seqlens_k, device=None):
        torch = _torch()
        self.cu_q_host = np.ascontiguousarray(np.asarray(cu_seqlens_q, dtype=np.int32))
        self.cu_k_host = np.ascontiguousarray(np.asarray(cu_seqlens_k, dtype=np.int32))
        self.B = len(self.cu_q_host) - 1
        dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.cu_q = torch.from_numpy(self.cu_q_host).to(dev)
        self.cu_k = torch.from_numpy(self.cu_k_host).to(dev)
        m = np.diff(self.cu_q_host) if self.B > 0 else np.zeros(0, np.int32)
        n = np.diff(self.cu_k_host) if self.B > 0 else np.zeros(0, np.int32)
        self.max_m = int(m.max()) if self.B > 0 else 0
        self.max_n = int(n.max()) if self.B > 0 else 0
        self.T = int(self.cu_q_host[-1]) if self.B >= 0 and len(self.cu_q_host) else 0
        self.Nk = int(self.cu_k_host[-1]) if len(self.cu_k_host) else 0

    def c(self) -> _Seqs:
        s = _Seqs()
        s.num_seqs = self.B
        s.cu_seqlens_q = self.cu_q.data_ptr() if self.B > 0 else None
        s.cu_seqlens_k = self.cu_k.data_ptr() if self.B > 0 else None
        s.cu_seqlens_q_host = self.cu_q_host.ctypes.data
        s.cu_seqlens_k_host = self.cu_k_host.ctypes.data
        s.max_seqlen_q = self.max_m
        s.max_seqlen_k = self.max_n
        return s


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return DSA_FP8_E4M3
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def scores_ld(max_seqlen_k: int) -> int:
    return max(4, (max_seqlen_k + 3) // 4 * 4)


# ---------------------------------------------------------------- argument checks
# The C layer sees pointers only, so shapes, storage types, layouts and devices are checked here,
# before any library call: a wrong one would make the kernels read or write outside the buffers.

def _dtypes(kind):
    torch = _torch()
    return {"fp8": (torch.float8_e4m3fn, torch.uint8), "f32": (torch.float32,), "bf16": (torch.bfloat16,),
            "i32": (torch.int32,), "u8": (torch.uint8,)}[kind]


def _need(name, t, kinds, shape):
    """t must be a tensor of one of the storage kinds, of the given shape (None: any extent),
    and contiguous."""
    torch = _torch()
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    allowed = tuple(d for k in kinds for d in _dtypes(k))
    if t.dtype not in allowed:
        raise TypeError(f"{name} must have dtype {' or '.join(str(d) for d in allowed)}, got {t.dtype}")
    if t.dim() != len(shape) or any(w is not None and g != w for g, w in zip(t.shape, shape)):
        want = ", ".join("*" if w is None else str(w) for w in shape)
        raise ValueError(f"{name} must have shape [{want}], got {list(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_scores(name, t, seqs):
    """Score rows: fp32 [T, >= max_seqlen_k] with unit column stride; the row stride is the
    leading dimension passed to the library."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must have dtype torch.float32, got {t.dtype}")
    if t.dim() != 2 or t.shape[0] != seqs.T or t.shape[1] < seqs.max_n:
        raise ValueError(f"{name} must have shape [{seqs.T}, >= {seqs.max_n}], got {list(t.shape)}")
    if t.stride(1) != 1 or t.stride(0) < t.shape[1]:
        raise ValueError(f"{name} rows must be dense (column stride 1), got strides {t.stride()}")


def _need_ws(name, t):
    if t is not None:
        _need(name, t, ("u8",), (None,))


def _same_device(seqs, *named):
    """Every tensor on the GPU that holds the sequence description."""
    dev = seqs.cu_q.device
    if dev.type != "cuda":
        raise ValueError(f"the sequence description must be on a GPU device, it is on {dev}")
    for name, t in named:
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the sequence description on {dev}")


def _check_indexer_args(seqs, q_idx, k_idx, w):
    _need("q_idx", q_idx, ("fp8", "f32"), (seqs.T, None, None))
    H_I, d_I = int(q_idx.shape[1]), int(q_idx.shape[2])
    kind = "f32" if q_idx.dtype == _torch().float32 else "fp8"
    _need("k_idx", k_idx, (kind,), (seqs.Nk, d_I))
    _need("w", w, ("f32",), (seqs.T, H_I))
    return H_I, d_I


def _check_attn_args(seqs, q, kv, indices, d_v, out, lse):
    _need("q", q, ("bf16", "f32"), (seqs.T, None, None))
    T, H, d_qk = (int(x) for x in q.shape)
    kind = "bf16" if q.dtype == _torch().bfloat16 else "f32"
    _need("kv", kv, (kind,), (seqs.Nk, d_qk))
    if indices is not None:
        _need("indices", indices, ("i32",), (T, None))
    if out is not None:
        _need("out", out, (kind,), (T, H, d_v))
    if lse is not None:
        _need("lse", lse, ("f32",), (T, H))
    return T, H, d_qk


# ---------------------------------------------------------------- the four calls

def indexer_workspace_size(seqs: Seqs, H_I: int, d_I: int, qk_dtype: int) -> int:
    cs = seqs.c()
    return int(_c_indexer_ws(ctypes.byref(cs), H_I, d_I, qk_dtype))


def indexer_scores(seqs: Seqs, q_idx, k_idx, w, scores=None, ws=None, stream=None):
    """I[r, s] for s <= pos(r); returns scores [T, ld] fp32 (entries beyond pos unspecified).
    q_idx [T, H_I, d_I] and k_idx [Nk, d_I] both FP8 (float8_e4m3fn / uint8 codes) or both
    fp32, w [T, H_I] fp32. `ws` (uint8 device tensor of indexer_workspace_size bytes) is
    allocated when not given."""
    torch = _torch()
    H_I, d_I = _check_indexer_args(seqs, q_idx, k_idx, w)
    if scores is not None:
        _need_scores("scores", scores, seqs)
    _need_ws("ws", ws)
    _same_device(seqs, ("q_idx", q_idx), ("k_idx", k_idx), ("w", w), ("scores", scores), ("ws", ws))
    if scores is None:
        scores = torch.empty((seqs.T, scores_ld(seqs.max_n)), dtype=torch.float32, device=q_idx.device)
    cs = seqs.c()
    dt = _dtype_code(q_idx)
    wsz = int(_c_indexer_ws(ctypes.byref(cs), H_I, d_I, dt))
    if ws is None and wsz:
        ws = torch.empty(wsz, dtype=torch.uint8, device=q_idx.device)
    elif ws is not None:
        wsz = ws.numel()
    _check(_c_indexer(ctypes.byref(cs), H_I, d_I, dt, _ptr(q_idx), _ptr(k_idx), _ptr(w),
                      _ptr(scores), int(scores.stride(0)), _ptr(ws), wsz, _stream(stream)),
           "dsa_indexer_scores")
    return scores


def indexer_scaled_workspace_size(seqs: Seqs, H_I: int, d_I: int, qk_dtype: int) -> int:
    cs = seqs.c()
    return int(_c_indexer_sws(ctypes.byref(cs), H_I, d_I, qk_dtype))


def indexer_scores_scaled(seqs: Seqs, q_idx, q_scale, k_idx, k_scale, w, scores=None, ws=None,
                          stream=None):
    """Scores of scaled inputs: q_scale [T, H_I] and k_scale [Nk] fp32 (positive) or None."""
    torch = _torch()
    H_I, d_I = _check_indexer_args(seqs, q_idx, k_idx, w)
    if q_scale is not None:
        _need("q_scale", q_scale, ("f32",), (seqs.T, H_I))
    if k_scale is not None:
        _need("k_scale", k_scale, ("f32",), (seqs.Nk,))
    if scores is not None:
        _need_scores("scores", scores, seqs)
    _need_ws("ws", ws)
    _same_device(seqs, ("q_idx", q_idx), ("k_idx", k_idx), ("w", w), ("q_scale", q_scale),
                 ("k_scale", k_scale), ("scores", scores), ("ws", ws))
    if scores is None:
        scores = torch.empty((seqs.T, scores_ld(seqs.max_n)), dtype=torch.float32, device=q_idx.device)
    cs = seqs.c()
    dt = _dtype_code(q_idx)
    wsz = int(_c_indexer_sws(ctypes.byref(cs), H_I, d_I, dt))
    if ws is None:
        ws = torch.empty(max(wsz, 1), dtype=torch.uint8, device=q_idx.device)
    else:
        wsz = ws.numel()
    _check(_c_indexer_s(ctypes.byref(cs), H_I, d_I, dt, _ptr(q_idx), _ptr(q_scale), _ptr(k_idx),
                        _ptr(k_scale), _ptr(w), _ptr(scores), int(scores.stride(0)), _ptr(ws), wsz,
                        _stream(stream)),
           "dsa_indexer_scores_scaled")
    return scores


def topk(seqs: Seqs, scores, k: int, indices=None, stream=None):
    """Top-k positions per row: ascending, ties to the lower position, -1 padded."""
    torch = _torch()
    _need_scores("scores", scores, seqs)
    if indices is not None:
        _need("indices", indices, ("i32",), (seqs.T, k))
    _same_device(seqs, ("scores", scores), ("indices", indices))
    if indices is None:
        indices = torch.empty((seqs.T, k), dtype=torch.int32, device=scores.device)
    cs = seqs.c()
    wsz = int(_c_topk_ws(ctypes.byref(cs), k))
    ws = torch.empty(max(wsz, 1), dtype=torch.uint8, device=scores.device) if wsz else None
    _check(_c_topk(ctypes.byref(cs), _ptr(scores), int(scores.stride(0)), k, _ptr(indices), _ptr(ws), wsz,
                   _stream(stream)), "dsa_topk")
    return indices


def indexer_topk_workspace_size(seqs: Seqs, H_I: int, d_I: int, qk_dtype: int, k: int) -> int:
    cs = seqs.c()
    return int(_c_itk_ws(ctypes.byref(cs), H_I, d_I, qk_dtype, k))


def indexer_topk(seqs: Seqs, q_idx, k_idx, w, k: int, scores=None, indices=None, ws=None, stream=None):
    """Indexer scores and top-k in one call (the selection fused into the indexer for decode
    batches); returns (scores [T, ld] fp32, indices [T, k] int32), identical to indexer_scores
    followed by topk."""
    torch = _torch()
    H_I, d_I = _check_indexer_args(seqs, q_idx, k_idx, w)
    if scores is not None:
        _need_scores("scores", scores, seqs)
    if indices is not None:
        _need("indices", indices, ("i32",), (seqs.T, k))
    _need_ws("ws", ws)
    _same_device(seqs, ("q_idx", q_idx), ("k_idx", k_idx), ("w", w), ("scores", scores), ("indices", indices),
                 ("ws", ws))
    dev = q_idx.device
    if scores is None:
        scores = torch.empty((seqs.T, scores_ld(seqs.max_n)), dtype=torch.float32, device=dev)
    if indices is None:
        indices = torch.empty((seqs.T, k), dtype=torch.int32, device=dev)
    cs = seqs.c()
    dt = _dtype_code(q_idx)
    wsz = int(_c_itk_ws(ctypes.byref(cs), H_I, d_I, dt, k))
    if ws is None:
        ws = torch.empty(max(wsz, 1), dtype=torch.uint8, device=dev)
    else:
        wsz = int(ws.numel())
    _check(_c_itk(ctypes.byref(cs), H_I, d_I, dt, _ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(scores),
                  int(scores.stride(0)), k, _ptr(indices), _ptr(ws), wsz, _stream(stream)), "dsa_indexer_topk")
    return scores, indices


def attn_workspace_size(seqs: Seqs, H: int, d_qk: int, d_v: int, k: int, dtype: int) -> int:
    cs = seqs.c()
    return int(_c_attn_ws(ctypes.byref(cs), H, d_qk, d_v, k, dtype))


def sparse_mla_attn(seqs: Seqs, q, kv, indices, scale: float, d_v: int = None, out=None, lse=None,
                    with_lse=True, ws=None, stream=None):
    """Attention of every head over the selected latent rows; returns (out, lse).
    q [T, H, d_qk] and kv [Nk, d_qk] both bf16 or both fp32, indices [T, k] int32.
    `ws` (uint8 device tensor of attn_workspace_size bytes) is allocated when not given."""
    torch = _torch()
    _need("q", q, ("bf16", "f32"), (seqs.T, None, None))
    if d_v is None:
        d_v = 512 if int(q.shape[2]) == 576 else int(q.shape[2])
    T, H, d_qk = _check_attn_args(seqs, q, kv, indices, d_v, out, lse)
    _need_ws("ws", ws)
    _same_device(seqs, ("q", q), ("kv", kv), ("indices", indices), ("out", out), ("lse", lse), ("ws", ws))
    k = int(indices.shape[1])
    if out is None:
        out = torch.empty((T, H, d_v), dtype=q.dtype, device=q.device)
    if lse is None and with_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    cs = seqs.c()
    dt = _dtype_code(q)
    wsz = int(_c_attn_ws(ctypes.byref(cs), H, d_qk, d_v, k, dt))
    if ws is None:
        ws = torch.empty(max(wsz, 1), dtype=torch.uint8, device=q.device) if wsz else None
    elif wsz:
        wsz = int(ws.numel())
    _check(_c_attn(ctypes.byref(cs), H, d_qk, d_v, dt, _ptr(q), _ptr(kv), _ptr(indices), k, float(scale),
                   _ptr(out), _ptr(lse), _ptr(ws), wsz, _stream(stream)), "dsa_sparse_mla_attn")
    return out, lse


def indexer_alignment(seqs: Seqs, q, kv, indices, scale: float, lse, scores, with_target=True,
                      kl=None, target=None, stream=None):
    """Indexer-alignment target (head-averaged attention distribution over each row's index list)
    and its KL divergence from the softmax of the indexer scores; returns (target or None, kl)."""
    torch = _torch()
    _need("q", q, ("bf16", "f32"), (seqs.T, None, None))
    T, H, d_qk = _check_attn_args(seqs, q, kv, indices, None, None, lse)
    _need("lse", lse, ("f32",), (T, H))
    _need_scores("scores", scores, seqs)
    k = int(indices.shape[1])
    if kl is not None:
        _need("kl", kl, ("f32",), (T,))
    if target is not None:
        _need("target", target, ("f32",), (T, k))
    _same_device(seqs, ("q", q), ("kv", kv), ("indices", indices), ("lse", lse), ("scores", scores),
                 ("kl", kl), ("target", target))
    if kl is None:
        kl = torch.empty((T,), dtype=torch.float32, device=q.device)
    if target is None and with_target:
        target = torch.empty((T, k), dtype=torch.float32, device=q.device)
    cs = seqs.c()
    _check(_c_align(ctypes.byref(cs), H, d_qk, _dtype_code(q), _ptr(q), _ptr(kv), _ptr(indices), k,
                    float(scale), _ptr(lse), _ptr(scores), int(scores.stride(0)), _ptr(target), _ptr(kl),
                    _stream(stream)), "dsa_indexer_alignment")
    return target, kl


NOALLOC_SCRATCH_BYTES = 128 << 20


class Forward:
    """Fused indexer -> top-k -> attention with a reusable workspace (one allocation per shape).

    With noalloc=True the calls go to dsa_forward_noalloc, whose workspace is the library's
    static device scratch (no workspace is allocated here; outputs still are, once, at
    construction)."""

    def __init__(self, seqs: Seqs, q_idx, k_idx, w, q, kv, k: int, scale: float, d_v: int = None,
                 keep_scores=False, keep_indices=False, with_lse=True, q_idx_scale=None, k_idx_scale=None,
                 noalloc=False):
        torch = _torch()
        self.seqs = seqs
        H_I, d_I = _check_indexer_args(seqs, q_idx, k_idx, w)
        _need("q", q, ("bf16", "f32"), (seqs.T, None, None))
        T, H, d_qk = (int(x) for x in q.shape)
        d_v = d_v if d_v is not None else (512 if d_qk == 576 else d_qk)
        _check_attn_args(seqs, q, kv, None, d_v, None, None)
        if q_idx_scale is not None:
            _need("q_idx_scale", q_idx_scale, ("f32",), (seqs.T, H_I))
        if k_idx_scale is not None:
            _need("k_idx_scale", k_idx_scale, ("f32",), (seqs.Nk,))
        _same_device(seqs, ("q_idx", q_idx), ("k_idx", k_idx), ("w", w), ("q", q), ("kv", kv),
                     ("q_idx_scale", q_idx_scale), ("k_idx_scale", k_idx_scale))
        dev = q.device
        self.out = torch.empty((T, H, d_v), dtype=q.dtype, device=dev)
        self.lse = torch.empty((T, H), dtype=torch.float32, device=dev) if with_lse else None
        self.scores = (torch.empty((T, scores_ld(seqs.max_n)), dtype=torch.float32, device=dev)
                       if keep_scores else None)
        self.indices = torch.empty((T, k), dtype=torch.int32, device=dev) if keep_indices else None
        a = _FwdArgs()
        a.H_I, a.d_I = H_I, d_I
        a.qk_dtype = _dtype_code(q_idx)
        a.q_idx, a.k_idx, a.w = _ptr(q_idx), _ptr(k_idx), _ptr(w)
        a.k = k
        a.H, a.d_qk, a.d_v = H, d_qk, d_v
        a.dtype = _dtype_code(q)
        a.q, a.kv = _ptr(q), _ptr(kv)
        a.softmax_scale = float(scale)
        a.out, a.lse = _ptr(self.out), _ptr(self.lse)
        a.scores_out = _ptr(self.scores)
        a.ld_scores_out = int(self.scores.stride(0)) if self.scores is not None else 0
        a.indices_out = _ptr(self.indices)
        a.q_idx_scale, a.k_idx_scale = _ptr(q_idx_scale), _ptr(k_idx_scale)
        self._args = a
        # keep the inputs alive while the object lives
        self._keep = (q_idx, k_idx, w, q, kv, q_idx_scale, k_idx_scale)
        self._cs = seqs.c()
        wsz = int(_c_fwd_ws(ctypes.byref(self._cs), ctypes.byref(a)))
        self.ws_bytes = wsz
        self.noalloc = bool(noalloc)
        self.ws = None if self.noalloc else torch.empty(max(wsz, 1), dtype=torch.uint8, device=dev)

    def __call__(self, stream=None):
        if self.noalloc:
            _check(_c_fwd_na(ctypes.byref(self._cs), ctypes.byref(self._args), _stream(stream)),
                   "dsa_forward_noalloc")
        else:
            _check(_c_fwd(ctypes.byref(self._cs), ctypes.byref(self._args), _ptr(self.ws), self.ws_bytes,
                          _stream(stream)), "dsa_forward")
        return self.out, self.lse


def forward(seqs: Seqs, q_idx, k_idx, w, q, kv, k: int, scale: float, d_v: int = None, stream=None):
    """One fused forward; returns (out, lse)."""
    f = Forward(seqs, q_idx, k_idx, w, q, kv, k, scale, d_v)
    return f(stream)
