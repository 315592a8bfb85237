"""dsa_forward_noalloc (the fused forward on the library's static device scratch) against
dsa_forward (caller workspace) through the C ABI: identical outputs, lse, scores and indices, on
two calls in a row -- the second with a smaller batch, so that it runs on scratch left over from
the first -- and a prefill batch that fits; a batch whose workspace exceeds the scratch is
rejected."""
import sys

import numpy as np
import pytest

import dsa_datagen as dg

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dev(x):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint8:
        t = t.view(torch.float8_e4m3fn)
    elif x.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.cuda()


def _both(gpu, wl, seed):
    x = dg.gen_inputs(wl, "normal", seed=seed)
    T = {kk: _dev(v) for kk, v in x.items() if kk not in ("cu_seqlens_q", "cu_seqlens_k")}
    seqs = gpu.Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    args = (seqs, T["qI"], T["kI"], T["w"], T["q"], T["kv"], wl.k, wl.scale, wl.d_v)
    ref = gpu.Forward(*args, keep_scores=True, keep_indices=True)
    na = gpu.Forward(*args, keep_scores=True, keep_indices=True, noalloc=True)
    assert na.ws is None and na.ws_bytes <= gpu.NOALLOC_SCRATCH_BYTES
    ref()
    na()
    torch.cuda.synchronize()
    _, pos = wl.row_positions()
    out_r, out_n = ref.out.view(torch.int16).cpu().numpy(), na.out.view(torch.int16).cpu().numpy()
    assert np.array_equal(out_r, out_n), "outputs differ"
    assert np.array_equal(ref.lse.cpu().numpy(), na.lse.cpu().numpy()), "lse differs"
    assert np.array_equal(ref.indices.cpu().numpy(), na.indices.cpu().numpy()), "indices differ"
    sr, sn = ref.scores.cpu().numpy(), na.scores.cpu().numpy()
    assert all(np.array_equal(sr[r, :p + 1], sn[r, :p + 1]) for r, p in enumerate(pos)), "scores differ"
    return na


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_forward_matches_forward(gpu, order):
    big = dg.custom(name="na_big", seqlens_q=[1] * 64, seqlens_k=[32768] * 64, H_I=64, d_I=128, k=2048,
                    H=128, d_qk=576, d_v=512, idx_dtype="fp8", attn_dtype="bf16", wid=40)
    small = dg.custom(name="na_small", seqlens_q=[1] * 5, seqlens_k=[300, 5000, 2049, 17, 9000], H_I=64,
                      d_I=128, k=2048, H=128, d_qk=576, d_v=512, idx_dtype="fp8", attn_dtype="bf16", wid=41)
    prefill = dg.custom(name="na_prefill", seqlens_q=[300, 40], seqlens_k=[300, 1000], H_I=64, d_I=128, k=64,
                        H=128, d_qk=576, d_v=512, idx_dtype="fp8", attn_dtype="bf16", wid=42)
    for wl in (big, small, prefill):
        print(f"noalloc {wl.name}: T={wl.T}", flush=True)
        _both(gpu, wl, seed=1)


def test_noalloc_rejects_batches_beyond_the_scratch(gpu):
    wl = dg.workload("prefill8k")   # scores alone need 268 MB
    seqs = gpu.Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    e8 = torch.zeros((wl.T, 64, 128), dtype=torch.float8_e4m3fn, device="cuda")
    f = gpu.Forward(seqs, e8, torch.zeros((wl.Nk, 128), dtype=torch.float8_e4m3fn, device="cuda"),
                    torch.zeros((wl.T, 64), device="cuda"),
                    torch.zeros((wl.T, 128, 576), dtype=torch.bfloat16, device="cuda"),
                    torch.zeros((wl.Nk, 576), dtype=torch.bfloat16, device="cuda"), wl.k, wl.scale, wl.d_v,
                    noalloc=True)
    assert f.ws_bytes > gpu.NOALLOC_SCRATCH_BYTES
    with pytest.raises(gpu.DSAError) as e:
        f()
    assert e.value.status == gpu.DSA_ERR_WORKSPACE and "scratch" in str(e.value)
