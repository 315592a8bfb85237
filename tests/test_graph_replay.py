"""The fused forward captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

Both fused entry points -- dsa_forward with a caller workspace and dsa_forward_noalloc on the
library's static scratch -- enqueue kernel launches only (no memset, copy or allocation), so a
captured call replays as the same launches on the same buffers. Each case captures one call,
then replays it several times; before every replay the inputs are overwritten in place with one
of three input sets, and eager work (an eager fused call on other buffers and, for the no-alloc
entry point, on the same scratch) plus a synchronisation sit between the replays. Every replay
must equal, bit for bit, the eager call on the same inputs: outputs, lse, indices and the
scores of every row's causal range."""
import numpy as np
import pytest

import dsa_datagen as dg

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NAMES = ("qI", "kI", "w", "q", "kv")


def _dev(x):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint8:
        t = t.view(torch.float8_e4m3fn)
    elif x.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.cuda()


def _workload(name):
    common = dict(H_I=64, d_I=128, H=128, d_qk=576, d_v=512, idx_dtype="fp8", attn_dtype="bf16")
    if name in ("decode", "decode_scaled"):
        # rows below, at and above k: split attention with its combine kernel, short rows
        return dg.custom(name=name, seqlens_q=[1] * 6, seqlens_k=[300, 5000, 2049, 17, 9000, 2048],
                         k=2048, wid=50, **common)
    if name == "prefill":
        return dg.custom(name=name, seqlens_q=[300, 40], seqlens_k=[300, 1000], k=64, wid=51, **common)
    if name == "short":
        # every sequence within k: the index-free dense path (no indexer or top-k launches)
        return dg.custom(name=name, seqlens_q=[200, 7], seqlens_k=[200, 90], k=2048, wid=52, **common)
    raise ValueError(name)


def _inputs(wl, seed, scaled):
    x = dg.gen_inputs(wl, "normal", seed=seed)
    t = {kk: _dev(x[kk]) for kk in NAMES}
    if scaled:
        g = torch.Generator().manual_seed(1000 + seed)
        t["q_idx_scale"] = (torch.rand((wl.T, wl.H_I), generator=g) * 1.5 + 0.25).cuda()
        t["k_idx_scale"] = (torch.rand((wl.Nk,), generator=g) * 1.5 + 0.25).cuda()
    return t


def _forward(gpu, seqs, wl, t, keep, noalloc):
    return gpu.Forward(seqs, t["qI"], t["kI"], t["w"], t["q"], t["kv"], wl.k, wl.scale, wl.d_v,
                       keep_scores=keep, keep_indices=keep, q_idx_scale=t.get("q_idx_scale"),
                       k_idx_scale=t.get("k_idx_scale"), noalloc=noalloc)


def _snapshot(f, pos):
    out = f.out.view(torch.int16).cpu().numpy()
    lse = f.lse.cpu().numpy()
    idx = f.indices.cpu().numpy() if f.indices is not None else None
    sc = None
    if f.scores is not None:
        s = f.scores.cpu().numpy()
        sc = [s[r, :p + 1].copy() for r, p in enumerate(pos)]
    return out, lse, idx, sc


def _same(a, b, what):
    out_a, lse_a, idx_a, sc_a = a
    out_b, lse_b, idx_b, sc_b = b
    assert np.array_equal(out_a, out_b), f"{what}: outputs differ"
    assert np.array_equal(lse_a, lse_b), f"{what}: lse differs"
    if idx_a is not None:
        assert np.array_equal(idx_a, idx_b), f"{what}: indices differ"
    if sc_a is not None:
        assert all(np.array_equal(x, y) for x, y in zip(sc_a, sc_b)), f"{what}: scores differ"


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
@pytest.mark.parametrize("name", ["decode", "decode_scaled", "prefill", "short"])
def test_graph_replay_matches_eager(gpu, name, noalloc):
    wl = _workload(name)
    scaled = name.endswith("_scaled")
    keep = name != "short"   # the short case also checks the path that launches no top-k
    print(f"graph {name} noalloc={noalloc}: T={wl.T} k={wl.k}", flush=True)
    seqs = gpu.Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    _, pos = wl.row_positions()
    sets = [_inputs(wl, seed, scaled) for seed in (1, 2, 3)]

    # eager results per input set, each on its own buffers and workspace
    refs = []
    for t in sets:
        e = _forward(gpu, seqs, wl, t, keep, noalloc=False)
        e()
        torch.cuda.synchronize()
        refs.append(_snapshot(e, pos))
    assert not np.array_equal(refs[0][0], refs[1][0]), "input sets must differ"

    live = {kk: v.clone() for kk, v in sets[0].items()}   # the buffers the graph reads
    f = _forward(gpu, seqs, wl, live, keep, noalloc)
    other = _forward(gpu, seqs, wl, {kk: v.clone() for kk, v in sets[2].items()}, keep, noalloc)

    # eager warm-up (also takes the scratch address of the device), then capture one call
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    _same(_snapshot(f, pos), refs[0], "eager warm-up")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        f()
    torch.cuda.synchronize()

    for rep, i in enumerate((1, 0, 2, 1, 1)):
        for kk in live:
            live[kk].copy_(sets[i][kk])
        f.out.zero_()
        f.lse.zero_()
        if f.indices is not None:
            f.indices.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        _same(_snapshot(f, pos), refs[i], f"replay {rep} (input set {i})")
        # eager work between replays: another fused call (for the no-alloc entry point, on the
        # same scratch), checked too
        other()
        torch.cuda.synchronize()
        _same(_snapshot(other, pos), refs[2], f"eager call after replay {rep}")
    del g
