"""GPU parity: every C-ABI entry point against the CPU oracle on the same seeded inputs.

Bars (see tests/dsa_check.py for the derivations):
  * integer-valued indexer inputs ("int" variant): scores and top-k indices bit-exact;
  * N(0,1) inputs, and FP8 codes over the whole e4m3 range ("e4m3" variant): scores within the
    accumulation error bound, top-k eps-valid;
  * inputs built so that the FP8 prefill kernel's linear term needs all four of its pieces
    while every partial sum stays exact: scores and top-k bit-exact;
  * attention (bf16): max-abs <= 2e-2, mean-abs <= 2e-3 against the oracle evaluated on the GPU's
    own validated index set; lse within 1e-3; fp32 path within 1e-4.
"""
import math
import sys

import numpy as np
import pytest

import dsa_datagen as dg
import oracle
from oracle.dsa import Seqs
from tests.dsa_check import DELTA_FP8_NORMAL, check_topk_row, fp8_delta, gamma, score_bound_row

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x, kind=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint8:
        t = t.view(torch.float8_e4m3fn)
    elif x.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.cuda()


def to_np_bf16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _same_causal_scores(wl, a, b):
    """Score rows equal on their causal part (entries past a row's position are unspecified)."""
    _, pos = wl.row_positions()
    return all(np.array_equal(a[r, :p + 1], b[r, :p + 1]) for r, p in enumerate(pos))


def run_all(gpu, wl, x):
    seqs = gpu.Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    T = {k: dev(v) for k, v in x.items() if k not in ("cu_seqlens_q", "cu_seqlens_k")}
    scores = gpu.indexer_scores(seqs, T["qI"], T["kI"], T["w"])
    idx = gpu.topk(seqs, scores, wl.k)
    out, lse = gpu.sparse_mla_attn(seqs, T["q"], T["kv"], idx, wl.scale, wl.d_v)
    fwd = gpu.Forward(seqs, T["qI"], T["kI"], T["w"], T["q"], T["kv"], wl.k, wl.scale, wl.d_v,
                      keep_scores=True, keep_indices=True)
    fout, flse = fwd()
    if wl.idx_dtype == "fp8" or wl.max_seqlen_q == 1:   # the fused indexer -> top-k call
        tsc, tidx = gpu.indexer_topk(seqs, T["qI"], T["kI"], T["w"], wl.k)
        torch.cuda.synchronize()
        assert np.array_equal(tidx.cpu().numpy(), idx.cpu().numpy()), "indexer_topk indices differ"
        assert _same_causal_scores(wl, tsc.cpu().numpy(), scores.cpu().numpy()), "indexer_topk scores differ"
    torch.cuda.synchronize()
    return dict(scores=scores.cpu().numpy(), idx=idx.cpu().numpy(), out=out, lse=lse.cpu().numpy(),
                fscores=fwd.scores.cpu().numpy(), fidx=fwd.indices.cpu().numpy(), fout=fout,
                flse=flse.cpu().numpy())


def out_np(t):
    return to_np_bf16(t) if t.dtype == torch.bfloat16 else t.cpu().numpy()


def check_rows(wl, x, res, rows, variant, delta, stats=None):
    """Every listed row against the oracle; returns the top-k overlaps with the oracle's sets
    (bounded variants). `stats`, if given, receives the largest |err| / eps of the scores."""
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    exact = variant in ("int", "split")
    outs = out_np(res["out"])
    fouts = out_np(res["fout"])
    overlaps = []
    worst = 0.0
    for r in rows:
        _, pos, _, _ = sq.locate(r)
        ref = oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"], r)
        got = res["scores"][r, :pos + 1].astype(np.float64)
        assert np.array_equal(res["fscores"][r, :pos + 1], res["scores"][r, :pos + 1]), "fused scores differ"
        if exact:
            assert np.array_equal(got, ref), f"row {r}: scores not bit-exact"
            assert res["idx"][r].tolist() == oracle.topk_row(ref, wl.k).tolist(), f"row {r}: top-k differs"
        else:
            eps = score_bound_row(sq, x["qI"], x["kI"], x["w"], r, delta)
            ratio = np.abs(got - ref) / eps
            worst = max(worst, float(ratio.max()))
            assert np.all(ratio <= 1.0), f"row {r}: {(ratio > 1).sum()} scores outside the bound, worst {ratio.max()}"
            overlaps.append(check_topk_row(res["idx"][r], ref, eps, wl.k, pos))
        assert np.array_equal(res["fidx"][r], res["idx"][r]), "fused indices differ"
        # attention on the GPU's own indices
        o, l = oracle.attn_row(sq, x["q"], x["kv"], res["idx"][r], wl.scale, wl.d_v, r)
        go = oracle.decode(outs[r])
        err = np.abs(go - o)
        if wl.attn_dtype == "bf16":
            assert err.max() <= 2e-2 and err.mean() <= 2e-3, f"row {r}: attn max {err.max()} mean {err.mean()}"
        else:
            assert err.max() <= 1e-4, f"row {r}: fp32 attn max err {err.max()}"
        fin = np.isfinite(l)
        assert np.array_equal(fin, np.isfinite(res["lse"][r]))
        assert np.all(np.abs(res["lse"][r][fin] - l[fin]) <= 1e-3)
        assert np.array_equal(fouts[r], outs[r]), "fused output differs"
        assert np.array_equal(res["flse"][r], res["lse"][r])
    if stats is not None:
        stats["worst_ratio"] = worst
    return overlaps


SMALL = {
    # name: (seqlens_q, seqlens_k, k)
    "prefill300_k64": ([300], [300], 64),
    "multiseq_k128": ([5, 37, 0, 130], [40, 37, 3, 700], 128),
    "decode_ragged_k2048": ([1, 1, 1, 1, 1], [1, 17, 300, 2100, 5000], 2048),
    "chunk_tail_k256": ([70], [1500], 256),
    # k not a multiple of the attention's 64-entry blocks: the last block of a list is partial,
    # and rows with at most k candidates (positions < 100) take the prefix-list path
    "odd_k100": ([3, 150], [400, 150], 100),
}


@pytest.mark.parametrize("variant", ["int", "normal", "e4m3"])
@pytest.mark.parametrize("case", list(SMALL))
def test_small_fp8_bf16(gpu, case, variant):
    sqs, sks, k = SMALL[case]
    wl = dg.custom(name=case, seqlens_q=sqs, seqlens_k=sks, H_I=64, d_I=128, k=k, H=128, d_qk=576,
                   d_v=512, idx_dtype="fp8", attn_dtype="bf16", wid=20 + list(SMALL).index(case))
    say(f"case {case} variant {variant} T={wl.T} Nk={wl.Nk}")
    x = dg.gen_inputs(wl, variant, seed=7)
    res = run_all(gpu, wl, x)
    st = {}
    ov = check_rows(wl, x, res, range(wl.T), variant, fp8_delta(variant), st)
    if ov:
        say(f"  mean overlap with the oracle set {np.mean(ov):.4f}; worst |err|/eps {st['worst_ratio']:.3g}")


@pytest.mark.parametrize("shape", [([40, 9], [600, 9]), ([1, 1, 1], [300, 77, 2500])])
def test_indexer_linear_split_exact(gpu, shape):
    """Inputs whose weighted query sum u needs all four FP8 pieces of the prefill kernel's linear
    term, with every partial sum exact in fp32 (dsa_datagen.gen_linear_split; the CPU model check
    is tests/test_score_bound.py): scores and top-k must equal the oracle bit for bit, so a piece
    that is dropped or scaled wrongly shows. The second shape runs the decode kernel on the same
    kind of rows."""
    sq_q, sq_k = shape
    wl = dg.custom(name="split", seqlens_q=sq_q, seqlens_k=sq_k, H_I=64, d_I=128, k=64, H=128, d_qk=576,
                   d_v=512, idx_dtype="fp8", attn_dtype="bf16", wid=37)
    x = dict(dg.gen_inputs(wl, "normal", seed=2, parts=("attn",)), **dg.gen_linear_split(wl, seed=2))
    res = run_all(gpu, wl, x)
    check_rows(wl, x, res, range(wl.T), "split", None)


def _fused_decode_indices(gpu, wl, x):
    """Indices of the fused indexer -> top-k call (decode batches: the indexer keeps per-chunk
    candidates and a merge selects) and of the separate indexer + top-k calls on the same inputs."""
    seqs = gpu.Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    T = {kk: dev(v) for kk, v in x.items() if kk in ("qI", "kI", "w")}
    fsc, fidx = gpu.indexer_topk(seqs, T["qI"], T["kI"], T["w"], wl.k)
    scores = gpu.indexer_scores(seqs, T["qI"], T["kI"], T["w"])
    idx = gpu.topk(seqs, scores, wl.k)
    torch.cuda.synchronize()
    assert _same_causal_scores(wl, fsc.cpu().numpy(), scores.cpu().numpy()), "fused and separate scores differ"
    return fidx.cpu().numpy(), idx.cpu().numpy(), fsc.cpu().numpy()


@pytest.mark.parametrize("k", [2048, 64])
def test_decode_fused_topk_rows(gpu, k):
    """The fused decode top-k on integer inputs (exact scores) against the oracle, bit for bit:
    rows of k + 1 keys up to the longest supported (131072), with ordinary rows and rows built to
    defeat the per-chunk candidates -- the top scores all in one chunk (the merge must detect that
    the chunk dropped keys above the threshold and select exactly from the scores), all scores
    equal (every chunk overflows on ties), and scores with only a few distinct values (many ties
    at the threshold across chunks, lowest positions first)."""
    lens = [k + 1, 3000, 5000, 32768, 65537, 131072, 40000, 40000, 40000, 1, 17]
    wl = dg.custom(name="fused_decode", seqlens_q=[1] * len(lens), seqlens_k=lens, H_I=64, d_I=128, k=k,
                   H=128, d_qk=576, d_v=512, idx_dtype="fp8", attn_dtype="bf16", wid=38)
    x = dg.gen_inputs(wl, "int", seed=11, parts=("idx",))
    cu_k = wl.cu_seqlens_k
    qI, kI, w = x["qI"], x["kI"].copy(), x["w"].copy()
    three = dg.to_fp8_e4m3fn_bytes(np.full(1, 3.0, np.float32))[0]
    # row 6: keys 5000..6023 (one chunk) score far above every other key
    qI = qI.copy()
    qI[6] = three
    w[6] = 1.0
    kI[cu_k[6] + 5000:cu_k[6] + 6024] = three
    # row 7: all scores zero
    w[7] = 0.0
    # row 8: ternary keys and queries, one head: scores take a few values only
    t = dg.gen_ternary(wl, seed=3)
    qI[8] = t["qI"][8]
    kI[cu_k[8]:cu_k[9]] = t["kI"][cu_k[8]:cu_k[9]]
    w[8] = 0.0
    w[8, 5] = 0.5
    x.update(qI=qI, kI=kI, w=w)
    fidx, sidx, fsc = _fused_decode_indices(gpu, wl, x)
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    for r in range(wl.T):
        ref_sc = oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"], r)
        _, pos, _, _ = sq.locate(r)
        assert np.array_equal(fsc[r, :pos + 1].astype(np.float64), ref_sc), f"row {r}: scores"
        ref = oracle.topk_row(ref_sc, k)
        assert fidx[r].tolist() == ref.tolist(), f"row {r} (n = {lens[r]}): fused top-k differs from the oracle"
        assert np.array_equal(sidx[r], fidx[r]), f"row {r}: fused and separate top-k differ"
    assert fidx[7, :k].tolist() == list(range(k))


@pytest.mark.parametrize("variant", ["int", "normal"])
def test_tiny_fp32_all_rows(gpu, variant):
    wl = dg.workload("tiny")
    x = dg.gen_inputs(wl, variant, seed=0)
    res = run_all(gpu, wl, x)
    check_rows(wl, x, res, range(wl.T), variant, gamma(wl.d_I))


def test_dense_special_case_bf16(gpu):
    """k >= every candidate count: the selection is every causal key (exact), and the attention
    is dense causal attention."""
    wl = dg.custom(name="dense", seqlens_q=[96], seqlens_k=[96], H_I=64, d_I=128, k=128, H=128,
                   d_qk=576, d_v=512, idx_dtype="fp8", attn_dtype="bf16", wid=30)
    x = dg.gen_inputs(wl, "normal", seed=1)
    res = run_all(gpu, wl, x)
    for r in range(wl.T):
        assert res["idx"][r].tolist() == list(range(r + 1)) + [-1] * (wl.k - r - 1)
    check_rows(wl, x, res, range(wl.T), "normal", DELTA_FP8_NORMAL)


@pytest.mark.parametrize("shape", [([5, 40, 1], [40, 100, 7], 128), ([1, 1, 1, 1], [100, 2000, 2048, 64], 2048)])
def test_short_context_forward(gpu, shape):
    """Every sequence has at most k keys: the fused call skips the indexer and the top-k and walks
    all causal candidates. Its output must equal, bit for bit, the attention call on the explicit
    list 0..pos (same kernel arithmetic), and the oracle within the attention bar. The second shape
    is a decode batch (the rows are split over several workgroups)."""
    sq_q, sq_k, k = shape
    wl = dg.custom(name="short", seqlens_q=sq_q, seqlens_k=sq_k, H_I=64, d_I=128, k=k, H=128,
                   d_qk=576, d_v=512, idx_dtype="fp8", attn_dtype="bf16", wid=33)
    x = dg.gen_inputs(wl, "normal", seed=7)
    seqs = gpu.Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    T = {kk: dev(v) for kk, v in x.items() if kk not in ("cu_seqlens_q", "cu_seqlens_k")}
    fwd = gpu.Forward(seqs, T["qI"], T["kI"], T["w"], T["q"], T["kv"], wl.k, wl.scale, wl.d_v)
    fout, flse = fwd()
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    full = np.full((wl.T, k), -1, np.int32)
    for r in range(wl.T):
        _, pos, _, _ = sq.locate(r)
        full[r, :pos + 1] = np.arange(pos + 1)
    out, lse = gpu.sparse_mla_attn(seqs, T["q"], T["kv"], dev(full), wl.scale, wl.d_v)
    torch.cuda.synchronize()
    fo, o = to_np_bf16(fout), to_np_bf16(out)
    assert np.array_equal(fo, o), "implicit candidate list differs from the explicit one"
    assert np.array_equal(flse.cpu().numpy(), lse.cpu().numpy())
    for r in range(wl.T):
        ref, refl = oracle.attn_row(sq, x["q"], x["kv"], full[r], wl.scale, wl.d_v, r)
        err = np.abs(oracle.decode(fo[r]) - ref)
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, f"row {r}: max {err.max()} mean {err.mean()}"
        assert np.all(np.abs(flse[r].cpu().numpy() - refl) <= 1e-3)


SCALED = {
    # name: (seqlens_q, seqlens_k, H_I, d_I, idx dtype, k)
    "prefill_fp8": ([300, 37], [300, 700], 64, 128, "fp8", 64),
    "decode_fp8": ([1, 1, 1], [40, 2100, 5000], 64, 128, "fp8", 256),
    "tiny_f32": ([50], [80], 4, 32, "f32", 16),
}


@pytest.mark.parametrize("sides", ["both", "q", "k"])
@pytest.mark.parametrize("variant", ["int", "normal"])
@pytest.mark.parametrize("case", list(SCALED))
def test_scaled_indexer(gpu, case, variant, sides):
    """Scaled indexer inputs (per query row and head, per key) against the oracle on the scaled
    vectors: bit-exact for integer inputs with power-of-two scales, else within the bound; the
    fused call with the same scales gives the same scores, and (integer case) the oracle's
    top-k."""
    sq_q, sq_k, H_I, d_I, idt, k = SCALED[case]
    wl = dg.custom(name="scaled", seqlens_q=sq_q, seqlens_k=sq_k, H_I=H_I, d_I=d_I, k=k, H=128,
                   d_qk=576, d_v=512, idx_dtype=idt, attn_dtype="bf16", wid=34)
    x = dg.gen_inputs(wl, variant, seed=3)
    sc = dg.gen_scales(wl, variant, seed=3)
    qs = sc["q_scale"] if sides in ("both", "q") else None
    ks = sc["k_scale"] if sides in ("both", "k") else None
    seqs = gpu.Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    T = {kk: dev(v) for kk, v in x.items() if kk not in ("cu_seqlens_q", "cu_seqlens_k")}
    dqs = dev(qs) if qs is not None else None
    dks = dev(ks) if ks is not None else None
    scores = gpu.indexer_scores_scaled(seqs, T["qI"], dqs, T["kI"], dks, T["w"])
    fwd = gpu.Forward(seqs, T["qI"], T["kI"], T["w"], T["q"], T["kv"], wl.k, wl.scale, wl.d_v,
                      keep_scores=True, keep_indices=True, q_idx_scale=dqs, k_idx_scale=dks)
    fwd()
    torch.cuda.synchronize()
    got_all, fs, fi = scores.cpu().numpy(), fwd.scores.cpu().numpy(), fwd.indices.cpu().numpy()
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    delta = DELTA_FP8_NORMAL if idt == "fp8" else gamma(d_I)
    for r in range(wl.T):
        _, pos, _, _ = sq.locate(r)
        ref = oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"], r, qs, ks)
        got = got_all[r, :pos + 1].astype(np.float64)
        assert np.array_equal(fs[r, :pos + 1], got_all[r, :pos + 1]), f"row {r}: fused scores differ"
        if variant == "int":
            assert np.array_equal(got, ref), f"row {r}: scaled scores not bit-exact"
            assert fi[r].tolist() == oracle.topk_row(ref, wl.k).tolist(), f"row {r}: top-k differs"
        else:
            eps = score_bound_row(sq, x["qI"], x["kI"], x["w"], r, delta, qs, ks)
            bad = np.abs(got - ref) > eps
            assert not bad.any(), f"row {r}: worst {np.max(np.abs(got - ref) / eps)}"


def _alignment_check(sq, x, wl, idx, scores_gpu, lse_gpu, tgt, kl):
    """Per entry, the GPU's p differs from the exact one by the logit error (fp32 accumulation:
    gamma(d_qk + 1) * scale * sum_d |q_hd c_ed|) plus its lse error (GPU lse against the exact
    lse over the same entries), both in the exponent; the KL bound follows term by term."""
    for r in range(wl.T):
        _, pos, k0, _ = sq.locate(r)
        ref_t, ref_kl = oracle.alignment_row(sq, x["q"], x["kv"], idx[r], wl.scale, scores_gpu[r].astype(np.float64), r)
        row = np.asarray(idx[r], np.int64)
        v = (row >= 0) & (row <= pos)
        if not v.any():
            assert np.all(tgt[r] == 0) and kl[r] == 0
            continue
        qr = oracle.decode(x["q"][r])
        c = oracle.decode(x["kv"][k0 + row[v]])
        _, lse_ex = oracle.attn_row(sq, x["q"], x["kv"], row[v], wl.scale, wl.d_v, r)
        dl = np.abs(lse_gpu[r].astype(np.float64) - lse_ex)                    # [H]
        ez = gamma(wl.d_qk + 1) * wl.scale * (np.abs(qr) @ np.abs(c).T)        # [H, |S|]
        delta = np.max(ez + dl[:, None], axis=0) + 1e-6                        # + exp/rounding
        rel = np.expm1(delta)
        p = ref_t[v]
        got = tgt[r][v].astype(np.float64)
        assert np.all(np.abs(got - p) <= rel * p + 1e-12), f"row {r}: target outside the bound"
        assert np.all(tgt[r][~v] == 0)
        sv = scores_gpu[r].astype(np.float64)[row[v]]
        lq = sv - sv.max() - np.log(np.sum(np.exp(sv - sv.max())))
        bound = np.sum(p * (rel * (np.abs(np.log(p) - lq) + 1) + delta)) + 1e-5
        assert abs(float(kl[r]) - ref_kl) <= bound, f"row {r}: kl {kl[r]} vs {ref_kl} (bound {bound})"


@pytest.mark.parametrize("case", ["prefill", "decode"])
def test_indexer_alignment(gpu, case):
    """Alignment target and KL on the GPU's own indices, scores and lse (the steps before are
    tested on their own) against the oracle; prefill rows with short (k > candidates) and long
    rows, and a decode batch."""
    if case == "prefill":
        sq_q, sq_k, k = [5, 37, 70], [40, 37, 1500], 128
    else:
        sq_q, sq_k, k = [1, 1, 1], [17, 2100, 5000], 2048
    wl = dg.custom(name="align", seqlens_q=sq_q, seqlens_k=sq_k, H_I=64, d_I=128, k=k, H=128,
                   d_qk=576, d_v=512, idx_dtype="fp8", attn_dtype="bf16", wid=35)
    x = dg.gen_inputs(wl, "normal", seed=9)
    seqs = gpu.Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    T = {kk: dev(v) for kk, v in x.items() if kk not in ("cu_seqlens_q", "cu_seqlens_k")}
    scores = gpu.indexer_scores(seqs, T["qI"], T["kI"], T["w"])
    idx = gpu.topk(seqs, scores, wl.k)
    _, lse = gpu.sparse_mla_attn(seqs, T["q"], T["kv"], idx, wl.scale, wl.d_v)
    tgt, kl = gpu.indexer_alignment(seqs, T["q"], T["kv"], idx, wl.scale, lse, scores)
    _, kl2 = gpu.indexer_alignment(seqs, T["q"], T["kv"], idx, wl.scale, lse, scores, with_target=False)
    torch.cuda.synchronize()
    assert np.array_equal(kl.cpu().numpy(), kl2.cpu().numpy())
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    _alignment_check(sq, x, wl, idx.cpu().numpy(), scores.cpu().numpy(), lse.cpu().numpy(),
                     tgt.cpu().numpy(), kl.cpu().numpy())


def test_indexer_alignment_edge_lists(gpu):
    """-1 entries, repeats, an entry list with a single valid key, a row without one."""
    wl = dg.custom(name="align_edge", seqlens_q=[4], seqlens_k=[50], H_I=64, d_I=128, k=70, H=128,
                   d_qk=576, d_v=512, idx_dtype="fp8", attn_dtype="bf16", wid=36)
    x = dg.gen_inputs(wl, "normal", seed=4)
    rng = np.random.default_rng(8)
    idx = np.full((4, 70), -1, np.int32)
    idx[0, :40] = rng.integers(0, 47, 40)      # row 0 sits at position 46: repeats, unsorted
    idx[1, 5:9] = [40, 3, 3, 47]               # position 47
    idx[2, 69] = 11                            # single valid entry at the end
    seqs = gpu.Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    T = {kk: dev(v) for kk, v in x.items() if kk not in ("cu_seqlens_q", "cu_seqlens_k")}
    scores = gpu.indexer_scores(seqs, T["qI"], T["kI"], T["w"])
    didx = dev(idx)
    _, lse = gpu.sparse_mla_attn(seqs, T["q"], T["kv"], didx, wl.scale, wl.d_v)
    tgt, kl = gpu.indexer_alignment(seqs, T["q"], T["kv"], didx, wl.scale, lse, scores)
    torch.cuda.synchronize()
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    _alignment_check(sq, x, wl, idx, scores.cpu().numpy(), lse.cpu().numpy(), tgt.cpu().numpy(),
                     kl.cpu().numpy())
    assert kl[3].item() == 0.0


def test_indexer_weight_extremes(gpu):
    """Rows whose head weights span the fp32 range (huge, tiny, zero, all negative, a single
    nonzero head): the per-row scaling of the FP8 prefill path's linear term must hold the error
    bound on every row."""
    wl = dg.custom(name="wext", seqlens_q=[40], seqlens_k=[300], H_I=64, d_I=128, k=64, H=128,
                   d_qk=576, d_v=512, idx_dtype="fp8", attn_dtype="bf16", wid=32)
    x = dg.gen_inputs(wl, "normal", seed=5)
    w = x["w"].copy()
    w[0] *= np.float32(2.0 ** 40)
    w[1] *= np.float32(2.0 ** -60)
    w[2] = 0.0
    w[3] = -np.abs(w[3])
    w[4] = 0.0
    w[4, 17] = np.float32(1e-3)
    w[5] *= np.float32(2.0 ** -110)
    w[6] = np.abs(w[6])
    x["w"] = w
    res = run_all(gpu, wl, x)
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    for r in range(wl.T):
        _, pos, _, _ = sq.locate(r)
        ref = oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"], r)
        got = res["scores"][r, :pos + 1].astype(np.float64)
        eps = score_bound_row(sq, x["qI"], x["kI"], x["w"], r, DELTA_FP8_NORMAL)
        assert np.all(np.abs(got - ref) <= eps), f"row {r}: worst {np.max(np.abs(got - ref) - eps)}"
        if r == 2:
            assert np.all(got == 0.0)


def test_attention_edge_indices(gpu):
    """-1 and out-of-range indices are skipped, repeats count twice, an empty row gives 0 / -inf."""
    wl = dg.custom(name="edge", seqlens_q=[4], seqlens_k=[50], H=128, d_qk=576, d_v=512,
                   idx_dtype="fp8", attn_dtype="bf16", wid=31, k=70)
    x = dg.gen_inputs(wl, "normal", seed=2, parts=("attn",))
    rng = np.random.default_rng(3)
    idx = np.full((4, 70), -1, np.int32)
    idx[0, :40] = rng.integers(0, 50, 40)          # unsorted, with repeats
    idx[1, 5:9] = [49, 50, 1000, -7]               # out of range entries
    idx[2, 69] = 3                                 # single valid at the end
    seqs = gpu.Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    out, lse = gpu.sparse_mla_attn(seqs, dev(x["q"]), dev(x["kv"]), dev(idx), wl.scale, 512)
    torch.cuda.synchronize()
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    outs, lses = to_np_bf16(out), lse.cpu().numpy()
    for r in range(4):
        o, l = oracle.attn_row(sq, x["q"], x["kv"], idx[r], wl.scale, 512, r)
        err = np.abs(oracle.decode(outs[r]) - o)
        assert err.max() <= 2e-2 and err.mean() <= 2e-3
        fin = np.isfinite(l)
        assert np.array_equal(fin, np.isfinite(lses[r]))
        assert np.all(np.abs(lses[r][fin] - l[fin]) <= 1e-3)
    assert np.all(oracle.decode(outs[3]) == 0) and np.all(lses[3] == -np.inf)


@pytest.mark.parametrize("T", [300, 3])
def test_attention_reference_restart(gpu, T):
    """Latent rows whose rope part is 64 times larger in the second half of every 64-entry block:
    those logits exceed the reference taken from the first half by far more than the weights'
    fp32 range allows, so rows restart with a larger reference (T = 300: one workgroup per row;
    T = 3: each row split into one-block runs, each of which restarts, then merged)."""
    nk, k = 2048, 1024
    wl = dg.custom(name="restart", seqlens_q=[T], seqlens_k=[nk], H=128, d_qk=576, d_v=512,
                   idx_dtype="fp8", attn_dtype="bf16", wid=33, k=k)
    x = dg.gen_inputs(wl, "normal", seed=4, parts=("attn",))
    q, kv = oracle.decode(x["q"]), oracle.decode(x["kv"])
    q[..., 512:] *= 2.0                                  # powers of two: exact in bf16
    kv[(np.arange(nk) // 32) % 2 == 1, 512:] *= 64.0
    x["q"], x["kv"] = dg.to_bf16_bits(q), dg.to_bf16_bits(kv)
    idx = np.tile(np.arange(k, dtype=np.int32), (T, 1))
    seqs = gpu.Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    out, lse = gpu.sparse_mla_attn(seqs, dev(x["q"]), dev(x["kv"]), dev(idx), wl.scale, 512)
    torch.cuda.synchronize()
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    outs, lses = to_np_bf16(out), lse.cpu().numpy()
    for r in range(0, T, 7 if T > 50 else 1):
        o, l = oracle.attn_row(sq, x["q"], x["kv"], idx[r], wl.scale, 512, r)
        err = np.abs(oracle.decode(outs[r]) - o)
        # the weights are nearly one-hot here, so outputs are single latent values (up to ~4.5):
        # the bf16 rounding of the weights (2^-9 relative, in the numerator only) and of the
        # output (2^-9 relative) reach one bf16 step of such values, beyond the absolute 2e-2
        assert np.all(err <= 2e-2 + np.abs(o) * 2.0 ** -7), f"row {r}: worst {np.max(err - np.abs(o) * 2.0 ** -7)}"
        assert err.mean() <= 2e-3, f"row {r}: mean {err.mean()}"
        assert np.all(np.abs(lses[r] - l) <= 1e-3), f"row {r}: lse {np.max(np.abs(lses[r] - l))}"


@pytest.mark.parametrize("T", [4, 260])
def test_attention_nonfinite_query(gpu, T):
    """A NaN or an infinity in one head's query makes only that head's output non-finite (T = 4:
    split rows, merged; T = 260: one workgroup per row): the other heads match the oracle, and
    the row does not keep restarting (no larger reference exists for such logits)."""
    nk, k = 600, 512
    wl = dg.custom(name="nonfinite", seqlens_q=[T], seqlens_k=[nk], H=128, d_qk=576, d_v=512,
                   idx_dtype="fp8", attn_dtype="bf16", wid=34, k=k)
    x = dg.gen_inputs(wl, "normal", seed=6, parts=("attn",))
    q = oracle.decode(x["q"])
    bad = {0: (5, np.nan), 1: (40, np.inf), 2: (100, -np.inf)}
    for r, (h, v) in bad.items():
        q[r, h, 3] = v
    x["q"] = dg.to_bf16_bits(q)
    idx = np.tile(np.arange(k, dtype=np.int32), (T, 1))
    seqs = gpu.Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    out, lse = gpu.sparse_mla_attn(seqs, dev(x["q"]), dev(x["kv"]), dev(idx), wl.scale, 512)
    torch.cuda.synchronize()
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    outs = oracle.decode(to_np_bf16(out))
    for r in sorted(set(bad) | set(range(0, T, 37))):
        o, _ = oracle.attn_row(sq, x["q"], x["kv"], idx[r], wl.scale, 512, r)
        keep = np.ones(128, bool)
        if r in bad:
            keep[bad[r][0]] = False
            assert not np.isfinite(outs[r, bad[r][0]]).all(), f"row {r}: the head with a non-finite query"
        err = np.abs(outs[r, keep] - o[keep])
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, f"row {r}: max {err.max()} mean {err.mean()}"


def test_topk_ties_and_zeros(gpu):
    """Many equal scores and signed zeros: lower positions win, +0 == -0."""
    T, n, k = 6, 3000, 100
    rng = np.random.default_rng(4)
    sc = rng.integers(-3, 4, size=(T, n)).astype(np.float32)
    sc[1] = 0.0
    sc[2] = np.where(rng.random(n) < 0.5, 0.0, -0.0).astype(np.float32)
    sc[3] = 5.0
    sc[4, :] = -1.0
    sc[4, 2900:] = 2.0
    cu_q, cu_k = [0, T], [0, n]
    # T query rows at positions n-T .. n-1
    seqs = gpu.Seqs(cu_q, cu_k)
    idx = gpu.topk(seqs, torch.from_numpy(sc).cuda(), k).cpu().numpy()
    for r in range(T):
        pos = n - T + r
        assert idx[r].tolist() == oracle.topk_row(sc[r, :pos + 1].astype(np.float64), k).tolist()


@pytest.mark.parametrize("rows,k", [(5, 2048), (600, 2048), (5, 4096)])
@pytest.mark.parametrize("n", [5000, 8200, 30000, 32768, 131072, 140000])
def test_topk_row_lengths_and_degenerate_rows(gpu, n, rows, k):
    """Every top-k code path: the streaming kernel with its exact fallback (k <= 2048, rows up to
    131072, small and large batches), register-resident rows of 1, 2..8, 9..32 tiles of 4096
    (larger k), the multi-pass kernel beyond 131072 -- each with degenerate rows: all equal,
    all +-0, one distinct value, integer ties, random floats, a row whose largest values all
    sit outside the sampled runs, and a row whose selection crosses zero."""
    rng = np.random.default_rng(n + rows)
    late = rng.standard_normal(n).astype(np.float32)
    late[n - 3000:] += 50.0   # the top scores cluster in one stretch of the row
    # the selection crosses zero: 700 positive scores, the rest negative, so the floor of the
    # candidate list is negative and its maximum positive (their keys differ in the top bit)
    cross = -np.abs(rng.standard_normal(n)).astype(np.float32)
    cross[rng.choice(n - 10, 700, replace=False)] = rng.uniform(1.0, 2.0, 700).astype(np.float32)
    pats = [np.full(n, 1.5, np.float32),
            np.where(rng.random(n) < 0.5, 0.0, -0.0).astype(np.float32),
            np.concatenate([np.full(n - 1, -2.0, np.float32), [3.0]]).astype(np.float32),
            rng.integers(-4, 5, size=n).astype(np.float32),
            rng.standard_normal(n).astype(np.float32),
            late, cross]
    T = max(rows, len(pats))
    sc = np.empty((T, n), np.float32)
    for r in range(T):
        sc[r] = pats[r] if r < len(pats) else rng.standard_normal(n).astype(np.float32)
    seqs = gpu.Seqs([0, T], [0, n])
    idx = gpu.topk(seqs, torch.from_numpy(sc).cuda(), k).cpu().numpy()
    check = list(range(len(pats))) + list(range(len(pats), T, max(1, T // 8)))[:8] + [T - 1]
    for r in check:
        pos = n - T + r
        assert idx[r].tolist() == oracle.topk_row(sc[r, :pos + 1].astype(np.float64), k).tolist(), f"row {r}"


def test_empty_batch_is_noop(gpu):
    seqs = gpu.Seqs([0], [0])
    z = torch.zeros(16, device="cuda")
    gpu.indexer_scores(seqs, z.view(1, 1, 16)[:0], z.view(1, 16)[:0], z.view(16, 1)[:0], scores=z.view(4, 4)[:0])
    e8 = torch.zeros(0, 64, 128, dtype=torch.float8_e4m3fn, device="cuda")
    out, lse = gpu.forward(seqs, e8, torch.zeros(0, 128, dtype=torch.float8_e4m3fn, device="cuda"),
                           torch.zeros(0, 64, device="cuda"),
                           torch.zeros(0, 128, 576, dtype=torch.bfloat16, device="cuda"),
                           torch.zeros(0, 576, dtype=torch.bfloat16, device="cuda"), 2048, 0.04)
    torch.cuda.synchronize()
    assert out.shape == (0, 128, 512) and lse.shape == (0, 128)


# ------------------------------------------------------------------ full-size workloads

# rows checked against the oracle: every row of the decode batches, sampled rows of the prefills
FULL_ROWS = {
    "prefill8k": [0, 1, 63, 2046, 2047, 2048, 4095, 5000, 8190, 8191] + list(range(100, 8192, 173)),
    "decode32k": None,
    "chunk128k": [0, 1, 2047, 4094, 4095] + list(range(37, 4096, 211)),
    "ragged": None,
}
# floor of the mean overlap of the GPU's top-k sets with the oracle's on N(0,1) data (different
# sets are valid where scores lie within the rounding error of the k-th one; the eps-valid check
# is the bar, this guards against a systematic shift)
MIN_MEAN_OVERLAP = 0.99


@pytest.mark.parametrize("variant", ["int", "normal"])
@pytest.mark.parametrize("name", list(FULL_ROWS))
def test_full_size_rows(gpu, name, variant):
    """The shapes and launch configuration the benchmark times: int variant, scores and indices
    bit-exact; N(0,1) variant (the benchmark's data), scores within the error bound, the top-k
    eps-valid and its mean overlap with the oracle's sets at least MIN_MEAN_OVERLAP; attention
    within tolerance on the GPU's indices. Every row of the decode batches, sampled rows of the
    prefills."""
    wl = dg.workload(name)
    say(f"full {name} ({variant}): generating T={wl.T} Nk={wl.Nk}")
    x = dg.gen_inputs(wl, variant, seed=0)
    say("  running")
    res = run_all(gpu, wl, x)
    rows = FULL_ROWS[name] if FULL_ROWS[name] is not None else range(wl.T)
    say(f"  checking {len(rows)} rows")
    st = {}
    ov = check_rows(wl, x, res, rows, variant, DELTA_FP8_NORMAL, st)
    if ov:
        say(f"  overlap with the oracle sets: mean {np.mean(ov):.5f} min {np.min(ov):.5f}; "
            f"worst |err|/eps {st['worst_ratio']:.3g}")
        assert np.mean(ov) >= MIN_MEAN_OVERLAP, f"mean overlap {np.mean(ov)}"
