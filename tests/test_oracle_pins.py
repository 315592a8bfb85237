"""Pins of the CPU oracle against facts fixed outside the oracle itself.

- the number formats: every FP8 e4m3fn code and a sweep of bf16 patterns against torch's own
  conversions (an independent implementation), plus values fixed by the format definition;
- hand-worked cases (tests/golden/handworked.json), derived by hand from the definitions;
- brute force: pure-Python loops and a sort-free top-k on tiny random inputs;
- special cases that reduce to a textbook routine: k >= number of candidates turns DSA into
  dense causal MQA attention, checked against torch's scaled_dot_product_attention in float64;
- invariants of the definitions (exact on integer-valued inputs).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import dsa_datagen as dg
import oracle
from oracle import brute
from oracle.dsa import Seqs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked.json")


# ------------------------------------------------------------------ number formats

def test_fp8_table_matches_torch_all_codes():
    tab = oracle.fp8_e4m3fn_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(tab), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(tab[~nan], ref[~nan])


def test_fp8_table_format_facts():
    tab = oracle.fp8_e4m3fn_table()
    assert tab[0x38] == 1.0            # exponent field 7 = bias
    assert tab[0x7E] == 448.0          # largest finite
    assert tab[0x01] == 2.0 ** -9      # smallest subnormal
    assert tab[0x08] == 2.0 ** -6      # smallest normal
    assert tab[0xB8] == -1.0
    assert tab[0x80] == 0.0 and math.copysign(1, tab[0x80]) == -1.0


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = np.concatenate([np.arange(0, 65536, 7, dtype=np.uint32),
                           rng.integers(0, 65536, 5000)]).astype(np.uint16)
    mine = oracle.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


def test_datagen_roundtrip_is_nearest():
    """The stored FP8 / bf16 inputs decode to the nearest representable value of the draw."""
    x = np.random.default_rng(1).standard_normal(4096).astype(np.float32) * 3
    f8 = oracle.decode(dg.to_fp8_e4m3fn_bytes(x))
    grid = np.unique(oracle.fp8_e4m3fn_table()[~np.isnan(oracle.fp8_e4m3fn_table())])
    best = np.abs(grid[None, :] - x[:, None].astype(np.float64)).min(axis=1)
    assert np.allclose(np.abs(f8 - x), best, rtol=0, atol=0)
    b = oracle.decode(dg.to_bf16_bits(x))
    assert np.all(np.abs(b - x) <= np.abs(x) * 2.0 ** -8)


# ------------------------------------------------------------------ hand-worked cases

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["indexer"], ids=lambda c: c["name"])
def test_handworked_indexer_and_topk(case):
    sq = Seqs(np.cumsum([0] + case["seqlens_q"]), np.cumsum([0] + case["seqlens_k"]))
    qI = np.asarray(case["qI"], np.float64)
    kI = np.asarray(case["kI"], np.float64)
    w = np.asarray(case["w"], np.float64)
    qs = np.asarray(case["q_scale"], np.float64) if "q_scale" in case else None
    ks = np.asarray(case["k_scale"], np.float64) if "k_scale" in case else None
    rows = oracle.indexer_scores(sq, qI, kI, w, q_scale=qs, k_scale=ks)
    assert len(rows) == len(case["scores"])
    for got, want in zip(rows, case["scores"]):
        assert got.shape[0] == len(want)        # exactly pos+1 candidates
        assert np.array_equal(got, np.asarray(want, np.float64))
    for k, want in case["topk"].items():
        got = oracle.topk(rows, int(k))
        assert got.tolist() == want


@pytest.mark.parametrize("case", _golden()["attention"], ids=lambda c: c["name"])
def test_handworked_attention(case):
    sq = Seqs(np.cumsum([0] + case["seqlens_q"]), np.cumsum([0] + case["seqlens_k"]))
    q = np.asarray(case["q"], np.float64)
    kv = np.asarray(case["kv"], np.float64)
    out, lse = oracle.sparse_mla_attn(sq, q, kv, np.asarray(case["indices"]), case["scale"], case["d_v"])
    assert np.allclose(out, np.asarray(case["out"]), rtol=0, atol=1e-14)
    want = np.asarray([[(-np.inf if v is None else v) for v in r] for r in case["lse"]])
    assert np.allclose(lse, want, rtol=0, atol=1e-14) or np.array_equal(lse, want)


# ------------------------------------------------------------------ brute force

def _tiny(seed, variant, seqlens_q=(5, 1, 7), seqlens_k=(9, 6, 7), H_I=3, d_I=5, H=2, d_qk=6, d_v=4):
    wl = dg.custom(seqlens_q=seqlens_q, seqlens_k=seqlens_k, H_I=H_I, d_I=d_I, H=H, d_qk=d_qk,
                   d_v=d_v, k=4)
    return wl, dg.gen_inputs(wl, variant, seed)


@pytest.mark.parametrize("variant", ["normal", "int"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_matches_vectorised(variant, seed):
    wl, x = _tiny(seed, variant)
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    seq_of, pos_of = wl.row_positions()
    dq = oracle.decode(x["qI"]).tolist()
    dk = oracle.decode(x["kI"]).tolist()
    dw = oracle.decode(x["w"]).tolist()
    dqq = oracle.decode(x["q"]).tolist()
    dkv = oracle.decode(x["kv"]).tolist()
    for r in range(wl.T):
        b, pos = int(seq_of[r]), int(pos_of[r])
        k0 = int(wl.cu_seqlens_k[b])
        bs = brute.indexer_row(dq[r], dk[k0:k0 + pos + 1], dw[r])
        vs = oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"], r)
        assert np.allclose(vs, bs, rtol=1e-12, atol=1e-12)
        for k in (1, 3, pos + 1, pos + 4):
            assert oracle.topk_row(vs, k).tolist() == brute.topk_by_rank(bs, k)
        sel = oracle.topk_row(vs, 3)
        bo, bl = brute.attn_row(dqq[r], [dkv[k0 + s] for s in sel if s >= 0], wl.scale, wl.d_v)
        vo, vl = oracle.attn_row(sq, x["q"], x["kv"], sel, wl.scale, wl.d_v, r)
        assert np.allclose(vo, bo, rtol=1e-12, atol=1e-12)
        assert np.allclose(vl, bl, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1])
def test_scaled_indexer_brute_force_and_identities(seed):
    """Scaled inputs: the vectorised oracle equals pure-Python loops over the scaled vectors; unit
    scales give the unscaled scores exactly; a key scale of 2^m multiplies that key's scores by
    2^m exactly, and a query scale a_j > 0 equals weights w_j a_j (positive homogeneity of ReLU)."""
    wl, x = _tiny(seed, "normal")
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    rng = np.random.default_rng(100 + seed)
    qs = np.exp2(rng.uniform(-2, 2, size=(wl.T, wl.H_I)))
    ks = np.exp2(rng.uniform(-2, 2, size=wl.Nk))
    seq_of, pos_of = wl.row_positions()
    dq, dk, dw = oracle.decode(x["qI"]), oracle.decode(x["kI"]), oracle.decode(x["w"])
    for r in range(wl.T):
        b, pos = int(seq_of[r]), int(pos_of[r])
        k0 = int(wl.cu_seqlens_k[b])
        q_sc = (dq[r] * qs[r][:, None]).tolist()
        k_sc = (dk[k0:k0 + pos + 1] * ks[k0:k0 + pos + 1][:, None]).tolist()
        bs = brute.indexer_row(q_sc, k_sc, dw[r].tolist())
        vs = oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"], r, qs, ks)
        assert np.allclose(vs, bs, rtol=1e-12, atol=1e-12)
        base = oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"], r)
        ones = oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"], r, np.ones_like(qs), np.ones_like(ks))
        assert np.array_equal(ones, base)
        p2 = np.exp2(rng.integers(-3, 4, size=wl.Nk)).astype(np.float64)
        scaled = oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"], r, None, p2)
        assert np.array_equal(scaled, base * p2[k0:k0 + pos + 1])
        folded = oracle.indexer_scores_row(sq, x["qI"], x["kI"], dw * qs, r)
        viaq = oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"], r, qs, None)
        assert np.allclose(folded, viaq, rtol=1e-12, atol=1e-12)


def test_brute_topk_integer_ties():
    """Integer scores with many ties: ranking by counting equals the sort-based top-k."""
    rng = np.random.default_rng(5)
    for n in (1, 2, 5, 17, 40):
        s = rng.integers(-2, 3, size=n).astype(np.float64)
        zero = rng.random(n) < 0.3
        s[zero] = np.where(rng.random(int(zero.sum())) < 0.5, 0.0, -0.0)
        for k in (1, 2, 4, n, n + 3):
            assert oracle.topk_row(s, k).tolist() == brute.topk_by_rank(s.tolist(), k)


# ------------------------------------------------------------------ special cases: textbook routines

def _sdpa_dense_causal(q, kv, cu_q, cu_k, scale, d_v):
    """Dense causal MQA attention, bottom-right aligned, via torch SDPA in float64."""
    outs = []
    for b in range(len(cu_q) - 1):
        m, n = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        if m == 0:
            continue
        Q = torch.from_numpy(q[cu_q[b]:cu_q[b + 1]]).permute(1, 0, 2)[None]          # [1,H,m,d]
        C = torch.from_numpy(kv[cu_k[b]:cu_k[b + 1]])[None, None]                     # [1,1,n,d]
        H = Q.shape[1]
        K = C.expand(1, H, n, C.shape[-1])
        V = C[..., :d_v].expand(1, H, n, d_v)
        pos = torch.arange(n - m, n)[:, None]
        mask = torch.arange(n)[None, :] <= pos                                        # [m, n]
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
        outs.append(o[0].permute(1, 0, 2).numpy())
    return np.concatenate(outs)


@pytest.mark.parametrize("seqs", [((512,), (512,)), ((3, 40, 1), (10, 40, 33))])
def test_dense_special_case_equals_sdpa(seqs):
    """k >= every row's candidate count: DSA is dense causal attention over the latent rows."""
    wl = dg.workload("tiny") if seqs[0] == (512,) else dg.custom(seqlens_q=seqs[0], seqlens_k=seqs[1],
                                                                  H_I=4, d_I=32, H=8, d_qk=80, d_v=64)
    x = dg.gen_inputs(wl, "normal", 3)
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    k = wl.max_seqlen_k
    rows = list(range(0, wl.T, max(1, wl.T // 37))) + [wl.T - 1]
    res = oracle.forward_rows(sq, x["qI"], x["kI"], x["w"], x["q"], x["kv"], k, wl.scale, wl.d_v, rows)
    ref = _sdpa_dense_causal(oracle.decode(x["q"]), oracle.decode(x["kv"]), wl.cu_seqlens_q,
                             wl.cu_seqlens_k, wl.scale, wl.d_v)
    assert np.allclose(res["out"], ref[rows], rtol=1e-11, atol=1e-12)
    # lse against torch.logsumexp of the scaled dense logits
    qd, kvd = oracle.decode(x["q"]), oracle.decode(x["kv"])
    for i, r in enumerate(rows):
        b, pos, k0, _ = sq.locate(r)
        z = torch.from_numpy(wl.scale * qd[r] @ kvd[k0:k0 + pos + 1].T)
        assert np.allclose(res["lse"][i], torch.logsumexp(z, dim=1).numpy(), rtol=1e-12, atol=1e-12)


def test_topk_of_tiny_first_rows_is_all_candidates():
    """Rows with pos+1 <= k select every candidate (the tiny workload with k=64, rows < 64)."""
    wl = dg.workload("tiny")
    x = dg.gen_inputs(wl, "normal", 0, parts=("idx",))
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    for r in range(0, 64, 7):
        idx = oracle.topk_row(oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"], r), wl.k)
        assert idx[:r + 1].tolist() == list(range(r + 1)) and np.all(idx[r + 1:] == -1)


def test_identical_scores_select_first_positions():
    assert oracle.topk_row(np.zeros(10), 4).tolist() == [0, 1, 2, 3]
    assert oracle.topk_row(np.full(3, 7.0), 5).tolist() == [0, 1, 2, -1, -1]


# ------------------------------------------------------------------ invariants

def _int_case(seed=0):
    wl = dg.custom(seqlens_q=(6, 9), seqlens_k=(20, 9), H_I=4, d_I=8, H=3, d_qk=10, d_v=6, k=5)
    return wl, dg.gen_inputs(wl, "int", seed)


def test_invariant_w_power_of_two_scaling():
    wl, x = _int_case()
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    for r in range(wl.T):
        a = oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"], r)
        b = oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"] * 8.0, r)
        assert np.array_equal(b, a * 8.0)
        assert oracle.topk_row(a, 5).tolist() == oracle.topk_row(b, 5).tolist()


def test_invariant_head_permutation():
    wl, x = _int_case(1)
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    perm = np.array([2, 0, 3, 1])
    for r in range(wl.T):
        a = oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"], r)
        b = oracle.indexer_scores_row(sq, x["qI"][:, perm], x["kI"], x["w"][:, perm], r)
        assert np.array_equal(a, b)


def test_invariant_prefill_row_equals_decode_at_same_position():
    """Row i of a chunk (m queries over n keys) equals a single-query decode over the first
    pos+1 keys -- this pins the bottom-right alignment."""
    wl, x = _int_case(2)
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    for r in range(wl.cu_seqlens_q[1]):
        _, pos, _, _ = sq.locate(r)
        dec = Seqs([0, 1], [0, pos + 1])
        a = oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"], r)
        b = oracle.indexer_scores_row(dec, x["qI"][r:r + 1], x["kI"][:pos + 1], x["w"][r:r + 1], 0)
        assert np.array_equal(a, b)
        ia, ib = oracle.topk_row(a, 5), oracle.topk_row(b, 5)
        oa, la = oracle.attn_row(sq, x["q"], x["kv"], ia, wl.scale, wl.d_v, r)
        ob, lb = oracle.attn_row(dec, x["q"][r:r + 1], x["kv"][:pos + 1], ib, wl.scale, wl.d_v, 0)
        assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_invariant_attention_shift_and_identical_rows():
    wl, x = _int_case(3)
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    kv = oracle.decode(x["kv"]).copy()
    q = oracle.decode(x["q"])
    sel = np.array([0, 3, 4, -1, -1])
    # identical selected rows -> the value part of that row, lse = logit + ln(count)
    kv2 = kv.copy()
    kv2[[0, 3, 4]] = kv[3]
    o, l = oracle.attn_row(sq, q, kv2, sel, wl.scale, wl.d_v, 0)
    assert np.allclose(o, np.broadcast_to(kv[3, :wl.d_v], o.shape), atol=1e-13)
    assert np.allclose(l, wl.scale * (q[0] @ kv[3]) + math.log(3), atol=1e-12)
    # adding a constant to every logit (via a query component along a constant key column)
    # shifts lse by that constant and leaves out unchanged
    kv3 = kv.copy()
    kv3[:, -1] = 1.0                      # last dim constant (beyond d_v: key-only)
    q3 = q.copy()
    o1, l1 = oracle.attn_row(sq, q3, kv3, sel, wl.scale, wl.d_v, 0)
    q3[0, :, -1] += 2.0
    o2, l2 = oracle.attn_row(sq, q3, kv3, sel, wl.scale, wl.d_v, 0)
    assert np.allclose(o1, o2, atol=1e-13)
    assert np.allclose(l2 - l1, 2.0 * wl.scale, atol=1e-12)


def test_duplicate_indices_count_as_multiset():
    sq = Seqs([0, 1], [0, 2])
    q = np.array([[[1.0, 0.0]]])
    kv = np.array([[1.0, 0.0], [0.0, 0.0]])
    o, l = oracle.attn_row(sq, q, kv, [0, 0, 1], 1.0, 1, 0)
    # logits (1, 1, 0): weights (e, e, 1)/(2e+1)
    assert np.allclose(o[0, 0], 2 * math.e / (2 * math.e + 1), atol=1e-14)
    assert np.allclose(l[0], math.log(2 * math.e + 1), atol=1e-14)


def test_error_bound_covers_float32_evaluations():
    """The score bound of the parity tests with the fp32 path's delta = gamma(d_I) holds for fp32
    evaluations in two different summation orders, and is tight enough that an fp32 evaluation
    leaving out one head's term (the head with the smallest weight) falls outside it."""
    from tests.dsa_check import gamma, score_bound_row
    wl = dg.custom(seqlens_q=(1,), seqlens_k=(300,), H_I=64, d_I=128, k=16)
    x = dg.gen_inputs(wl, "normal", 4, parts=("idx",))
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    exact = oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"], 0)
    eps = score_bound_row(sq, x["qI"], x["kI"], x["w"], 0, gamma(wl.d_I))
    q32 = x["qI"][0].astype(np.float32)
    k32 = x["kI"].astype(np.float32)
    w32 = x["w"][0].astype(np.float32)
    a = (w32[:, None] * np.maximum(q32 @ k32.T, np.float32(0))).sum(axis=0, dtype=np.float32)
    b = np.zeros(300, np.float32)
    for j in range(63, -1, -1):
        d = np.zeros(300, np.float32)
        for dd in range(127, -1, -1):
            d = d + q32[j, dd] * k32[:, dd]
        b = b + w32[j] * np.maximum(d, np.float32(0))
    assert np.all(np.abs(a - exact) <= eps) and np.all(np.abs(b - exact) <= eps)
    assert np.all(eps > 0)
    j = int(np.argmin(np.abs(w32)))
    keep = np.arange(64) != j
    c = (w32[keep, None] * np.maximum(q32[keep] @ k32.T, np.float32(0))).sum(axis=0, dtype=np.float32)
    assert np.any(np.abs(c - exact) > eps)


# ------------------------------------------------------------------ indexer-alignment target

@pytest.mark.parametrize("case", _golden()["alignment"], ids=lambda c: c["name"])
def test_handworked_alignment(case):
    sq = Seqs(np.cumsum([0] + case["seqlens_q"]), np.cumsum([0] + case["seqlens_k"]))
    q = np.asarray(case["q"], np.float64)
    kv = np.asarray(case["kv"], np.float64)
    for r in range(len(case["indices"])):
        tgt, kl = oracle.alignment_row(sq, q, kv, case["indices"][r], case["scale"], case["scores"][r], r)
        assert np.allclose(tgt, case["target"][r], rtol=0, atol=1e-15)
        assert abs(kl - case["kl"][r]) <= 1e-15


@pytest.mark.parametrize("variant", ["normal", "int"])
@pytest.mark.parametrize("seed", [0, 1])
def test_alignment_brute_force(variant, seed):
    wl, x = _tiny(seed, variant)
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    seq_of, pos_of = wl.row_positions()
    dqq, dkv = oracle.decode(x["q"]).tolist(), oracle.decode(x["kv"]).tolist()
    for r in range(wl.T):
        b, pos = int(seq_of[r]), int(pos_of[r])
        k0 = int(wl.cu_seqlens_k[b])
        sc = oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"], r)
        sel = oracle.topk_row(sc, 3)
        tgt, kl = oracle.alignment_row(sq, x["q"], x["kv"], sel, wl.scale, sc, r)
        valid = [s for s in sel if s >= 0]
        bp, bkl = brute.alignment_row(dqq[r], [dkv[k0 + s] for s in valid], wl.scale, [sc[s] for s in valid])
        assert np.allclose(tgt[:len(valid)], bp, rtol=1e-12, atol=1e-15)
        assert np.all(tgt[len(valid):] == 0)
        assert abs(kl - bkl) <= 1e-12 * max(1.0, abs(bkl))


def test_alignment_single_head_is_relative_entropy():
    """With one head the target is that head's softmax and the loss is the relative entropy
    between two softmaxes: checked with scipy's softmax and rel_entr (independent routines)."""
    from scipy.special import rel_entr, softmax
    rng = np.random.default_rng(11)
    n = 7
    sq = Seqs([0, 1], [0, n])
    q = rng.standard_normal((1, 1, 5))
    kv = rng.standard_normal((n, 5))
    scores = rng.standard_normal(n) * 2
    idx = [6, 2, 0, 5]
    tgt, kl = oracle.alignment_row(sq, q, kv, idx, 0.7, scores, 0)
    p = softmax(0.7 * (kv[idx] @ q[0, 0]))
    qi = softmax(scores[idx])
    assert np.allclose(tgt, p, rtol=1e-13, atol=0)
    assert abs(kl - rel_entr(p, qi).sum()) <= 1e-13


def test_alignment_invariants():
    """KL >= 0; zero queries give the uniform target; an indexer whose softmax equals the target
    gives KL = 0; adding a constant to every score changes nothing; no valid entry gives 0."""
    wl, x = _tiny(3, "normal")
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    for r in range(wl.T):
        sc = oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"], r)
        sel = oracle.topk_row(sc, 4)
        tgt, kl = oracle.alignment_row(sq, x["q"], x["kv"], sel, wl.scale, sc, r)
        assert kl >= -1e-15
        _, kl2 = oracle.alignment_row(sq, x["q"], x["kv"], sel, wl.scale, sc + 5.25, r)
        assert abs(kl2 - kl) <= 1e-12
        v = np.asarray(sel) >= 0
        matched = np.full(sc.shape[0], -np.inf)
        matched[np.asarray(sel)[v]] = np.log(tgt[v])
        _, kl0 = oracle.alignment_row(sq, x["q"], x["kv"], sel, wl.scale, matched, r)
        assert abs(kl0) <= 1e-12
        tz, _ = oracle.alignment_row(sq, np.zeros((wl.T, wl.H, wl.d_qk)), x["kv"], sel, wl.scale, sc, r)
        assert np.allclose(tz[v], 1.0 / v.sum(), rtol=0, atol=1e-15)
    t_e, k_e = oracle.alignment_row(sq, x["q"], x["kv"], [-1, -1], wl.scale, sc, 0)
    assert k_e == 0.0 and np.all(t_e == 0)
