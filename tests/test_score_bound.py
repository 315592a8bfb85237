"""The indexer-score parity bound (tests/dsa_check.py) against a NumPy model of the FP8 prefill
kernel's arithmetic (tests/kernel_model.py), both ways:

  * the bound covers the model's scores, with the matrix instruction's error at its measured
    worst rate (N(0,1)-drawn codes and codes over the whole e4m3 range);
  * it is tight enough that leaving out one head's term (any head whose weight is not close to
    zero), or either of the two leading FP8 pieces of the linear term, puts some score of a
    workload-shaped row outside it.

The two trailing pieces of the linear term carry 2^-8 .. 2^-16 of u and fall below what the
matrix instruction's own rounding allows on such data; they are pinned bit for bit instead, by
inputs built so that every partial sum is exact and all four pieces are nonzero
(dsa_datagen.gen_linear_split: checked here on the model, on the GPU by
test_gpu_parity.test_indexer_linear_split_exact).
"""
import numpy as np
import pytest

import dsa_datagen as dg
import oracle
from oracle.dsa import Seqs
from tests import kernel_model as km
from tests.dsa_check import (DELTA_FP8_FULL, DELTA_FP8_NORMAL, MFMA_RATE_FULL, MFMA_RATE_NORMAL,
                             score_bound_row)


def _row(variant, seed, n=3000):
    wl = dg.custom(name="bound", seqlens_q=(1,), seqlens_k=(n,), H_I=64, d_I=128, k=2048, idx_dtype="fp8",
                   wid=60)
    x = dg.gen_inputs(wl, variant, seed, parts=("idx",))
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    return sq, x, oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"], 0)


@pytest.mark.parametrize("variant,delta,rate", [("normal", DELTA_FP8_NORMAL, MFMA_RATE_NORMAL),
                                                ("e4m3", DELTA_FP8_FULL, MFMA_RATE_FULL)])
@pytest.mark.parametrize("seed", [0, 1])
def test_bound_covers_kernel_model(variant, delta, rate, seed):
    sq, x, exact = _row(variant, seed)
    eps = score_bound_row(sq, x["qI"], x["kI"], x["w"], 0, delta)
    rng = np.random.default_rng(seed)
    got = km.prefill_scores(x["qI"][0], x["kI"], x["w"][0], mfma_rel=rate, rng=rng).astype(np.float64)
    ratio = np.abs(got - exact) / eps
    assert np.all(ratio <= 1.0), f"worst |err| / eps = {ratio.max()}"
    # and without the matrix-instruction error the model is far inside
    clean = km.prefill_scores(x["qI"][0], x["kI"], x["w"][0]).astype(np.float64)
    assert np.max(np.abs(clean - exact) / eps) < 0.25


@pytest.mark.parametrize("seed", [0, 1])
def test_bound_detects_a_dropped_head(seed):
    """Every head whose weight is at least 1/16 of the row's median |w| (all but the odd head
    whose weight is close to zero, and whose term is then below the rounding of the others) is
    missed by some score if left out."""
    sq, x, exact = _row("normal", seed)
    eps = score_bound_row(sq, x["qI"], x["kI"], x["w"], 0, DELTA_FP8_NORMAL)
    w = np.abs(x["w"][0])
    heads = [j for j in range(64) if w[j] >= np.median(w) / 16]
    assert len(heads) >= 60
    missed = []
    for j in heads:
        got = km.prefill_scores(x["qI"][0], x["kI"], x["w"][0], drop_head=j).astype(np.float64)
        if not np.any(np.abs(got - exact) > eps):
            missed.append(j)
    assert not missed, f"dropping head(s) {missed} stays inside the bound"


@pytest.mark.parametrize("piece", [0, 1])
@pytest.mark.parametrize("seed", [0, 1])
def test_bound_detects_a_dropped_leading_piece(seed, piece):
    sq, x, exact = _row("normal", seed)
    eps = score_bound_row(sq, x["qI"], x["kI"], x["w"], 0, DELTA_FP8_NORMAL)
    got = km.prefill_scores(x["qI"][0], x["kI"], x["w"][0], drop_piece=piece).astype(np.float64)
    assert np.any(np.abs(got - exact) > eps)


def test_linear_split_inputs_are_exact_and_use_four_pieces():
    """The exact-split inputs: the model reproduces the oracle bit for bit (so the GPU must too),
    every row's linear term has four nonzero pieces that add up to u exactly, and leaving out any
    one piece changes some score."""
    wl = dg.custom(name="split", seqlens_q=(24,), seqlens_k=(300,), H_I=64, d_I=128, k=64, idx_dtype="fp8",
                   wid=61)
    x = dg.gen_linear_split(wl, seed=0)
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    for r in range(wl.T):
        _, pos, k0, _ = sq.locate(r)
        keys = x["kI"][k0:k0 + pos + 1]
        exact = oracle.indexer_scores_row(sq, x["qI"], x["kI"], x["w"], r)
        pieces, e = km.linear_pieces(x["qI"][r], x["w"][r])
        u = oracle.decode(x["w"][r]) @ oracle.decode(x["qI"][r])
        assert np.all(np.any(pieces != 0, axis=1)), f"row {r}: a piece is zero everywhere"
        recon = sum(pieces[p].astype(np.float64) * 16.0 ** -p for p in range(4)) * 2.0 ** e
        assert np.array_equal(recon, u), f"row {r}: the four pieces do not add up to u"
        got = km.prefill_scores(x["qI"][r], keys, x["w"][r]).astype(np.float64)
        assert np.array_equal(got, exact), f"row {r}: model differs from the oracle"
        for p in range(4):
            dropped = km.prefill_scores(x["qI"][r], keys, x["w"][r], drop_piece=p).astype(np.float64)
            assert not np.array_equal(dropped, exact), f"row {r}: piece {p} makes no difference"
