#!/usr/bin/env python3
"""Benchmark of the DSA forward hot path (lightning indexer -> top-k -> sparse MLA attention) on
one MI355X.

A step is one fused forward (dsa_forward: indexer, top-k, attention) over one batch of synthetic
inputs already resident in HBM. The headline workload is the 128K-context prefill chunk: 4096
query rows at positions 126976..131071 against 131072 causal keys, H_I = 64, d_I = 128 (FP8
e4m3), k = 2048, 128 heads with 576/512 latent dims (bf16). value = query tokens per second.

Besides the fused step, each kernel is timed alone with HIP events on the stream it runs on, and
the dominant kernel's achieved rate is reported against the MI355X peak (roofline). The CPU
oracle is timed on a bounded sample of the same workload's rows (cpu_baseline).

Progress goes to stderr; the result is one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0

TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "indexer_fp8_chunk128k_hbm_traffic.md")


def measured_traffic():
    """HBM bytes per launch of the indexer prefill kernel from the committed counter summary, or
    None when the kernel source has changed since those counters were taken."""
    import hashlib
    try:
        line = [l for l in open(TRAFFIC_RECORD) if l.startswith("record: ")][-1]
        rec = json.loads(line[len("record: "):])
        src = open(os.path.join(ROOT, rec["kernel_source"]), "rb").read()
        if hashlib.sha256(src).hexdigest()[:16] != rec["source_sha256_16"]:
            return None
        return float(rec["bytes_per_launch"])
    except (OSError, IndexError, KeyError, ValueError):
        return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def causal_pairs(wl):
    """Number of (query row, candidate key) pairs and of selected keys."""
    pairs = 0
    sel = 0
    for m, n in zip(wl.seqlens_q, wl.seqlens_k):
        pos = np.arange(n - m, n, dtype=np.int64)
        pairs += int((pos + 1).sum())
        sel += int(np.minimum(pos + 1, wl.k).sum())
    return pairs, sel


def algorithmic(wl):
    pairs, sel = causal_pairs(wl)
    T = wl.T
    idx_flop = 2.0 * wl.H_I * wl.d_I * pairs
    attn_flop = 2.0 * wl.H * (wl.d_qk + wl.d_v) * sel
    topk_bytes = 4.0 * pairs + 4.0 * wl.k * T
    # decode-style HBM bytes: indexer keys + gathered latent rows + per-query vectors
    vec_bytes = T * (wl.H_I * wl.d_I * 1 + wl.H_I * 4 + wl.H * wl.d_qk * 2 + wl.H * wl.d_v * 2 + wl.H * 4)
    dec_bytes = float(sum(wl.seqlens_k)) * wl.d_I + sel * wl.d_qk * 2.0 + vec_bytes
    return dict(pairs=pairs, selected=sel, indexer_flop=idx_flop, attn_flop=attn_flop,
                topk_bytes=topk_bytes, decode_bytes=dec_bytes)


def to_dev(torch, a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint8:
        t = t.view(torch.float8_e4m3fn)
    elif a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.cuda()


def time_loop(torch, fn, steps, warmup):
    """Average milliseconds per call, HIP events on the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def setup(torch, dsa, dg, name, seed=0):
    wl = dg.workload(name)
    t0 = time.time()
    x = dg.gen_inputs(wl, "normal", seed=seed)
    T = {k: to_dev(torch, v) for k, v in x.items() if k not in ("cu_seqlens_q", "cu_seqlens_k")}
    seqs = dsa.Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    torch.cuda.synchronize()
    log(f"[bench] {name}: inputs generated and uploaded in {time.time() - t0:.1f}s")
    return wl, x, T, seqs


def measure(torch, dsa, wl, T, seqs, steps, warmup, scales=None):
    """Fused step time and per-kernel times for one workload (and, with `scales`, the indexer on
    scaled inputs)."""
    fwd = dsa.Forward(seqs, T["qI"], T["kI"], T["w"], T["q"], T["kv"], wl.k, wl.scale, wl.d_v)
    scores = torch.empty((wl.T, dsa.scores_ld(wl.max_seqlen_k)), dtype=torch.float32, device="cuda")
    idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
    out = torch.empty((wl.T, wl.H, wl.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((wl.T, wl.H), dtype=torch.float32, device="cuda")
    iws_n = dsa.indexer_workspace_size(seqs, wl.H_I, wl.d_I, dsa._dtype_code(T["qI"]))
    iws = torch.empty(max(iws_n, 1), dtype=torch.uint8, device="cuda")
    # the stages alone (each on its own, inputs produced by the previous stage)
    dsa.indexer_scores(seqs, T["qI"], T["kI"], T["w"], scores=scores, ws=iws)
    dsa.topk(seqs, scores, wl.k, indices=idx)
    t_idx = time_loop(torch, lambda: dsa.indexer_scores(seqs, T["qI"], T["kI"], T["w"], scores=scores, ws=iws),
                      steps, warmup)
    t_topk = time_loop(torch, lambda: dsa.topk(seqs, scores, wl.k, indices=idx), steps, warmup)
    aws_n = dsa.attn_workspace_size(seqs, wl.H, wl.d_qk, wl.d_v, wl.k, dsa._dtype_code(T["q"]))
    aws = torch.empty(max(aws_n, 1), dtype=torch.uint8, device="cuda")
    t_attn = time_loop(torch, lambda: dsa.sparse_mla_attn(seqs, T["q"], T["kv"], idx, wl.scale, wl.d_v,
                                                          out=out, lse=lse, ws=aws), steps, warmup)
    t_fwd = time_loop(torch, fwd, steps, warmup)
    res = dict(fused_ms=t_fwd, indexer_ms=t_idx, topk_ms=t_topk, attn_ms=t_attn)
    if scales is not None and wl.attn_dtype == "bf16":   # the indexer-alignment target of the same rows
        kl = torch.empty((wl.T,), dtype=torch.float32, device="cuda")
        tgt = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")
        res["alignment_ms"] = time_loop(
            torch, lambda: dsa.indexer_alignment(seqs, T["q"], T["kv"], idx, wl.scale, lse, scores,
                                                 kl=kl, target=tgt), steps, warmup)
    if scales is not None:
        qs, ks = to_dev(torch, scales["q_scale"]), to_dev(torch, scales["k_scale"])
        sws_n = dsa.indexer_scaled_workspace_size(seqs, wl.H_I, wl.d_I, dsa._dtype_code(T["qI"]))
        sws = torch.empty(max(sws_n, 1), dtype=torch.uint8, device="cuda")
        res["indexer_scaled_ms"] = time_loop(
            torch, lambda: dsa.indexer_scores_scaled(seqs, T["qI"], qs, T["kI"], ks, T["w"], scores=scores,
                                                     ws=sws), steps, warmup)
    return res


def cpu_baseline(wl, x, seconds):
    """The oracle (untuned) on a bounded sample of the workload's rows, all three steps."""
    import oracle
    from oracle.dsa import Seqs
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    sq = Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    rows = np.linspace(0, wl.T - 1, num=min(wl.T, 512)).astype(int)
    rows = rows[np.random.default_rng(0).permutation(len(rows))]
    done = 0
    t0 = time.time()
    for r in rows:
        oracle.forward_rows(sq, x["qI"], x["kI"], x["w"], x["q"], x["kv"], wl.k, wl.scale, wl.d_v, [r])
        done += 1
        if time.time() - t0 >= seconds:
            break
    el = time.time() - t0
    return dict(value=done / el, unit="tokens/s" if wl.max_seqlen_q > 1 else "queries/s", cores=int(threads),
                kind="oracle", sample=f"{done} query rows of {wl.name} (all three steps, float64), {el:.1f}s")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="chunk128k")
    ap.add_argument("--secondary", default="decode32k,short2k",
                    help="comma-separated extra workloads reported under 'secondary' ('' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain device copy of 1 GiB (for scaling HBM counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU sharding of "
              f"this path is a design note, not an implemented mode.", file=sys.stderr)
        sys.exit(2)

    import torch
    import dsa_datagen as dg
    import sparse_attention_head_amd as dsa

    torch.cuda.set_device(0)
    wl, x, T, seqs = setup(torch, dsa, dg, args.workload)
    alg = algorithmic(wl)
    log(f"[bench] timing {args.workload}: warmup {args.warmup}, steps {args.steps}")
    tm = measure(torch, dsa, wl, T, seqs, args.steps, args.warmup,
                 scales=dg.gen_scales(wl, "normal") if wl.idx_dtype == "fp8" else None)
    log(f"[bench] {args.workload}: {tm}")

    prefill = wl.max_seqlen_q > 1
    value = wl.T / (tm["fused_ms"] / 1e3)
    idx_tflops = alg["indexer_flop"] / (tm["indexer_ms"] / 1e3) / 1e12
    attn_tflops = alg["attn_flop"] / (tm["attn_ms"] / 1e3) / 1e12
    topk_gbs = alg["topk_bytes"] / (tm["topk_ms"] / 1e3) / 1e9
    stages = dict(
        indexer=dict(ms=tm["indexer_ms"], tflops=idx_tflops, frac_fp8=idx_tflops / PEAK_FP8_TFLOPS,
                     flop=alg["indexer_flop"]),
        topk=dict(ms=tm["topk_ms"], gbs=topk_gbs, frac_hbm=topk_gbs / PEAK_HBM_GBS, bytes=alg["topk_bytes"]),
        attention=dict(ms=tm["attn_ms"], tflops=attn_tflops, frac_bf16=attn_tflops / PEAK_BF16_TFLOPS,
                       flop=alg["attn_flop"]),
    )
    if "alignment_ms" in tm:   # logits of every selected entry again: 2 H d_qk flop each
        af = 2.0 * wl.H * wl.d_qk * alg["selected"]
        at = af / (tm["alignment_ms"] / 1e3) / 1e12
        stages["alignment"] = dict(ms=tm["alignment_ms"], tflops=at, frac_bf16=at / PEAK_BF16_TFLOPS, flop=af)
    if "indexer_scaled_ms" in tm:   # scaled FP8 inputs (per row and head, per key)
        st = alg["indexer_flop"] / (tm["indexer_scaled_ms"] / 1e3) / 1e12
        stages["indexer_scaled"] = dict(ms=tm["indexer_scaled_ms"], tflops=st, frac_fp8=st / PEAK_FP8_TFLOPS)
    if prefill:
        roof = dict(kernel="indexer_fp8", bound="mfma", achieved=idx_tflops, peak=PEAK_FP8_TFLOPS,
                    unit="TFLOP/s", frac=idx_tflops / PEAK_FP8_TFLOPS,
                    traffic=measured_traffic() if wl.name == "chunk128k" else None)
    else:
        gbs = alg["decode_bytes"] / (tm["fused_ms"] / 1e3) / 1e9
        roof = dict(kernel="fused_decode", bound="hbm", achieved=gbs, peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=gbs / PEAK_HBM_GBS, traffic=None)

    secondary = {}
    for name in [s for s in args.secondary.split(",") if s and s != args.workload]:
        del T
        torch.cuda.empty_cache()
        wl2, x2, T, seqs2 = setup(torch, dsa, dg, name)
        tm2 = measure(torch, dsa, wl2, T, seqs2, max(3, args.steps // 2), 1)
        a2 = algorithmic(wl2)
        q_s = wl2.T / (tm2["fused_ms"] / 1e3)
        if wl2.max_seqlen_q == 1:   # decode: HBM-bound as a whole
            secondary[name] = dict(
                fused_ms=tm2["fused_ms"], per_s=q_s, unit="queries/s",
                hbm_gbs=a2["decode_bytes"] / (tm2["fused_ms"] / 1e3) / 1e9,
                hbm_frac=a2["decode_bytes"] / (tm2["fused_ms"] / 1e3) / 1e9 / PEAK_HBM_GBS,
                indexer_ms=tm2["indexer_ms"], topk_ms=tm2["topk_ms"], attn_ms=tm2["attn_ms"])
        else:   # prefill: stages alone, and the attention's share of the BF16 peak
            secondary[name] = dict(
                fused_ms=tm2["fused_ms"], per_s=q_s, unit="tokens/s",
                indexer_ms=tm2["indexer_ms"], topk_ms=tm2["topk_ms"], attn_ms=tm2["attn_ms"],
                attn_frac_bf16=a2["attn_flop"] / (tm2["attn_ms"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                short_context=bool(wl2.max_seqlen_k <= wl2.k))
        log(f"[bench] {name}: {secondary[name]}")
        del x2

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle for ~{args.cpu_seconds:.0f}s")
        cpu = cpu_baseline(wl, x, args.cpu_seconds)

    res = dict(
        metric="DSA prefill tokens/s @128K ctx; decode queries/s; % of MFMA/HBM roofline",
        value=value, unit="tokens/s" if prefill else "queries/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=tm["fused_ms"], higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="fp8-e4m3 indexer, bf16 attention (fp32 accumulate)", data="synthetic",
        config=dict(workload=wl.name, query_rows=wl.T, keys_per_seq=wl.max_seqlen_k, sequences=wl.num_seqs,
                    H_I=wl.H_I, d_I=wl.d_I, k=wl.k, H=wl.H, d_qk=wl.d_qk, d_v=wl.d_v),
        roofline=roof, cpu_baseline=cpu, stages=stages, secondary=secondary,
    )
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
