#!/usr/bin/env python3
"""Benchmark of the DSA forward hot path (lightning indexer -> top-k -> sparse MLA attention) on
one MI355X.

A step is one fused forward (dsa_forward: indexer, top-k, attention) over one batch of synthetic
inputs already resident in HBM. The headline workload is the 128K-context prefill chunk: 4096
query rows at positions 126976..131071 against 131072 causal keys, H_I = 64, d_I = 128 (FP8
e4m3), k = 2048, 128 heads with 576/512 latent dims (bf16). value = query tokens per second.

Timing protocol: before every timed step a 1 GiB buffer is read (the inputs are then in
neither L2 nor the 256 MB last-level cache), and the step runs between its own pair of HIP events on
the stream the library launches on; value and ms_per_step come from the median step, the minimum
and mean are reported beside it, and so is one back-to-back loop with warm caches. Besides the fused
step, each stage is timed alone the same way, and the dominant kernel's achieved rate is reported
against the MI355X peak (roofline). The other workloads -- prefill8k, decode32k (64 x 32K),
ragged (128 decode rows of 4K..128K keys) and short2k -- are timed the same way under `secondary`.
The CPU oracle is timed on a bounded sample of the headline workload's rows (cpu_baseline). A
plain device copy of 256 MiB and of 1 GiB, timed the same way, goes under timing.plain_copy (bytes
read plus written per second): what streaming reaches on this GPU, beside the datasheet peak the
HBM-bound stages' fractions are quoted on.

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
    # latent rows the attention and the alignment target gather: one d_qk-dim bf16 row per
    # selected entry (their other roofline besides the matrix core)
    gather_bytes = sel * wl.d_qk * 2.0
    return dict(pairs=pairs, selected=sel, indexer_flop=idx_flop, attn_flop=attn_flop,
                topk_bytes=topk_bytes, decode_bytes=dec_bytes, gather_bytes=gather_bytes)


def to_dev(torch, a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint8:
        t = t.view(torch.float8_e4m3fn)
    elif a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.cuda()


FLUSH_BYTES = 1 << 30   # read between timed reps: 4x the 256 MB last-level cache


class Timer:
    """Cold-cache timing: before every timed rep a 1 GiB buffer is read (so L2 and the last-level
    cache hold none of the inputs, only clean lines: a written buffer would leave dirty lines whose
    write-back the next kernel pays for), then the rep runs between its own pair of HIP events on
    the current stream (the stream the library launches on). Reports the median, min and mean of
    the reps; `warm` also times one back-to-back loop (caches warm) for comparison."""

    def __init__(self, torch):
        self.torch = torch
        self.scratch = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
        self.sink = torch.empty((), dtype=torch.int32, device="cuda")

    def flush(self):
        torch = self.torch
        torch.amax(self.scratch, dim=0, out=self.sink)

    def __call__(self, fn, reps, warmup, warm=False):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:
            self.flush()
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        t = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
        res = dict(median=float(np.median(t)), min=float(t.min()), mean=float(t.mean()), reps=reps)
        if warm:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            res["warm_mean"] = e0.elapsed_time(e1) / reps
        return res


def copy_calibration(torch, timer, reps=7):
    """What plain streaming reaches on this GPU (the context for the HBM-bound stages' fractions):
    a device-to-device copy of 256 MiB and of 1 GiB, each rep after the usual cache flush, timed
    with its own event pair; median rate of the bytes read plus written, GB/s, per size."""
    out = {}
    for nbytes in (256 << 20, 1 << 30):
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        t = timer(lambda: dst.copy_(src), reps, 1)
        out[f"{nbytes >> 20}MiB"] = {"ms": t["median"], "gbs": 2 * nbytes / (t["median"] / 1e3) / 1e9}
        del src, dst
    return out


def setup(torch, dsa, dg, name, seed=0):
    wl = dg.workload(name)
    t0 = time.time()
    x = dg.gen_inputs(wl, "normal", seed=seed)
    T = {k: to_dev(torch, v) for k, v in x.items() if k not in ("cu_seqlens_q", "cu_seqlens_k")}
    seqs = dsa.Seqs(wl.cu_seqlens_q, wl.cu_seqlens_k)
    torch.cuda.synchronize()
    log(f"[bench] {name}: inputs generated and uploaded in {time.time() - t0:.1f}s")
    return wl, x, T, seqs


def measure(torch, dsa, timer, wl, T, seqs, steps, warmup, scales=None, fused_only=False):
    """Fused step and per-stage times for one workload (and, with `scales`, the indexer on scaled
    inputs and the indexer-alignment target); each a dict of median / min / mean ms."""
    fwd = dsa.Forward(seqs, T["qI"], T["kI"], T["w"], T["q"], T["kv"], wl.k, wl.scale, wl.d_v)
    res = dict(fused=timer(fwd, steps, warmup, warm=True))
    if fused_only:
        return res
    scores = torch.empty((wl.T, dsa.scores_ld(wl.max_seqlen_k)), dtype=torch.float32, device="cuda")
    idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
    out = torch.empty((wl.T, wl.H, wl.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((wl.T, wl.H), dtype=torch.float32, device="cuda")
    iws_n = dsa.indexer_workspace_size(seqs, wl.H_I, wl.d_I, dsa._dtype_code(T["qI"]))
    iws = torch.empty(max(iws_n, 1), dtype=torch.uint8, device="cuda")
    # the stages alone (each on its own, inputs produced by the previous stage)
    dsa.indexer_scores(seqs, T["qI"], T["kI"], T["w"], scores=scores, ws=iws)
    dsa.topk(seqs, scores, wl.k, indices=idx)
    res["indexer"] = timer(lambda: dsa.indexer_scores(seqs, T["qI"], T["kI"], T["w"], scores=scores, ws=iws),
                           steps, warmup)
    res["topk"] = timer(lambda: dsa.topk(seqs, scores, wl.k, indices=idx), steps, warmup)
    # the fused indexer -> top-k call (fused for decode batches, the two steps otherwise)
    itws_n = dsa.indexer_topk_workspace_size(seqs, wl.H_I, wl.d_I, dsa._dtype_code(T["qI"]), wl.k)
    itws = torch.empty(max(itws_n, 1), dtype=torch.uint8, device="cuda")
    res["indexer_topk"] = timer(lambda: dsa.indexer_topk(seqs, T["qI"], T["kI"], T["w"], wl.k, scores=scores,
                                                         indices=idx, ws=itws), steps, warmup)
    aws_n = dsa.attn_workspace_size(seqs, wl.H, wl.d_qk, wl.d_v, wl.k, dsa._dtype_code(T["q"]))
    aws = torch.empty(max(aws_n, 1), dtype=torch.uint8, device="cuda")
    res["attention"] = timer(lambda: dsa.sparse_mla_attn(seqs, T["q"], T["kv"], idx, wl.scale, wl.d_v,
                                                         out=out, lse=lse, ws=aws), steps, warmup)
    if scales is not None and wl.attn_dtype == "bf16":   # the indexer-alignment target of the same rows
        kl = torch.empty((wl.T,), dtype=torch.float32, device="cuda")
        tgt = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")
        res["alignment"] = timer(
            lambda: dsa.indexer_alignment(seqs, T["q"], T["kv"], idx, wl.scale, lse, scores, kl=kl, target=tgt),
            steps, warmup)
    if scales is not None:
        qs, ks = to_dev(torch, scales["q_scale"]), to_dev(torch, scales["k_scale"])
        sws_n = dsa.indexer_scaled_workspace_size(seqs, wl.H_I, wl.d_I, dsa._dtype_code(T["qI"]))
        sws = torch.empty(max(sws_n, 1), dtype=torch.uint8, device="cuda")
        res["indexer_scaled"] = timer(
            lambda: dsa.indexer_scores_scaled(seqs, T["qI"], qs, T["kI"], ks, T["w"], scores=scores, ws=sws),
            steps, warmup)
    return res


def gather_rate(alg, t):
    """The gathered latent rows per second of a stage, against the HBM peak."""
    gbs = alg["gather_bytes"] / (t["median"] / 1e3) / 1e9
    return {"gather_gbs": gbs, "gather_frac_hbm": gbs / PEAK_HBM_GBS}


def stage_report(wl, tm):
    """Per-stage rates against the MI355X peaks (median times; min-time rates alongside)."""
    alg = algorithmic(wl)

    def rate(work, t, peak, unit, key):
        r = work / (t["median"] / 1e3) / (1e12 if unit == "tflops" else 1e9)
        best = work / (t["min"] / 1e3) / (1e12 if unit == "tflops" else 1e9)
        return {"ms": t["median"], "ms_min": t["min"], unit: r, key: r / peak, key + "_at_min": best / peak}

    out = {}
    if "indexer" in tm:
        out["indexer"] = rate(alg["indexer_flop"], tm["indexer"], PEAK_FP8_TFLOPS, "tflops", "frac_fp8")
        out["topk"] = rate(alg["topk_bytes"], tm["topk"], PEAK_HBM_GBS, "gbs", "frac_hbm")
        out["attention"] = rate(alg["attn_flop"], tm["attention"], PEAK_BF16_TFLOPS, "tflops", "frac_bf16")
        out["attention"].update(gather_rate(alg, tm["attention"]))
    if "indexer_topk" in tm:   # one call for both steps; against the two calls' medians
        sep = tm["indexer"]["median"] + tm["topk"]["median"]
        out["indexer_topk"] = {"ms": tm["indexer_topk"]["median"], "ms_min": tm["indexer_topk"]["min"],
                               "fused": bool(wl.max_seqlen_q == 1 and wl.k <= 2048 and wl.max_seqlen_k <= 131072),
                               "separate_ms": sep, "speedup_vs_separate": sep / tm["indexer_topk"]["median"]}
    if "alignment" in tm:   # logits of every selected entry again: 2 H d_qk flop each
        out["alignment"] = rate(2.0 * wl.H * wl.d_qk * alg["selected"], tm["alignment"], PEAK_BF16_TFLOPS,
                                "tflops", "frac_bf16")
        out["alignment"].update(gather_rate(alg, tm["alignment"]))
    if "indexer_scaled" in tm:
        out["indexer_scaled"] = rate(alg["indexer_flop"], tm["indexer_scaled"], PEAK_FP8_TFLOPS, "tflops",
                                     "frac_fp8")
    return out


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
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="chunk128k")
    ap.add_argument("--secondary", default="prefill8k,decode32k,ragged,short2k",
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
    timer = Timer(torch)
    wl, x, T, seqs = setup(torch, dsa, dg, args.workload)
    alg = algorithmic(wl)
    log(f"[bench] timing {args.workload}: warmup {args.warmup}, steps {args.steps} (cold cache, one event "
        f"pair per step)")
    torch.cuda.synchronize()
    t_wall = time.time()
    tm = measure(torch, dsa, timer, wl, T, seqs, args.steps, args.warmup,
                 scales=dg.gen_scales(wl, "normal") if wl.idx_dtype == "fp8" else None)
    torch.cuda.synchronize()
    log(f"[bench] {args.workload}: {json.dumps(tm)} ({time.time() - t_wall:.1f}s)")

    prefill = wl.max_seqlen_q > 1
    fused = tm["fused"]
    value = wl.T / (fused["median"] / 1e3)
    stages = stage_report(wl, tm)
    if prefill:
        st = stages["indexer"]
        roof = dict(kernel="indexer_fp8 (prep + prefill kernel)", bound="mfma", achieved=st["tflops"],
                    peak=PEAK_FP8_TFLOPS, unit="TFLOP/s", frac=st["frac_fp8"],
                    traffic=measured_traffic() if wl.name == "chunk128k" else None)
    else:
        gbs = alg["decode_bytes"] / (fused["median"] / 1e3) / 1e9
        roof = dict(kernel="fused_decode", bound="hbm", achieved=gbs, peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=gbs / PEAK_HBM_GBS, traffic=None)

    secondary = {}
    for name in [s for s in args.secondary.split(",") if s and s != args.workload]:
        del T
        torch.cuda.empty_cache()
        wl2, x2, T, seqs2 = setup(torch, dsa, dg, name)
        del x2
        tm2 = measure(torch, dsa, timer, wl2, T, seqs2, args.steps, max(1, args.warmup // 2))
        a2 = algorithmic(wl2)
        f2 = tm2["fused"]
        rec = dict(fused_ms=f2["median"], fused_ms_min=f2["min"], fused_ms_warm=f2["warm_mean"],
                   per_s=wl2.T / (f2["median"] / 1e3), stages=stage_report(wl2, tm2))
        if wl2.max_seqlen_q == 1:   # decode: HBM-bound as a whole
            gbs = a2["decode_bytes"] / (f2["median"] / 1e3) / 1e9
            rec.update(unit="queries/s", hbm_gbs=gbs, hbm_frac=gbs / PEAK_HBM_GBS,
                       hbm_frac_at_min=a2["decode_bytes"] / (f2["min"] / 1e3) / 1e9 / PEAK_HBM_GBS,
                       decode_bytes=a2["decode_bytes"])
        else:
            rec.update(unit="tokens/s", short_context=bool(wl2.max_seqlen_k <= wl2.k))
        secondary[name] = rec
        log(f"[bench] {name}: {json.dumps(rec)}")

    copy_cal = copy_calibration(torch, timer)
    log(f"[bench] plain copy: {json.dumps(copy_cal)}")

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
        warmup=args.warmup, ms_per_step=fused["median"], higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="fp8-e4m3 indexer, bf16 attention (fp32 accumulate)", data="synthetic",
        config=dict(workload=wl.name, query_rows=wl.T, keys_per_seq=wl.max_seqlen_k, sequences=wl.num_seqs,
                    H_I=wl.H_I, d_I=wl.d_I, k=wl.k, H=wl.H, d_qk=wl.d_qk, d_v=wl.d_v),
        timing=dict(protocol="cold cache: 1 GiB read before each step; one HIP event pair per step; "
                             "value and ms_per_step from the median step", ms_min=fused["min"],
                    ms_mean=fused["mean"], ms_warm_loop=fused["warm_mean"],
                    plain_copy=copy_cal),
        roofline=roof, cpu_baseline=cpu, stages=stages, secondary=secondary,
    )
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
