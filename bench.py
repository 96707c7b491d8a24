#!/usr/bin/env python3
"""Benchmark of the weight-only-quantized LM-head hot path on one MI355X.

One step = one pass of the per-call hot path over one batch of synthetic input
on the 151936 x 1024 int4 g64 fp16-scale head at the decode shape: the logits
call at M = 1 followed by top-8 exact rescoring.  The K timed steps give
`ms_per_step`.  Each call (logits at M = 1, 32 and 256, and the rescoring) is
then also timed on its own as K back-to-back calls between two HIP events, as
the metric asks ("each timed separately"); those give `per_call` and `value`.
The load-time quantize and pack run once before the timed region and are
reported separately.

Inputs are resident in HBM before timing starts.  Each step reads a different
copy of the packed head (R copies, >= 1 GB in total) so the 256 MB last-level
cache cannot serve the weights: the numbers are cold/HBM numbers.

Prints ONE JSON line.  `value` is the mean time of the M = 1 logits call in
microseconds (lower is better); `per_call` has every call's time, GB/s and
roofline fraction; `roofline` is the M = 1 kernel's achieved algorithmic bandwidth
(measured with HIP events on the stream the library launches on) against the
8 TB/s HBM peak; `cpu_baseline` times the fp64 oracle on the host.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/call + achieved HBM GB/s (% of peak) for W4-g64 151936×1024 logits, M=1/32/256"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
PAGES_US_M1 = 240.0  # fused Marlin, RTX 5080, same head and M = 1 (vLLM PR #48870 perf table)


def algorithmic_bytes(M, V, K, bits, G):
    return V * K * bits // 8 + V * (K // G) * 2 + M * K * 2 + M * V * 4


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, help="synthetic workload name (default: the headline)")
    ap.add_argument("--ms", default=None, help="comma-separated M list (default: the workload's)")
    ap.add_argument("--topk", type=int, default=8)
    ap.add_argument("--path", type=int, default=0, help="0 automatic, 1 force the GEMV, 2 force the MFMA kernel")
    ap.add_argument("--hot", action="store_true", help="reuse one copy of the head (cache-hot; labelled)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the head would be "
              "sharded along the vocabulary, one shard per GPU); run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    import weight_only_quantized_lmhead_amd as lmh

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.workload or synth.HEADLINE]
    Ms = [int(m) for m in args.ms.split(",")] if args.ms else list(w.Ms)
    TD = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
    sdt = TD[w.scale_dtype]

    def to_dev(a, dt):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    t0 = time.time()
    W = synth.weight(w)
    Wd = to_dev(W, w.w_dtype)
    print(f"[bench] {w.name}: weight generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    # load-time rows: quantize and pack (one warm-up call each, then one timed call)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    q, s = lmh.quantize(Wd, w.bits, w.group, sdt, w.clip)
    blob = lmh.pack(q, s, w.bits, w.group)
    torch.cuda.synchronize()
    e0, e1, e2 = ev(), ev(), ev()
    e0.record()
    q, s = lmh.quantize(Wd, w.bits, w.group, sdt, w.clip)
    e1.record()
    blob = lmh.pack(q, s, w.bits, w.group)
    e2.record()
    torch.cuda.synchronize()
    quant_ms, pack_ms = e0.elapsed_time(e1), e1.elapsed_time(e2)
    del q, s

    # unquantized 16-bit reference rows for rescoring
    if w.w_dtype == "f32":
        Wref = Wd.to(torch.float16)
        del Wd
    else:
        Wref = Wd
    blob_bytes = blob.numel()
    R = 1 if args.hot else max(2, math.ceil(1e9 / blob_bytes))
    blobs = [blob] + [blob.clone() for _ in range(R - 1)]
    xs = {M: to_dev(synth.activations(w, M), w.x_dtype) for M in Ms}
    outs = {M: torch.empty((M, w.V), dtype=torch.float32, device=dev) for M in Ms}
    wss = {M: lmh.logits_workspace(M, w.K, TD[w.x_dtype], dev) for M in Ms}
    m_rs = Ms[0]
    tws = lmh.topk_workspace(m_rs, w.V, args.topk, dev)
    torch.cuda.synchronize()

    m_hd = Ms[0]  # the headline call: the decode case

    def call(M, i):
        lmh.logits(xs[M], blobs[i % R], w.V, w.K, w.bits, w.group, sdt, out=outs[M], workspace=wss[M],
                   path=args.path)

    def rescore():
        lmh.topk_rescore(xs[m_rs], Wref, outs[m_rs], args.topk, workspace=tws)

    def step(i):
        # one pass of the per-call hot path at the headline M: logits, then exact top-K rescoring
        call(m_hd, i)
        rescore()

    # ---- the timed region: K steps, synchronised on both sides ----
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start, t_end = ev(), ev()
    t_start.record()
    for i in range(args.steps):
        step(args.warmup + i)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)

    # ---- each call timed on its own: K back-to-back calls between two events on
    # the library's stream (torch's current stream), rotating the head copies ----
    def timed_loop(fn, n):
        for i in range(min(args.warmup, n)):
            fn(i)
        torch.cuda.synchronize()
        a_, b_ = ev(), ev()
        a_.record()
        for i in range(n):
            fn(i)
        b_.record()
        torch.cuda.synchronize()
        return a_.elapsed_time(b_) / n * 1e3  # us per call

    per_call = {}
    for M in Ms:
        t_us = timed_loop(lambda i, M=M: call(M, i), args.steps)
        B = algorithmic_bytes(M, w.V, w.K, w.bits, w.group)
        F = 2.0 * M * w.V * w.K
        gbs = B / (t_us * 1e-6) / 1e9
        tfl = F / (t_us * 1e-6) / 1e12
        per_call[f"M={M}"] = {
            "us": round(t_us, 3),
            "kernel": {1: "gemv", 2: "mfma"}.get(args.path, "gemv" if M == 1 and w.K <= 32768 else "mfma"),
            "algorithmic_bytes": B, "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "TFLOP/s": round(tfl, 2), "frac_mfma_f16_peak": round(tfl / MFMA_F16_PEAK_TFLOPS, 4),
        }
    rs_us = timed_loop(lambda i: rescore(), args.steps)
    per_call[f"top{args.topk}_rescore"] = {"us": round(rs_us, 3), "M": m_rs}

    m1 = per_call[f"M={Ms[0]}"]
    value = m1["us"]
    roofline = {
        "bound": "hbm", "kernel": f"lmh gemv, M={Ms[0]}", "achieved": m1["GB/s"], "peak": HBM_PEAK_GBS,
        "unit": "GB/s", "frac": m1["frac_hbm_peak"], "traffic": None,
        "bytes_per_launch": m1["algorithmic_bytes"],
    }

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        ratios = oracle.MSE_RATIOS if w.clip == "mse" else oracle.RTN_RATIOS
        od = {"f16": oracle.F16, "bf16": oracle.BF16, "f32": oracle.F32}
        rows = None
        if w.K > 2048:  # bound the sample for the widest head
            rows = np.arange(0, w.V, 8)
        Wh = W if rows is None else np.ascontiguousarray(W[rows])
        qo, so = oracle.quantize(Wh, w.bits, w.group, od[w.scale_dtype], ratios, w_dtype=od[w.w_dtype])
        x1 = synth.activations(w, Ms[0])
        n, t_cpu = 0, 0.0
        while n < 3 and (n == 0 or t_cpu < args.cpu_seconds):
            c0 = time.perf_counter()
            oracle.logits(x1, qo, so, od[w.scale_dtype], w.group, x_dtype=od[w.x_dtype])
            t_cpu += time.perf_counter() - c0
            n += 1
        frac_rows = 1.0 if rows is None else len(rows) / w.V
        us_call = t_cpu / n / frac_rows * 1e6
        cpu = {"value": round(us_call, 1), "unit": "us/call", "cores": 1, "kind": "oracle",
               "sample": f"fp64 oracle logits, M={Ms[0]}, {'all' if rows is None else len(rows)} of "
                         f"{w.V} rows, {n} calls, single thread; scaled to one whole call",
               "host_threads_available": os.cpu_count()}

    line = {
        "metric": METRIC, "value": value, "unit": "us/call", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": False, "scaling": "weak",
        "vs_baseline": round(value / PAGES_US_M1, 5) if w.name == synth.HEADLINE and Ms[0] == 1 else None,
        "vs_baseline_note": "value / 240 us (fused Marlin on RTX 5080, same head, M=1; context only)",
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": w.name, "V": w.V, "K": w.K, "bits": w.bits, "group": w.group,
                   "scale": w.scale_dtype, "x": w.x_dtype, "M": Ms, "topk": args.topk,
                   "rotating_copies": R, "cache": "hot" if args.hot else "cold"},
        "per_call": per_call,
        "load_time": {"quantize_ms": round(quant_ms, 3), "pack_ms": round(pack_ms, 3),
                      "clip": w.clip},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
