#!/usr/bin/env python3
"""Benchmark of the weight-only-quantized LM-head hot path on one MI355X.

One step = one pass of the per-call hot path over one batch of synthetic input
on the 151936 x 1024 int4 g64 fp16-scale head at the decode shape: the logits
at M = 1 and top-8 exact rescoring, in one call (lmhead_logits_topk).  The K
timed steps give `ms_per_step`.  Each call (logits at every M of the workload,
16-bit output, the zero-point form, the separate rescoring, the one-call
decode path, the embedding gather, the unquantized 16-bit control GEMV) is
then also timed on its own (the metric: "each timed separately"): at least
200 back-to-back calls between two HIP events (`us`), and the same calls
replayed from a HIP graph (`us_graph`, no host work between kernels).  All
calls are prepared once (lmh.PreparedCall), so the host issues them faster
than the GPU runs them.  The load-time quantize and pack run once before the
timed region and are reported separately.

Inputs are resident in HBM before timing starts.  Each call reads a different
copy of the packed head (R copies, >= 1 GB in total) so the 256 MB last-level
cache cannot serve the weights: the numbers are cold/HBM numbers.

Prints ONE JSON line.  `value` is the mean time of the M = 1 logits call in
microseconds (lower is better); `per_call` has every call's time, GB/s and
roofline fraction; `roofline` is the M = 1 kernel's achieved algorithmic
bandwidth (HIP events on the stream the calls run on) against the 8 TB/s HBM
peak, with the read-only ceiling measured in the same run (lmhead_stream_read
over the same bytes); every call beyond one activation row also carries the
read+write ceiling for its own byte mix (lmhead_stream_mix: the head's bytes
read, its logits buffer written) and, on an MFMA kernel, the MFMA ceiling for
its flops (lmhead_mfma_ceiling); `cpu_baseline` times the fp64 oracle on the
host cores.  With --size-sweep, `size_sweep` has the read-only stream and the
first M's logits call on heads of several times the vocabulary, each fitted
as a fixed cost per launch plus bytes over a steady rate.
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


# Sources whose change invalidates a recorded traffic measurement of the
# logits kernels.
TRAFFIC_SOURCES = ["weight_only_quantized_lmhead_amd/csrc/gemv.hip",
                   "weight_only_quantized_lmhead_amd/csrc/gemv_kernels.h",
                   "weight_only_quantized_lmhead_amd/csrc/logits_common.h",
                   "weight_only_quantized_lmhead_amd/csrc/lmh_internal.h",
                   "weight_only_quantized_lmhead_amd/build.py"]


def fit_fixed_rate(nbytes, us):
    """Least-squares fit of time = fixed + bytes / rate to calls of several
    sizes: the steady rate (GB/s, and as a fraction of the HBM peak) and the
    fixed cost of a launch (us)."""
    import numpy as np

    slope, icpt = np.polyfit(np.asarray(nbytes, dtype=np.float64), np.asarray(us, dtype=np.float64), 1)
    return {"GB/s": round(1e-3 / slope, 1), "frac_of_hbm_peak": round(1e-3 / slope / HBM_PEAK_GBS, 4),
            "fixed_us": round(icpt, 3)}


def sources_sha() -> str:
    import hashlib

    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_file(workload: str) -> str:
    """The committed counter summary of a workload: logits_<workload>_... for
    the headline head, hotpath_<workload>_... for the others."""
    for kind in ("logits", "hotpath"):
        f = os.path.join(ROOT, "profiles", f"{kind}_{workload}_hbm_traffic.md")
        if os.path.exists(f):
            return f
    return os.path.join(ROOT, "profiles", f"logits_{workload}_hbm_traffic.md")


def recorded_traffic(workload: str, kernel_prefix: str, suffix: str):
    """HBM bytes per launch of the kernel whose summary name starts with
    `kernel_prefix` and whose template arguments end with `suffix` (e.g. the
    GEMV's zero-point and top-K flags) from the committed counter summary, or
    None when there is none or the kernel sources changed since."""
    f = traffic_file(workload)
    if not os.path.exists(f):
        return None
    for line in open(f):
        if line.startswith("<!-- traffic "):
            rec = json.loads(line[len("<!-- traffic "):].rsplit("-->", 1)[0])
            if rec.get("sources_sha") != sources_sha():
                return None
            for k in rec["kernels"]:
                name = k["kernel"].split(" grid")[0]
                if name.startswith(kernel_prefix) and name.endswith(suffix):
                    return k
    return None


def _short_kernel(name: str) -> str:
    import re

    m = re.match(r"_ZN3lmh12_GLOBAL__N_1(\d+)(\w+)", name)
    if m:
        n = int(m.group(1))
        base, rest = m.group(2)[:n], m.group(2)[n:]
        targs = rest.split("EEv")[0] if "EEv" in rest else rest
        vals = [v if t == "i" else ("true" if v == "1" else "false")
                for t, v in re.findall(r"L([ib])(\d+)E", targs + "E")]
        return f"{base}<{','.join(vals)}>"
    name = name.replace("void ", "").replace("lmh::(anonymous namespace)::", "")
    name = name.split("(")[0]
    return (name.replace(" ", "") if name.startswith(("gemv_", "mfma_", "quant_", "embed_", "topk_"))
            else name[:60])


def summarize(args) -> int:
    """Write a profiles/ summary from rocprofv3 CSV output: the kernel-trace
    statistics and, when given, the FETCH_SIZE / WRITE_SIZE counter runs
    scaled by the copy kernel of known size (the packed-head clones)."""
    import csv
    import statistics

    import synth
    import weight_only_quantized_lmhead_amd as lmh

    w = synth.WORKLOADS[args.workload or synth.HEADLINE]
    out = []
    out.append(f"# Hot path on {w.name} ({w.V} x {w.K}, int{w.bits}, G={w.group}, {w.clip}), one MI355X\n")
    out.append("Commands (from the repository root; `cd /tmp && export TMPDIR=/tmp` first):\n")
    out.append("```")
    out.extend(args.cmd)
    out.append("```\n")
    rows = list(csv.DictReader(open(args.stats)))
    out.append("## Kernel durations (rocprofv3 --kernel-trace --stats)\n")
    out.append("| kernel | calls | average (us) | min (us) | max (us) | share |")
    out.append("|---|---|---|---|---|---|")
    for r in rows:
        out.append(f"| `{_short_kernel(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.1f}% |")
    out.append("")
    text = "\n".join(out) + "\n"
    if args.fetch and args.write:
        # the largest copies are the clones of the zero-point head (the
        # symmetric head's clones are smaller by one byte per row and group)
        blob = lmh.packed_bytes(w.V, w.K, w.bits | lmh.ZP, w.group)

        def per_kernel(path, counter):
            # keyed by kernel and grid size (one logits kernel serves several M)
            vals = {}
            for r in csv.DictReader(open(path)):
                if r["Counter_Name"] == counter:
                    k = _short_kernel(r["Kernel_Name"])
                    if not k.startswith("__amd"):
                        k = f"{k} grid {r['Grid_Size']}"
                    vals.setdefault(k, []).append(float(r["Counter_Value"]))
            return vals

        fv, wv = per_kernel(args.fetch, "FETCH_SIZE"), per_kernel(args.write, "WRITE_SIZE")
        # reads: the read-only stream kernel reads exactly the packed head once
        # per dispatch (and writes nothing); writes: the copies that clone the
        # zero-point packed head (their written bytes are that head's size)
        head = lmh.packed_bytes(w.V, w.K, w.bits, w.group)
        rd = [v for k, v in fv.items() if k.startswith("stream_read_kernel")][0]
        copy_f = statistics.mean(rd)
        kf = head / 1024 / copy_f
        clones = [v for v in wv["__amd_rocclr_copyBuffer"] if abs(v * 1024 / blob - 1) < 0.03]
        copy_w = statistics.mean(clones) if clones else float("nan")
        kw = blob / 1024 / copy_w if clones else 1.0
        t = ["## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE)\n",
             f"Calibration: the read-only stream kernel (lmhead_stream_read over the {head}-byte packed "
             f"head) reads FETCH_SIZE = {copy_f:.1f} KiB per dispatch, and the copies that clone the "
             f"{blob}-byte zero-point packed head write WRITE_SIZE = {copy_w:.1f} KiB, so bytes read = "
             f"FETCH_SIZE x {kf:.5f} x 1024 and bytes written = WRITE_SIZE x {kw:.5f} x 1024.\n",
             "| kernel | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | read (B) | written (B) | total (B) |",
             "|---|---|---|---|---|---|---|"]
        recs = []
        for k in sorted(fv):
            if not k.startswith(("gemv_kernel", "mfma", "topk", "quant_", "embed_", "stream_read",
                                 "stream_mix", "dense_kernel", "x_to_f16")):
                continue
            f_ = statistics.mean(fv[k])
            w_ = statistics.mean(wv.get(k, [0.0]))
            rb, wb = f_ * kf * 1024, w_ * kw * 1024
            t.append(f"| `{k}` | {len(fv[k])} | {f_:.1f} | {w_:.1f} | {rb:.0f} | {wb:.0f} | {rb + wb:.0f} |")
            recs.append({"kernel": k, "read_bytes": round(rb), "write_bytes": round(wb),
                         "bytes": round(rb + wb), "dispatches": len(fv[k])})
        t.append("")
        t.append("Per-dispatch averages over every dispatch of the kernel in the run (the counter runs "
                 "use the M values named in the commands).  `sources_sha` below is a hash of the kernel "
                 "sources; bench.py reports `traffic` only while it matches.\n")
        rec = {"workload": w.name, "sources_sha": sources_sha(), "kernels": recs}
        t.append("<!-- traffic " + json.dumps(rec) + " -->")
        text += "\n".join(t) + "\n"
    with open(args.out, "w") as fh:
        fh.write(text)
    print(text)
    return 0


SQ_PASSES = [
    ["SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
     "SQ_ACTIVE_INST_VMEM", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY",
     "GRBM_GUI_ACTIVE"],
    ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR",
     "SQ_INSTS_SALU", "SQ_LDS_BANK_CONFLICT", "SQ_WAVES", "GRBM_GUI_ACTIVE"],
]


def summarize_sq(args) -> int:
    """Write a profiles/ summary of SQ counters per kernel (the logits
    kernels, the read-only stream, the quantizer and packers) from the
    counter_collection.csv files of the SQ_PASSES runs (--sq, one per pass)."""
    import csv
    import statistics

    vals = {}  # (kernel, grid) -> counter -> [values]
    for path in args.sq:
        for r in csv.DictReader(open(path)):
            k = _short_kernel(r["Kernel_Name"])
            if not k.startswith(("gemv_kernel", "mfma", "stream_read", "quant_", "pack_")):
                continue
            key = f"{k} grid {r['Grid_Size']}"
            vals.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = [f"# SQ counters per kernel ({args.workload or 'headline'} head), one MI355X\n",
           "Commands (from the repository root; `export TMPDIR=/tmp` first):\n", "```"]
    out += args.cmd
    out += ["```\n",
            "Per-dispatch means over every dispatch of a kernel (one kernel per M; the grid says which). "
            "Derived columns, with the kernel's GPU cycles = GRBM_GUI_ACTIVE / 8 (the counter is summed "
            "over the 8 XCDs) and 1024 SIMDs: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024) "
            "(matches 16 cycles per 16x16x32 fp16 MFMA x SQ_INSTS_MFMA); VALU busy = 4 x (SQ_INSTS_VALU - "
            "SQ_INSTS_MFMA) / (cycles x 1024) (a wave64 VALU instruction holds its SIMD 4 cycles); LDS "
            "and VMEM active = SQ_ACTIVE_INST_* / SQ_WAVE_CYCLES; wait = SQ_WAIT_INST_ANY / "
            "SQ_WAVE_CYCLES; VALU/MFMA = non-MFMA VALU instructions per MFMA; bank conflicts per LDS "
            "instruction.\n",
            "| kernel | MFMA busy | VALU busy | LDS active | VMEM active | wait | VALU/MFMA | LDS instr/MFMA | bank conflicts/LDS instr | waves |",
            "|---|---|---|---|---|---|---|---|---|---|"]
    for key in sorted(vals):
        c = {n: statistics.mean(v) for n, v in vals[key].items()}
        g = lambda n: c.get(n, float("nan"))
        # GRBM_GUI_ACTIVE is summed over the 8 XCDs, the MFMA busy cycles over
        # the 1024 SIMDs; SQ_INSTS_VALU counts MFMA instructions too, and one
        # VALU instruction of a wave occupies its SIMD for 4 cycles
        gpu_cycles = g("GRBM_GUI_ACTIVE") / 8
        busy = g("SQ_VALU_MFMA_BUSY_CYCLES") / (gpu_cycles * 1024)
        mf = g("SQ_INSTS_MFMA")
        valu_busy = (g("SQ_INSTS_VALU") - mf) * 4 / (gpu_cycles * 1024)
        wc = g("SQ_WAVE_CYCLES")
        out.append(f"| `{key}` | {busy:.1%} | {valu_busy:.1%} | "
                   f"{g('SQ_ACTIVE_INST_LDS') / wc:.1%} | {g('SQ_ACTIVE_INST_VMEM') / wc:.1%} | "
                   f"{g('SQ_WAIT_INST_ANY') / wc:.1%} | "
                   f"{(g('SQ_INSTS_VALU') - mf) / mf if mf else float('nan'):.2f} | "
                   f"{g('SQ_INSTS_LDS') / mf if mf else float('nan'):.2f} | "
                   f"{g('SQ_LDS_BANK_CONFLICT') / max(g('SQ_INSTS_LDS'), 1):.2f} | {g('SQ_WAVES'):.0f} |")
    out.append("\nRaw means:\n")
    out.append("| kernel | " + " | ".join(sorted({n for v in vals.values() for n in v})) + " |")
    names = sorted({n for v in vals.values() for n in v})
    out.append("|---|" + "---|" * len(names))
    for key in sorted(vals):
        out.append(f"| `{key}` | " + " | ".join(
            f"{statistics.mean(vals[key][n]):.4g}" if n in vals[key] else "" for n in names) + " |")
    text = "\n".join(out) + "\n"
    with open(args.out, "w") as fh:
        fh.write(text)
    print(text)
    return 0


def decode_agreement(args, w, lmh, synth, to_dev, blob, Wref, sdt, dev):
    """Top-1 agreement of the quantized head with the unquantized 16-bit weight
    (lmhead_dense_logits: exact 16-bit products, fp32 sums) over N seeded
    decode states, before and after exact top-K rescoring (vLLM PR #48870,
    review comment, point 2), and the overlap of the quantized and reference
    top-K sets.  Each state is one activation row; they are run in batches."""
    import torch

    n, K = args.agreement, args.topk
    X = to_dev(synth.decode_states(w, 0, n), w.x_dtype)
    ref1 = torch.empty(n, dtype=torch.int64, device=dev)
    margin = torch.empty(n, dtype=torch.float32, device=dev)
    ref_sets, q_sets = [], []
    for i in range(0, n, 4):  # the dense control takes up to 4 rows per call
        yd = lmh.dense_logits(X[i:i + 4], Wref)
        ref1[i:i + 4] = torch.argmax(yd, dim=1)
        t2 = torch.topk(yd, 2, dim=1).values
        margin[i:i + 4] = t2[:, 0] - t2[:, 1]
        ref_sets.append(torch.topk(yd, K, dim=1).indices)
    B = 64
    q1 = torch.empty(n, dtype=torch.int64, device=dev)
    r1 = torch.empty(n, dtype=torch.int64, device=dev)
    for i in range(0, n, B):
        xb = X[i:i + B]
        yq = lmh.logits(xb, blob, w.V, w.K, w.bits, w.group, sdt)
        q1[i:i + B] = torch.argmax(yq, dim=1)
        q_sets.append(torch.topk(yq, K, dim=1).indices)
        _, _, t1 = lmh.logits_topk(xb, blob, w.V, w.K, w.bits, w.group, sdt, Wref, K)
        r1[i:i + B] = t1.long()
    rs, qs = torch.cat(ref_sets), torch.cat(q_sets)
    overlap = (rs.unsqueeze(2) == qs.unsqueeze(1)).any(dim=2).float().mean().item()
    flip_q = q1 != ref1
    flip_r = r1 != ref1
    worst = margin[flip_r].max().item() if flip_r.any() else 0.0
    return {"states": n, "topk": K,
            "reference": "unquantized 16-bit weight, fp32-accumulated GEMV (lmhead_dense_logits)",
            "top1_agreement_quantized": round(1.0 - flip_q.float().mean().item(), 6),
            "top1_agreement_rescored": round(1.0 - flip_r.float().mean().item(), 6),
            "flips_quantized": int(flip_q.sum().item()), "flips_rescored": int(flip_r.sum().item()),
            "max_reference_margin_of_rescored_flips": worst,
            "states_with_reference_margin_below_1e-3": int((margin < 1e-3).sum().item()),
            "topk_set_overlap": round(overlap, 6)}


def cpu_oracle_baseline(w, W, Ms, synth, np, budget_s):
    """The fp64 oracle on the host cores: logits at the first M (one thread and
    all cores, median of 3) and the quantizer (RTN and MSE clip search, all
    cores), each on a bounded row sample scaled to the whole head."""
    import platform
    import statistics

    import oracle

    od = {"f16": oracle.F16, "bf16": oracle.BF16, "f32": oracle.F32}
    ratios = oracle.MSE_RATIOS if w.clip == "mse" else oracle.RTN_RATIOS
    threads = oracle.default_threads()
    cpu_model = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass

    def med3(fn):
        ts = []
        for _ in range(3):
            c0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - c0)
        return statistics.median(ts)

    # row samples sized from a probe so that each measurement takes ~budget/8
    x1 = synth.activations(w, Ms[0])
    probe = np.ascontiguousarray(W[: min(w.V, 2048)])
    qp, sp = oracle.quantize(probe, w.bits, w.group, od[w.scale_dtype], ratios, w_dtype=od[w.w_dtype])
    t_probe = med3(lambda: oracle.logits(x1, qp, sp, od[w.scale_dtype], w.group,
                                        x_dtype=od[w.x_dtype], threads=1))
    per_row = t_probe / probe.shape[0]
    n_rows = int(min(w.V, max(2048, budget_s / 8 / max(per_row, 1e-9))))
    step = max(1, w.V // n_rows)
    rows = np.arange(0, w.V, step)
    Wr = np.ascontiguousarray(W[rows])
    frac = len(rows) / w.V
    qo, so = oracle.quantize(Wr, w.bits, w.group, od[w.scale_dtype], ratios, w_dtype=od[w.w_dtype])
    t1 = med3(lambda: oracle.logits(x1, qo, so, od[w.scale_dtype], w.group, x_dtype=od[w.x_dtype],
                                    threads=1))
    tn = med3(lambda: oracle.logits(x1, qo, so, od[w.scale_dtype], w.group, x_dtype=od[w.x_dtype],
                                    threads=threads))
    # the quantizer on a smaller sample (RTN; the 5-ratio search)
    qrows = rows[:: max(1, len(rows) // 4096)] if len(rows) > 4096 else rows
    Wq = np.ascontiguousarray(W[qrows])
    qfrac = len(qrows) / w.V
    t_rtn = med3(lambda: oracle.quantize(Wq, w.bits, w.group, od[w.scale_dtype], oracle.RTN_RATIOS,
                                         w_dtype=od[w.w_dtype], threads=threads))
    t_mse = med3(lambda: oracle.quantize(Wq, w.bits, w.group, od[w.scale_dtype], oracle.MSE_RATIOS,
                                         w_dtype=od[w.w_dtype], threads=threads))
    return {"value": round(tn / frac * 1e6, 1), "unit": "us/call", "cores": threads,
            "kind": "oracle",
            "sample": (f"fp64 oracle logits, M={Ms[0]}, every {step}th of the {w.V} rows "
                       f"({len(rows)} rows), median of 3 runs on {threads} threads (row ranges "
                       f"side by side), scaled to one whole call"),
            "single_thread_us": round(t1 / frac * 1e6, 1),
            "quantize_rtn_ms": round(t_rtn / qfrac * 1e3, 1),
            "quantize_mse_ms": round(t_mse / qfrac * 1e3, 1),
            "quantize_sample": (f"{len(qrows)} rows, median of 3 on {threads} threads, scaled to "
                                f"the whole head"),
            "cpu_model": cpu_model, "host_threads_visible": os.cpu_count()}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--calls", type=int, default=None,
                    help="calls per per-call timing loop (default 200 whatever --steps is; "
                         "profiled runs may ask for fewer)")
    ap.add_argument("--workload", default=None, help="synthetic workload name (default: the headline)")
    ap.add_argument("--ms", default=None, help="comma-separated M list (default: the workload's)")
    ap.add_argument("--topk", type=int, default=8)
    ap.add_argument("--path", type=int, default=0, help="0 automatic, 1 GEMV, 2 register-fed MFMA, 3 LDS-staged MFMA, 4 activation-resident MFMA, 5 split-K MFMA")
    ap.add_argument("--hot", action="store_true", help="reuse one copy of the head (cache-hot; labelled)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the logits calls of the workload (no 16-bit output, zero-point, "
                         "top-K, embedding or control entries)")
    ap.add_argument("--agreement", type=int, default=0, metavar="N",
                    help="also report, over N seeded decode states (one activation row each), the "
                         "top-1 agreement with the unquantized 16-bit weight before and after exact "
                         "top-K rescoring, and the top-K set overlap")
    ap.add_argument("--size-sweep", default=None, metavar="MULTS",
                    help="also time the read-only stream and the first M's logits call on heads of "
                         "these multiples of the workload's vocabulary (e.g. 2,4,8; cold), and fit "
                         "time = fixed + bytes / rate to both")
    ap.add_argument("--cpu-seconds", type=float, default=16.0)
    ap.add_argument("--record", metavar="PATH",
                    help="also write the JSON line, with the command that made it, as a markdown file")
    ap.add_argument("--summarize", action="store_true",
                    help="write a profiles/ summary from rocprofv3 CSV files instead of timing")
    ap.add_argument("--stats", help="kernel_stats.csv of a --kernel-trace --stats run")
    ap.add_argument("--fetch", help="counter_collection.csv of a --pmc FETCH_SIZE run")
    ap.add_argument("--write", help="counter_collection.csv of a --pmc WRITE_SIZE run")
    ap.add_argument("--out", help="summary file to write")
    ap.add_argument("--cmd", action="append", default=[], help="command line to record (repeatable)")
    ap.add_argument("--summarize-sq", action="store_true",
                    help="write a profiles/ summary of SQ counters (--sq files) instead of timing")
    ap.add_argument("--sq", action="append", default=[],
                    help="counter_collection.csv of one SQ_PASSES run (repeatable)")
    args = ap.parse_args()
    if args.summarize:
        return summarize(args)
    if args.summarize_sq:
        return summarize_sq(args)

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
    ncalls = 200 if args.calls is None else max(1, args.calls)

    def to_dev(a, dt):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    t0 = time.time()
    W = synth.weight(w)
    Wd = to_dev(W, w.w_dtype)
    log(f"{w.name}: weight generated in {time.time() - t0:.1f}s")

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
    # the fused quantize + pack writes the same blob with no int8 copy of the codes
    fused = lmh.quantize_pack(Wd, w.bits, w.group, sdt, w.clip)
    torch.cuda.synchronize()
    e0.record()
    lmh.quantize_pack(Wd, w.bits, w.group, sdt, w.clip, out=fused)
    e1.record()
    torch.cuda.synchronize()
    qp_ms = e0.elapsed_time(e1)
    if not torch.equal(fused, blob):
        print("bench.py: fused quantize+pack blob differs from pack(quantize(w))", file=sys.stderr)
        return 1
    del fused
    # the zero-point (asymmetric) form of the same head: round to nearest only
    zbits = w.bits | lmh.ZP
    zblob = lmh.quantize_pack(Wd, zbits, w.group, sdt)
    torch.cuda.synchronize()
    e0.record()
    lmh.quantize_pack(Wd, zbits, w.group, sdt, out=zblob)
    e1.record()
    torch.cuda.synchronize()
    qpz_ms = e0.elapsed_time(e1)
    log(f"load-time kernels done")

    # unquantized 16-bit reference rows for rescoring (and the control GEMV)
    if w.w_dtype == "f32":
        Wref = Wd.to(torch.float16)
        del Wd
    else:
        Wref = Wd
    blob_bytes = blob.numel()
    R = 1 if args.hot else max(2, math.ceil(1e9 / blob_bytes))
    blobs = [blob] + [blob.clone() for _ in range(R - 1)]
    zblobs = [zblob] + [zblob.clone() for _ in range(R - 1)] if not args.no_extras else []
    xs = {M: to_dev(synth.activations(w, M), w.x_dtype) for M in Ms}
    outs = {M: torch.empty((M, w.V), dtype=torch.float32, device=dev) for M in Ms}
    wss = {M: lmh.logits_workspace(M, w.K, TD[w.x_dtype], dev) for M in Ms}
    m_rs = Ms[0]
    tws = lmh.topk_workspace(m_rs, w.V, args.topk, dev)
    fws = lmh.logits_topk_workspace(m_rs, w.V, w.K, TD[w.x_dtype], args.topk, dev)
    t_idx = torch.empty((m_rs, args.topk), dtype=torch.int32, device=dev)
    t_val = torch.empty((m_rs, args.topk), dtype=torch.float32, device=dev)
    t_top1 = torch.empty((m_rs,), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    # Every timed call is a prepared call (arguments converted once, see
    # lmh.PreparedCall), so the host issues calls faster than the GPU runs
    # them.  Each entry is timed two ways on the stream the calls are bound
    # to: `us`, back-to-back calls between two HIP events (rotating the head
    # copies); `us_graph`, the same calls captured once in a HIP graph and
    # replayed (no host work at all between kernels).
    def ev_time(calls, n):
        for i in range(min(args.warmup, n)):
            calls[i % len(calls)]()
        torch.cuda.synchronize()
        a_, b_ = ev(), ev()
        a_.record()
        for i in range(n):
            calls[i % len(calls)]()
        b_.record()
        torch.cuda.synchronize()
        return a_.elapsed_time(b_) / n * 1e3

    def graph_time(make_calls, n):
        gs = torch.cuda.Stream()
        with torch.cuda.stream(gs):
            calls = make_calls()
            for i in range(min(args.warmup, n)):
                calls[i % len(calls)]()
        gs.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gs):
            for i in range(n):
                calls[i % len(calls)]()
        a_, b_ = ev(), ev()
        reps = 5
        with torch.cuda.stream(gs):  # replay() launches on the current stream
            g.replay()
            gs.synchronize()
            a_.record(gs)
            for _ in range(reps):
                g.replay()
            b_.record(gs)
        gs.synchronize()
        t_ = a_.elapsed_time(b_) / (reps * n) * 1e3
        del g
        return t_

    def both(make_calls):
        return round(ev_time(make_calls(), ncalls), 3), round(graph_time(make_calls, ncalls), 3)

    def prep_logits(M, bl, bits, out, path=None):
        return lambda: [lmh.prepare_logits(xs[M], b, w.V, w.K, bits, w.group, sdt, out=out,
                                           workspace=wss[M], path=args.path if path is None else path)
                        for b in bl]

    def prep_one_call():
        return [lmh.prepare_logits_topk(xs[m_rs], b, w.V, w.K, w.bits, w.group, sdt, Wref, args.topk,
                                        t_idx, t_val, t_top1, out=outs[m_rs], workspace=fws)
                for b in blobs]

    # ---- the timed region: K steps of the per-call hot path at the decode
    # shape (logits + top-K rescoring in one call), synchronised on both sides ----
    steps_calls = prep_one_call()
    for i in range(args.warmup):
        steps_calls[i % R]()
    torch.cuda.synchronize()
    t_start, t_end = ev(), ev()
    t_start.record()
    for i in range(args.steps):
        steps_calls[(args.warmup + i) % R]()
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    log(f"timed region: {total_ms / args.steps * 1e3:.2f} us per step")

    def auto_kernel(M):
        names = {lmh.PATH_GEMV: "gemv", lmh.PATH_MFMA: "mfma", lmh.PATH_MFMA_LDS: "mfma_lds",
                 lmh.PATH_MFMA_XRES: "mfma_xres", lmh.PATH_MFMA_SPLITK: "mfma_splitk"}
        xdt = torch.bfloat16 if w.x_dtype == "bf16" else torch.float16
        return names[lmh.auto_path(M, w.K, w.bits, w.group, xdt)]

    def mix_ceiling(out, kernel_us):
        """The practical HBM rate for this call's mix of bytes: lmhead_stream_mix
        reading the packed head (the same rotating copies) and writing the
        call's logits buffer, timed the same two ways."""
        cu, cug = both(lambda: [lmh.prepare_stream_mix(b, out) for b in blobs])
        wb = out.numel() * out.element_size()
        return {"us": cu, "us_graph": cug, "read_bytes": blob_bytes, "write_bytes": wb,
                "GB/s": round((blob_bytes + wb) / (cu * 1e-6) / 1e9, 1),
                "kernel_frac_of_mix_ceiling": round(cu / kernel_us, 4)}

    per_call = {}
    csink = torch.empty(lmh.MFMA_CEILING_SINK, dtype=torch.float32, device=dev)
    for M in Ms:
        us, usg = both(prep_logits(M, blobs, w.bits, outs[M]))
        B = algorithmic_bytes(M, w.V, w.K, w.bits, w.group)
        F = 2.0 * M * w.V * w.K
        gbs = B / (us * 1e-6) / 1e9
        tfl = F / (us * 1e-6) / 1e12
        per_call[f"M={M}"] = {
            "us": us, "us_graph": usg,
            "kernel": {1: "gemv", 2: "mfma", 3: "mfma_lds", 4: "mfma_xres",
                       5: "mfma_splitk"}.get(args.path, auto_kernel(M)),
            "algorithmic_bytes": B, "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "TFLOP/s": round(tfl, 2), "frac_mfma_f16_peak": round(tfl / MFMA_F16_PEAK_TFLOPS, 4),
        }
        log(f"M={M}: {us:.2f} us (graph {usg:.2f})")
        if M > 2 and per_call[f"M={M}"]["kernel"] != "gemv":
            # the practical MFMA ceiling for the same flops on the same grid
            # shape (lmhead_mfma_ceiling: MFMA chains alone, then with 2 and 4
            # independent fp32 FMAs per MFMA -- a G-column group's scale FMAs
            # are 128 / G per MFMA)
            rounds = max(1, round(F / lmh.mfma_ceiling_flops(1)))
            cf = lmh.mfma_ceiling_flops(rounds)
            mc = {}
            for nv in (0, 2, 4):
                cu, cug = both(lambda nv=nv: [lmh.prepare_mfma_ceiling(rounds, nv, csink)])
                mc[nv] = cu
            ctf = cf / (mc[0] * 1e-6) / 1e12
            per_call[f"M={M}"]["mfma_ceiling"] = {
                "rounds": rounds, "flops": cf, "us": mc[0], "TFLOP/s": round(ctf, 2),
                "frac_of_mfma_f16_peak": round(ctf / MFMA_F16_PEAK_TFLOPS, 4),
                "us_with_2_fma_per_mfma": mc[2], "us_with_4_fma_per_mfma": mc[4],
                "kernel_frac_of_ceiling": round(tfl / ctf, 4)}
        if M > 1:
            per_call[f"M={M}"]["mix_ceiling"] = mix_ceiling(outs[M], us)
    if not args.no_extras:
        # 16-bit logits (fp16 output: half the output bytes) at every M > 1
        for M in Ms:
            if M == 1:
                continue
            o16 = torch.empty((M, w.V), dtype=torch.float16, device=dev)
            us, usg = both(prep_logits(M, blobs, w.bits, o16))
            B = algorithmic_bytes(M, w.V, w.K, w.bits, w.group) - M * w.V * 2
            per_call[f"M={M} y=f16"] = {"us": us, "us_graph": usg, "algorithmic_bytes": B,
                                         "GB/s": round(B / (us * 1e-6) / 1e9, 1),
                                         "TFLOP/s": round(2.0 * M * w.V * w.K / (us * 1e-6) / 1e12, 2),
                                         "mix_ceiling": mix_ceiling(o16, us)}
            del o16
        # zero-point heads: the same kernels with a per-row, per-group zero point
        for M in Ms:
            us, usg = both(prep_logits(M, zblobs, zbits, outs[M]))
            B = algorithmic_bytes(M, w.V, w.K, w.bits, w.group) + w.V * (w.K // w.group)
            per_call[f"M={M} zp"] = {"us": us, "us_graph": usg, "algorithmic_bytes": B,
                                      "GB/s": round(B / (us * 1e-6) / 1e9, 1),
                                      "TFLOP/s": round(2.0 * M * w.V * w.K / (us * 1e-6) / 1e12, 2)}
        us, usg = both(lambda: [lmh.prepare_topk_rescore(xs[m_rs], Wref, outs[m_rs], args.topk, t_idx,
                                                         t_val, t_top1, tws)])
        per_call[f"top{args.topk}_rescore"] = {"us": us, "us_graph": usg, "M": m_rs}
        us, usg = both(prep_one_call)
        per_call[f"logits+top{args.topk}_one_call"] = {"us": us, "us_graph": usg, "M": m_rs}
        # input-embedding gather from the same packed blob: one decode token and a
        # 4096-token prefill, rows in the activation dtype
        gen = torch.Generator(device="cpu").manual_seed(w.wid)
        for T in (1, 4096):
            ids = torch.randint(0, w.V, (T,), generator=gen, dtype=torch.int32).to(dev)
            eo = torch.empty((T, w.K), dtype=TD[w.x_dtype], device=dev)
            us, usg = both(lambda ids=ids, eo=eo: [lmh.prepare_embed(ids, b, w.V, w.K, w.bits, w.group,
                                                                     sdt, eo) for b in blobs])
            eb = T * (w.K * w.bits // 8 + (w.K // w.group) * 2 + w.K * 2 + 4)
            per_call[f"embed_T={T}"] = {"us": us, "us_graph": usg, "algorithmic_bytes": eb,
                                         "GB/s": round(eb / (us * 1e-6) / 1e9, 1)}
        # the unquantized 16-bit control GEMV at one activation row (vLLM PR
        # #48870, review comment, point 1), over rotating copies of the weight
        RC = 1 if args.hot else max(2, math.ceil(1e9 / (Wref.numel() * 2)))
        wrefs = [Wref] + [Wref.clone() for _ in range(RC - 1)]
        x1 = xs[Ms[0]][:1]
        oc = torch.empty((1, w.V), dtype=torch.float32, device=dev)
        us, usg = both(lambda: [lmh.prepare_dense_logits(x1, wr, oc) for wr in wrefs])
        Bc = w.V * w.K * 2 + w.K * 2 + w.V * 4
        qus = per_call[f"M={Ms[0]}"]["us"] if Ms[0] == 1 else None
        per_call["control_16bit_gemv_M=1"] = {
            "us": us, "us_graph": usg, "algorithmic_bytes": Bc, "GB/s": round(Bc / (us * 1e-6) / 1e9, 1),
            "frac_hbm_peak": round(Bc / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "quantized_speedup": round(us / qus, 3) if qus else None, "weight_copies": RC}
        del wrefs

    agreement = decode_agreement(args, w, lmh, synth, to_dev, blob, Wref, sdt, dev) if args.agreement else None

    m1 = per_call[f"M={Ms[0]}"]
    value = m1["us"]
    # the symmetric GEMV without the top-K epilogue (template flags ZP, TK, and
    # the activation source: 0 fp16 through the scalar unit, 2 bf16 converted)
    xm = "2" if w.x_dtype == "bf16" else "0"
    tr = (recorded_traffic(w.name, "gemv_kernel<", f",false,false,{xm}>")
          if m1["kernel"] == "gemv" else None)
    roofline = {
        "bound": "hbm", "kernel": f"lmh {m1['kernel']}, M={Ms[0]}", "achieved": m1["GB/s"],
        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": m1["frac_hbm_peak"],
        "traffic": tr["bytes"] if tr else None, "bytes_per_launch": m1["algorithmic_bytes"],
        "traffic_source": os.path.relpath(traffic_file(w.name), ROOT) if tr else None,
    }
    # the practical read ceiling measured in the same run: a read-only kernel
    # (lmhead_stream_read) over the same bytes as the packed head, rotating the
    # same copies, timed the same way
    sink = torch.empty(1024, dtype=torch.uint8, device=dev)
    rd_us, rd_usg = both(lambda: [lmh.prepare_stream_read(b, sink) for b in blobs])
    rd_gbs = blob_bytes / (rd_us * 1e-6) / 1e9
    roofline["read_ceiling"] = {"GB/s": round(rd_gbs, 1), "us": rd_us, "us_graph": rd_usg,
                                "bytes": blob_bytes, "frac_of_hbm_peak": round(rd_gbs / HBM_PEAK_GBS, 4)}
    roofline["frac_of_read_ceiling"] = round(rd_us / value, 4) if Ms[0] == 1 else None

    sweep = None
    if args.size_sweep:
        # the same two calls on longer vocabularies: the slope of time against
        # bytes is the steady rate, the intercept the fixed cost of a launch
        mults = [1] + [int(m) for m in args.size_sweep.split(",") if int(m) > 1]
        pts = [(1, blob_bytes, R, rd_us, m1["us"])]
        gen = torch.Generator(device=dev).manual_seed(w.wid)
        for mult in mults[1:]:
            Vm = w.V * mult
            Wm = (torch.randn((Vm, w.K), generator=gen, device=dev) * 0.02).to(torch.float16)
            bm = lmh.quantize_pack(Wm, w.bits, w.group, sdt)
            del Wm
            Rm = 1 if args.hot else max(2, math.ceil(1e9 / bm.numel()))
            bms = [bm] + [bm.clone() for _ in range(Rm - 1)]
            om = torch.empty((Ms[0], Vm), dtype=torch.float32, device=dev)
            r_us, _ = both(lambda: [lmh.prepare_stream_read(b, sink) for b in bms])
            l_us, _ = both(lambda: [lmh.prepare_logits(xs[Ms[0]], b, Vm, w.K, w.bits, w.group, sdt,
                                                       out=om, workspace=wss[Ms[0]], path=args.path)
                                    for b in bms])
            pts.append((mult, bm.numel(), Rm, r_us, l_us))
            log(f"size x{mult}: read {r_us:.2f} us, logits {l_us:.2f} us")
            del bms, bm, om
            torch.cuda.empty_cache()

        sweep = {"multiples": [p[0] for p in pts], "bytes": [p[1] for p in pts],
                 "copies": [p[2] for p in pts], "read_us": [p[3] for p in pts],
                 "logits_us": [p[4] for p in pts], "M": Ms[0],
                 "read_fit": fit_fixed_rate([p[1] for p in pts], [p[3] for p in pts]),
                 "logits_fit": fit_fixed_rate([p[1] for p in pts], [p[4] for p in pts])}

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle on the host cores)")
        cpu = cpu_oracle_baseline(w, W, Ms, synth, np, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": value, "unit": "us/call", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": False, "scaling": "weak",
        "vs_baseline": round(value / PAGES_US_M1, 5) if w.name == synth.HEADLINE and Ms[0] == 1 else None,
        "vs_baseline_note": "value / 240 us (fused Marlin on RTX 5080, same head, M=1; context only)",
        "dtype": "f16" if w.x_dtype == "f16" else "bf16->f16", "data": "synthetic",
        "config": {"workload": w.name, "V": w.V, "K": w.K, "bits": w.bits, "group": w.group,
                   "scale": w.scale_dtype, "x": w.x_dtype, "M": Ms, "topk": args.topk,
                   "rotating_copies": R, "cache": "hot" if args.hot else "cold",
                   "calls_per_timing": ncalls},
        "per_call": per_call,
        "load_time": {"quantize_ms": round(quant_ms, 3), "pack_ms": round(pack_ms, 3),
                      "quantize_pack_ms": round(qp_ms, 3),
                      "quantize_pack_zp_ms": round(qpz_ms, 3),
                      "clip": w.clip},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if agreement is not None:
        line["agreement"] = agreement
    if sweep is not None:
        line["size_sweep"] = sweep
    print(json.dumps(line), flush=True)
    if args.record:
        argv, skip = [], False
        for a in sys.argv[1:]:
            if skip:
                skip = False
            elif a == "--record":
                skip = True
            elif not a.startswith("--record="):
                argv.append(a)
        with open(args.record, "w") as f:
            f.write(f"# bench.py line: {w.name}\n\nCommand (from the repository root): "
                    f"`python3 bench.py {' '.join(argv)}`\n\n```json\n{json.dumps(line)}\n```\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
