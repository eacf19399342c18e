"""Benchmark of the fused integer-only attention on one MI355X.

A step is one fused launch over the whole batch of the ViT-B/DeiT-B-shaped
workload (B=128, H=12, N=197, d=64, seeded synthetic int8 inputs already
resident in HBM).  Prints one JSON line:
  value      int8 TOPS = 4 N^2 d B H / (time per step)  (both contractions,
             a multiply-accumulate counted as 2 ops)
  roofline   achieved HBM GB/s of the fused kernel (algorithmic bytes
             4 N d per head: Q, K, V read once, Out written once) against the
             8 TB/s peak; the per-launch duration comes from HIP events
             around every launch on the launch stream
  traffic    HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE,
             read from profiles/ when recorded for the current kernel source
  cpu_baseline  the CPU oracle (single thread) on the same inputs

`--record-traffic FETCH_CSV WRITE_CSV` turns the counter files of two
rocprofv3 --pmc runs of `bench.py --copy-calib` (FETCH_SIZE, then WRITE_SIZE)
into profiles/traffic_<workload>.json: each counter's KiB per dispatch of the
attention kernel, scaled by the factor that maps the same counter on the
256 MiB device copy to its known size.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_I8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA
# VALU lane rate: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz, one 32-bit integer
# operation per lane and cycle (a wave64 instruction occupies a SIMD 4 cycles)
VALU_LANE_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
KERNEL_DIR = os.path.join(ROOT, "integer_only_quantized_int8_amd", "csrc")
METRIC = "integer-only MSA int8 TOPS + % roofline, B=128 H=12 N=197 d=64, 1 MI355X"


def kernel_source_hash() -> str:
    """Hash of the attention kernel's sources (the traffic record is tied to it)."""
    h = hashlib.sha256()
    for name in sorted(n for n in os.listdir(KERNEL_DIR)
                       if n.startswith("iqattn_") and n.endswith((".hip", ".h"))):
        h.update(name.encode())
        h.update(open(os.path.join(KERNEL_DIR, name), "rb").read())
    return h.hexdigest()[:16]


def _load_record(kind: str, workload: str):
    """A committed counter record of profiles/, or None when it is missing or
    belongs to other attention sources."""
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec


def load_traffic(workload: str):
    return _load_record("traffic", workload)


def load_counters(workload: str):
    return _load_record("counters", workload)


# one rocprofv3 --pmc pass: every counter of it, averaged over the attention
# kernel's dispatches (GRBM_GUI_ACTIVE sums the 8 XCDs' busy cycles)
UNIT_COUNTERS = ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES",
                 "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE")
SIMDS = 256 * 4


def record_counters(csv_path: str, workload: str) -> dict:
    """Per-dispatch unit counters of the attention kernel from a rocprofv3 --pmc
    counter file, with the figures derived from them."""
    import csv
    sums, counts = {}, {}
    kernel = None
    for r in csv.DictReader(open(csv_path)):
        if not _is_attention_kernel(r["Kernel_Name"]):
            continue
        kernel = r["Kernel_Name"]
        c = r["Counter_Name"]
        sums[c] = sums.get(c, 0.0) + float(r["Counter_Value"])
        counts[c] = counts.get(c, 0) + 1
    if not sums:
        raise SystemExit(f"{csv_path}: no attention-kernel dispatches")
    avg = {c: sums[c] / counts[c] for c in sums}
    valu = avg["SQ_INSTS_VALU"] - avg.get("SQ_INSTS_MFMA", 0.0)
    xcd_cycles = avg["GRBM_GUI_ACTIVE"] / 8.0
    rec = {"workload": workload, "kernel": kernel, "kernel_source_sha256_16": kernel_source_hash(),
           "dispatches": min(counts.values()), "per_dispatch": {c: round(v) for c, v in avg.items()},
           "valu_insts_per_launch": round(valu),
           # wave64 VALU instructions x 4 cycles (16 lanes per cycle) per SIMD over the
           # dispatch's busy cycles, and the matrix cores' busy share
           "valu_busy_share": round(4.0 * valu / SIMDS / xcd_cycles, 4),
           "mfma_busy_share": round(avg.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / SIMDS / xcd_cycles, 4)}
    return rec


COPY_CALIB_BYTES = 256 << 20


def _counter_rows(path, counter):
    import csv
    return [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]


def _is_attention_kernel(name: str) -> bool:
    return "iqattn::" in name and ("iqattn_fast" in name or "iqattn_generic" in name)


def record_traffic(fetch_csv: str, write_csv: str, workload: str) -> dict:
    """Calibrated HBM bytes per launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch)."""
    rec = {"workload": workload, "kernel_source_sha256_16": kernel_source_hash(),
           "copy_calibration_bytes": COPY_CALIB_BYTES}
    total = 0.0
    for key, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"),
                               ("write", write_csv, "WRITE_SIZE")):
        rows = _counter_rows(path, counter)
        kern = [float(r["Counter_Value"]) for r in rows if _is_attention_kernel(r["Kernel_Name"])]
        copy = [float(r["Counter_Value"]) for r in rows
                if "copyBuffer" in r["Kernel_Name"] or "elementwise" in r["Kernel_Name"]]
        if not kern or not copy:
            raise SystemExit(f"{path}: no attention-kernel or copy dispatches with {counter}")
        copy_kib = max(copy)            # the 256 MiB calibration copy is the largest
        scale = COPY_CALIB_BYTES / (copy_kib * 1024.0)
        kib = sum(kern) / len(kern)
        rec[key] = {"counter": counter, "kernel_kib_per_dispatch": round(kib, 3),
                    "dispatches": len(kern), "copy_kib": round(copy_kib, 3),
                    "scale": round(scale, 4), "bytes_per_launch": round(kib * 1024.0 * scale)}
        total += kib * 1024.0 * scale
    rec["hbm_bytes_per_launch"] = round(total)
    return rec


def bench_linear(args):
    """Time one int8 linear layer (x W^T with the fused requantisation) on the
    ViT-B projection shapes; roofline against the dense int8 MFMA peak."""
    import numpy as np
    import torch
    from integer_only_quantized_int8_amd import workloads as W
    from integer_only_quantized_int8_amd.iqattn import IQLinear
    lw = W.linear_workload(args.linear)
    P = lw.params
    dev = torch.device("cuda:0")
    x = torch.from_numpy(lw.x).to(dev)
    w = torch.from_numpy(lw.w).to(dev)
    lin = IQLinear(P)
    outs = None
    if P["layout"] == 1:
        shape = (P["batch"], P["heads"], P["seq_len"], P["head_dim"])
        outs = tuple(torch.empty(shape, dtype=torch.int8, device=dev) for _ in range(3))
    else:
        outs = torch.empty((P["rows"], P["out_features"]), dtype=torch.int8, device=dev)
    for _ in range(args.warmup):
        lin.forward(x, w, outs)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(args.steps):
            lin.forward(x, w, outs)
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    g0.record(stream)
    graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    kern_ms = g0.elapsed_time(g1) / args.steps
    M, K, Nc = P["rows"], P["in_features"], P["out_features"]
    ops = 2.0 * M * K * Nc
    tops = ops / (step_ms * 1e-3) / 1e12
    ktops = ops / (kern_ms * 1e-3) / 1e12
    hbm = float(M * K + Nc * K + M * Nc)
    res = {"metric": f"integer-only int8 linear TOPS, {lw.name}", "value": round(tops, 2),
           "unit": "TOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(step_ms, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "int8", "data": "synthetic (seeded int8 x and w)",
           "config": {"workload": lw.name, "rows": M, "in_features": K, "out_features": Nc,
                      "layout": "qkv_heads" if P["layout"] == 1 else "plain"},
           "kernel_us_mean": round(kern_ms * 1e3, 3),
           "roofline": {"bound": "mfma", "achieved": round(ktops, 1), "peak": MFMA_I8_PEAK_TOPS,
                        "unit": "TFLOP/s", "frac": round(ktops / MFMA_I8_PEAK_TOPS, 4),
                        "traffic": None, "algorithmic_bytes_per_launch": int(hbm),
                        "hbm_gbs_at_algorithmic_bytes": round(hbm / (kern_ms * 1e-3) / 1e9, 1)}}
    if not args.no_cpu:
        # the oracle on the first rows of the same x (every output column, each
        # (b, c) pair on its slice of W), a bounded sample of about 2 s
        import oracle
        rows = min(M, 1536)
        npairs = 3 if P["layout"] == 1 else 1
        width = Nc // npairs
        t1 = time.perf_counter()
        for i in range(npairs):
            oracle.linear(lw.x[:rows], lw.w[i * width:(i + 1) * width], P["b"][i], P["c"][i])
        cpu_s = time.perf_counter() - t1
        res["cpu_baseline"] = {"value": round(2.0 * rows * K * Nc / cpu_s / 1e12, 6),
                               "unit": "TOPS", "cores": 1, "kind": "oracle",
                               "sample": f"the first {rows} of {M} rows, all {Nc} output columns, "
                                         f"{cpu_s:.2f} s single-threaded C -O2 on {cpu_model()}"}
    lin.close()
    print(json.dumps(res), flush=True)


def bench_block(args):
    """Time ShiftGELU or I-LayerNorm on the ViT-B shapes (MLP activation
    25216 x 3072, LayerNorm input 25216 x 768); roofline against HBM."""
    import numpy as np
    import torch
    from integer_only_quantized_int8_amd import workloads as W
    from integer_only_quantized_int8_amd.iqattn import IQGelu, IQLayerNorm
    dev = torch.device("cuda:0")
    if args.block == "gelu":
        wl = W.gelu_workload("vitb_mlp_b128_n197_c3072")
        op = IQGelu(dict(wl.params, rows=wl.rows, cols=wl.cols))
        x = torch.from_numpy(wl.x).to(dev)
        out = torch.empty_like(x)
        run = lambda: op.forward(x, out)  # noqa: E731
        affine_bytes = 0
    else:
        wl = W.layernorm_workload("vitb_ln_b128_n197_c768")
        op = IQLayerNorm(dict(wl.params, rows=wl.rows, cols=wl.cols))
        x = torch.from_numpy(wl.x).to(dev)
        g = torch.from_numpy(wl.gamma).to(dev)
        b = torch.from_numpy(wl.beta).to(dev)
        out = torch.empty_like(x)
        run = lambda: op.forward(x, g, b, out)  # noqa: E731
        affine_bytes = 5 * wl.cols
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(args.steps):
            run()
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    g0.record(stream)
    graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    kern_ms = g0.elapsed_time(g1) / args.steps
    elems = wl.rows * wl.cols
    algo = float(2 * elems + affine_bytes)  # int8 in + int8 out (+ gamma, beta)
    gbs = algo / (kern_ms * 1e-3) / 1e9
    res = {"metric": f"integer-only {'ShiftGELU' if args.block == 'gelu' else 'I-LayerNorm'} "
                     f"Gelem/s, {wl.name}",
           "value": round(elems / (step_ms * 1e-3) / 1e9, 2), "unit": "Gelem/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
           "data": "synthetic (seeded int8 activations)",
           "config": {"workload": wl.name, "rows": wl.rows, "cols": wl.cols},
           "kernel_us_mean": round(kern_ms * 1e3, 3),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                        "algorithmic_bytes_per_launch": int(algo)}}
    if not args.no_cpu:
        import oracle
        t1 = time.perf_counter()
        if args.block == "gelu":
            oracle.shiftgelu(wl.x, wl.params)
        else:
            oracle.ilayernorm(wl.x, wl.gamma, wl.beta, wl.params)
        cpu_s = time.perf_counter() - t1
        res["cpu_baseline"] = {"value": round(elems / cpu_s / 1e9, 4), "unit": "Gelem/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"the whole {wl.rows} x {wl.cols} tensor, "
                                         f"{cpu_s:.2f} s single-threaded C -O2 on {cpu_model()}"}
    op.close()
    print(json.dumps(res), flush=True)


def bench_linattn(args):
    """Time the softmax-free integer linear attention on an EfficientViT-style
    shape; roofline against HBM (Q, K, V read once, Out written once)."""
    import torch
    from integer_only_quantized_int8_amd import workloads as W
    from integer_only_quantized_int8_amd.iqattn import IQLinAttn
    wl = W.linattn_workload(args.linattn)
    B, H, N, d = wl.q.shape
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(t).to(dev) for t in (wl.q, wl.k, wl.v))
    out = torch.empty_like(q)
    op = IQLinAttn(wl.q.shape, wl.params)
    for _ in range(args.warmup):
        op.forward(q, k, v, out)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(args.steps):
            op.forward(q, k, v, out)
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    g0.record(stream)
    graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    kern_ms = g0.elapsed_time(g1) / args.steps
    heads = B * H
    algo = float(4 * N * d * heads)
    ops = 4.0 * N * d * d * heads  # the two int8 contractions, 2 N d^2 each
    gbs = algo / (kern_ms * 1e-3) / 1e9
    res = {"metric": f"integer-only linear attention int8 TOPS, {wl.name}",
           "value": round(ops / (step_ms * 1e-3) / 1e12, 3), "unit": "TOPS", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
           "data": "synthetic (seeded int8 Q, K, V)",
           "config": {"workload": wl.name, "batch": B, "heads": H, "seq_len": N, "head_dim": d},
           "kernel_us_mean": round(kern_ms * 1e3, 3),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                        "algorithmic_bytes_per_launch": int(algo)}}
    if not args.no_cpu:
        import oracle
        passes, t1 = 0, time.perf_counter()
        while True:  # whole passes over every head, about 2 s of CPU time
            oracle.linattn(wl.q, wl.k, wl.v, wl.params)
            passes += 1
            cpu_s = time.perf_counter() - t1
            if cpu_s >= 2.0:
                break
        res["cpu_baseline"] = {"value": round(ops * passes / cpu_s / 1e12, 6),
                               "unit": "TOPS", "cores": 1, "kind": "oracle",
                               "sample": f"{passes} whole pass(es) over the {heads} heads, "
                                         f"{cpu_s:.2f} s single-threaded C -O2 on {cpu_model()}"}
    op.close()
    print(json.dumps(res), flush=True)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def workload_name(args) -> str:
    """Name of the benchmarked workload (the LIS shape with the MFMA engine
    carries an _mfma suffix)."""
    from integer_only_quantized_int8_amd import workloads as W
    name = W.CONFIGS[args.config]["name"]
    if args.lis_engine == 1:
        name += "_mfma"
    return name


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="workload shape 0..4 (2 = headline)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads timed on the CPU oracle (0 = all heads, at most ~30 s)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 256 MiB device copy (HBM counter calibration)")
    ap.add_argument("--linear", default=None,
                    help="time an int8 linear layer instead (workload name from "
                         "workloads.LINEAR_CONFIGS, e.g. vitb_qkv_b128_n197_c768)")
    ap.add_argument("--linattn", default=None,
                    help="time the softmax-free linear attention on this EfficientViT-style shape")
    ap.add_argument("--block", default=None, choices=("gelu", "layernorm"),
                    help="time ShiftGELU or I-LayerNorm on the ViT-B shapes instead")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 --pmc "
                         "counter files and exit (no GPU use)")
    ap.add_argument("--record-counters", metavar="PMC_CSV",
                    help="write profiles/counters_<workload>.json from a rocprofv3 --pmc file of "
                         "the unit counters (" + " ".join(UNIT_COUNTERS) + ") and exit")
    ap.add_argument("--lis-engine", type=int, default=None, choices=(0, 1),
                    help="P.V engine of the Log-Int-Softmax shape (0 VALU shift-add, 1 MFMA bit planes)")
    ap.add_argument("--cold-sets", type=int, default=5,
                    help="input sets rotated through the cold-cache timing (0 = skip)")
    args = ap.parse_args()

    if args.record_traffic or args.record_counters:
        name = workload_name(args)
        if args.record_traffic:
            rec = record_traffic(args.record_traffic[0], args.record_traffic[1], name)
            out = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
        else:
            rec = record_counters(args.record_counters, name)
            out = os.path.join(ROOT, "profiles", f"counters_{name}.json")
        os.makedirs(os.path.dirname(out), exist_ok=True)
        with open(out, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))
        return

    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (--gpus {args.gpus} requested); "
              "the path has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from integer_only_quantized_int8_amd import workloads as W
    from integer_only_quantized_int8_amd.iqattn import IQAttn

    if args.linear:
        bench_linear(args)
        return
    if args.block:
        bench_block(args)
        return
    if args.linattn:
        bench_linattn(args)
        return

    t0 = time.time()
    w = W.config_workload(args.config)
    if args.lis_engine is not None:
        w.params["lis_engine"] = args.lis_engine
    wname = workload_name(args)
    B, H, N, d = w.q.shape
    heads = B * H
    print(f"[bench] generated {w.name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(dev) for x in (w.q, w.k, w.v))
    out = torch.empty_like(q)
    att = IQAttn(w.q.shape, w.params)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        att.forward(q, k, v, out)
    torch.cuda.synchronize()

    # per-launch kernel duration: HIP events around single launches on the
    # launch stream (torch's current stream, which iqattn_forward uses)
    n_ev = min(args.steps, 50)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_ev)]
    for i in range(n_ev):
        ev[i][0].record(stream)
        att.forward(q, k, v, out)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    launch_ms = np.array([a.elapsed_time(b) for a, b in ev])

    # timed region: exactly K steps back to back, captured once in a HIP graph
    # (one kernel node per step) so that host launch latency does not gap them
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(args.steps):
            att.forward(q, k, v, out)
    graph.replay()  # untimed replay (graph upload)
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    g0.record(stream)
    graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step_ms = wall * 1e3 / args.steps
    graph_step_ms = g0.elapsed_time(g1) / args.steps
    # average launch duration of the kernel: HIP events over the timed region
    kern_ms = graph_step_ms
    del graph

    # cold caches: the same launches rotating over `cold_sets` copies of the
    # inputs and outputs (more bytes than the 256 MB Infinity Cache), so that
    # each launch reads its operands from HBM; reported beside the headline
    cold = None
    if args.cold_sets > 0:
        sets = [(q.clone(), k.clone(), v.clone(), torch.empty_like(out))
                for _ in range(args.cold_sets)]
        torch.cuda.synchronize()
        gc = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gc):
            for i in range(args.steps):
                cq, ck, cv, co = sets[i % len(sets)]
                att.forward(cq, ck, cv, co)
        gc.replay()
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        gc.replay()
        c1.record(stream)
        torch.cuda.synchronize()
        cold_ms = c0.elapsed_time(c1) / args.steps
        rot = len(sets) * 4 * q.numel()
        same_cold = all(torch.equal(s_[3], out) for s_ in sets)
        del gc, sets
        cold = {"input_sets": args.cold_sets, "bytes_in_rotation": int(rot),
                "kernel_us_mean": round(cold_ms * 1e3, 3), "outputs_equal_hot": bool(same_cold)}

    if args.copy_calib:
        src = torch.empty(COPY_CALIB_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    gpu_out = out.cpu().numpy()
    ops = 4.0 * N * N * d * heads
    alg_bytes = 4.0 * N * d * heads
    if w.params.get("rel_bias") is not None:
        alg_bytes += np.asarray(w.params["rel_bias"]).nbytes
    tops = ops / (step_ms * 1e-3) / 1e12
    achieved_gbs = alg_bytes / (kern_ms * 1e-3) / 1e9

    traffic = None
    trec = load_traffic(wname)
    if trec is not None:
        traffic = trec["hbm_bytes_per_launch"]
    crec = load_counters(wname)
    if cold is not None:
        cold_gbs = alg_bytes / (cold["kernel_us_mean"] * 1e-6) / 1e9
        cold.update({"achieved_gbs": round(cold_gbs, 1), "frac": round(cold_gbs / HBM_PEAK_GBS, 4)})

    result = {
        "metric": METRIC if args.config == 2 else f"integer-only MSA int8 TOPS, {w.name}",
        "value": round(tops, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded int8 Q/K/V, ViT-B/DeiT-B-shaped; no dataset or weights)",
        "config": {"workload": wname, "batch": B, "heads": H, "seq_len": N, "head_dim": d,
                   "variant": "lis" if w.params["variant"] == 1 else "shiftmax",
                   "seed": 1000 + args.config, "parallelism": "none (1 GPU)"},
        "kernel_us_mean": round(kern_ms * 1e3, 3),
        "single_launch_us_mean": round(float(launch_ms.mean()) * 1e3, 3),
        "single_launch_us_min": round(float(launch_ms.min()) * 1e3, 3),
        "heads_per_s": round(heads / (step_ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": int(alg_bytes),
                     "mfma_int8": {"achieved_tops": round(ops / (kern_ms * 1e-3) / 1e12, 2),
                                   "peak_tops": MFMA_I8_PEAK_TOPS,
                                   "frac": round(ops / (kern_ms * 1e-3) / 1e12 / MFMA_I8_PEAK_TOPS, 4)}},
    }
    # the third roofline, from the committed unit-counter record of these
    # sources: executed VALU instructions (MFMA excluded) x 64 lanes over the
    # live launch time, against 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
    hbm_frac = result["roofline"]["frac"]
    mfma_frac = result["roofline"]["mfma_int8"]["frac"]
    valu = None
    if crec is not None:
        lane_ops = crec["valu_insts_per_launch"] * 64.0
        valu_tops = lane_ops / (kern_ms * 1e-3) / 1e12
        valu = {"achieved_tops": round(valu_tops, 2), "peak_tops": round(VALU_LANE_PEAK_TOPS, 2),
                "frac": round(valu_tops / VALU_LANE_PEAK_TOPS, 4),
                "valu_insts_per_launch": crec["valu_insts_per_launch"],
                "counter_busy_share": crec["valu_busy_share"],
                "mfma_busy_share": crec["mfma_busy_share"],
                "source": f"profiles/counters_{wname}.json"}
        result["roofline"]["valu"] = valu
    fracs = {"hbm": hbm_frac, "mfma": mfma_frac}
    if valu is not None:
        fracs["valu"] = valu["frac"]
    result["roofline"]["busiest_unit"] = max(fracs, key=fracs.get)
    if cold is not None:
        result["cold_hbm"] = cold
    if w.params["variant"] == 1 and int(w.params.get("lis_engine", 0)) == 0:
        # the LIS BitShift P.V on the VALU: one shift-add per (query, key,
        # feature), N^2 d per head, bounds this launch (HBM and MFMA stay listed)
        shifts = float(N) * N * d * heads
        alu = shifts / (kern_ms * 1e-3) / 1e12
        hbm = result["roofline"]
        result["roofline"] = {
            "bound": "alu", "achieved": round(alu, 2), "peak": round(VALU_LANE_PEAK_TOPS, 2),
            "unit": "TOP/s", "frac": round(alu / VALU_LANE_PEAK_TOPS, 4), "traffic": traffic,
            "algorithmic_shift_adds_per_launch": int(shifts),
            "hbm": {"achieved_gbs": hbm["achieved"], "peak_gbs": HBM_PEAK_GBS, "frac": hbm["frac"],
                    "algorithmic_bytes_per_launch": hbm["algorithmic_bytes_per_launch"]},
            "mfma_int8": hbm["mfma_int8"], "busiest_unit": "alu"}
        if valu is not None:
            result["roofline"]["valu"] = valu

    if not args.no_cpu:
        import oracle
        if not os.path.exists(oracle.library_path()):
            oracle.build()
        # bounded sample: whole passes over the first n_cpu heads until at least
        # ~10 s of single-threaded oracle time (at most ~30 s)
        per_head_guess = 0.0025 * (N / 197.0) ** 2 * (d / 64.0)
        n_cpu = args.cpu_heads or min(heads, max(1, int(25.0 / per_head_guess)))
        print(f"[bench] CPU oracle on {n_cpu} heads ...", file=sys.stderr, flush=True)
        passes, cpu_s, same = 0, 0.0, True
        while passes == 0 or (cpu_s < 10.0 and cpu_s * (passes + 1) / passes < 30.0):
            t1 = time.perf_counter()
            ref = oracle.forward(w.q, w.k, w.v, w.params, heads=(0, n_cpu))
            cpu_s += time.perf_counter() - t1
            passes += 1
            same = same and bool(np.array_equal(gpu_out.reshape(heads, N, d)[:n_cpu], ref))
        done = n_cpu * passes
        result["cpu_baseline"] = {
            "value": round(4.0 * N * N * d * done / cpu_s / 1e12, 6), "unit": "TOPS",
            "cores": 1, "kind": "oracle",
            "sample": f"{passes} pass(es) over heads 0..{n_cpu - 1} of {w.name} "
                      f"(seed {1000 + args.config}), {cpu_s:.2f} s single-threaded C -O2 on "
                      f"{cpu_model()} (host nproc {os.cpu_count()})",
            "heads_per_s": round(done / cpu_s, 2)}
        result["bit_exact_vs_oracle"] = {"heads_compared": n_cpu, "equal": same}
    att.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
