"""Benchmark of the W4A16 GEMM on one MI355X.

Default workload ("decode7b"): the linear layers of one Llama-2-7B decode step
-- 32 layers x (o_proj 4096x4096, fused qkv 12288x4096, fused gate+up
22016x4096, down 4096x11008), g = 128, asymmetric -- at batch M in
{1, 4, 8, 16, 32}.  One step runs all of them: 5 x 32 x 4 = 640 GEMMs over
3.2 GB of distinct int4 weights (one seeded random weight per shape, copied
into 32 per-layer buffers on the device), so every GEMM reads its weights from
HBM and not from the 256 MB Infinity Cache.

Each (M, shape) block of 32 launches is captured once in a HIP graph and
replayed; events on the launch stream bracket every block, so the per-kernel
time is GPU time, free of host launch gaps.

Prints one JSON line (see the end of main()).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "W4A16 GEMM TFLOPS + HBM GB/s (% roofline), Llama-7B shapes, M=1..2048"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA
LAYERS = 32

WORKLOADS = {
    "decode7b": dict(shapes=workloads.LLAMA7B_SHAPES, ms=workloads.DECODE_M, outliers=False,
                     desc="Llama-2-7B linear layers x32, M in {1,4,8,16,32}, g=128 asym"),
    "prefill7b": dict(shapes=workloads.LLAMA7B_SHAPES, ms=workloads.PREFILL_M, outliers=True,
                      desc="Llama-2-7B linear layers x32, M in {64,128,256,512,2048}, "
                           "g=128 asym, 1% outlier columns x20"),
}


def alg_bytes(M, N, K, g, sym=False):
    G = -(-K // g)
    return N * K // 2 + 2 * N * G + (0 if sym else N * (-(-G // 2))) + 2 * M * K + 2 * M * N


def alg_flops(M, N, K):
    return 2 * M * N * K


SMALL_M_MAX = 64  # the library picks its small-M kernel up to this M


def kernel_name(M):
    return "gemm_small_m_kernel" if M <= SMALL_M_MAX else "gemm_large_m_kernel"


def cpu_baseline(wl, frac_rows, layers):
    """The CPU oracle, untuned, on a bounded sample: every (shape, M) of
    `layers` of the 32 layers (1 in `frac_rows` weight rows); reported in the
    step's unit."""
    import oracle
    t_total, bytes_total, flops_total = 0.0, 0, 0
    for name, (N, K) in wl["shapes"].items():
        c = workloads.draw(max(wl["ms"]), N, K, 128, False,
                           seed=workloads.shape_seed(wl["key"], N, K, 128, False),
                           outliers=wl["outliers"])
        qp, zp = oracle.pack(c.codes), oracle.pack(c.zeros)
        rows = np.arange(0, N, frac_rows, dtype=np.int64)
        G = -(-K // 128)
        R = rows.size
        for M in wl["ms"]:
            X = np.ascontiguousarray(c.X[:M])
            for _ in range(layers):
                t0 = time.perf_counter()
                oracle.gemm_rows(X, qp, c.scales, zp, K, 128, False, rows=rows)
                t_total += time.perf_counter() - t0
                bytes_total += R * (K // 2 + 2 * G + (-(-G // 2))) + 2 * M * K + 2 * M * R
                flops_total += 2 * M * R * K
    return t_total, bytes_total, flops_total, oracle.num_threads()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode7b", choices=sorted(WORKLOADS))
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="oracle runs 1 in this many weight rows (default: 1 decode, 64 prefill)")
    ap.add_argument("--cpu-layers", type=int, default=None,
                    help="layers of the step the oracle computes (default: 5 decode, 1 prefill)")
    ap.add_argument("--detail", action="store_true", help="print one line per (M, shape) on stderr")
    args = ap.parse_args()

    if args.cpu_sample is None:
        args.cpu_sample = 1 if args.workload == "decode7b" else 64
    if args.cpu_layers is None:
        args.cpu_layers = 5 if args.workload == "decode7b" else 1
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only: --gpus must be 1 "
                                   "(the multi-GPU sharding is a design note, not built)"}))
        sys.exit(2)

    import torch
    import weight_only_int4_02_amd as w4

    wl = dict(WORKLOADS[args.workload])
    wl["key"] = args.workload
    torch.cuda.set_device(0)
    w4.device_check()
    dev = torch.device("cuda:0")
    shapes = wl["shapes"]
    ms = wl["ms"]
    Mmax = max(ms)
    g = 128

    # ---- inputs: one seeded weight per shape, cloned into 32 layer buffers ----
    weights, xs, outs = {}, {}, {}
    for name, (N, K) in shapes.items():
        c = workloads.draw(Mmax, N, K, g, False,
                           seed=workloads.shape_seed(args.workload, N, K, g, False),
                           outliers=wl["outliers"])
        base = w4.quantized_weight(torch.from_numpy(c.codes).to(dev),
                                   torch.from_numpy(c.scales).to(dev),
                                   torch.from_numpy(c.zeros).to(dev), g)
        layers = [base] + [w4.PackedWeight(base.q.clone(), base.s.clone(), base.z.clone(),
                                           N, K, g, base.flags) for _ in range(LAYERS - 1)]
        weights[name] = layers
        xs[name] = torch.from_numpy(c.X).to(dev)
        for M in ms:
            outs[(M, name)] = [torch.empty((M, N), dtype=torch.float16, device=dev)
                               for _ in range(LAYERS)]
    torch.cuda.synchronize()

    cases = [(M, name) for M in ms for name in shapes]

    def run_block(M, name):
        X = xs[name][:M]
        for layer in range(LAYERS):
            w4.gemm(X, weights[name][layer], out=outs[(M, name)][layer])

    # eager reference outputs of layer 0 for the graph-replay check
    ref = {}
    for M, name in cases:
        w4.gemm(xs[name][:M], weights[name][0], out=outs[(M, name)][0])
        ref[(M, name)] = outs[(M, name)][0].clone()
    torch.cuda.synchronize()

    graphs = {}
    use_graph = not args.no_graph
    if use_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for M, name in cases:   # warm the launch path before capture
                run_block(M, name)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for M, name in cases:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                run_block(M, name)
            graphs[(M, name)] = gr
        torch.cuda.synchronize()

    def block(M, name):
        if use_graph:
            graphs[(M, name)].replay()
        else:
            run_block(M, name)

    for _ in range(args.warmup):
        for M, name in cases:
            block(M, name)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps ----
    stream = torch.cuda.current_stream()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(cases) + 1)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for st in range(args.steps):
        evs[st][0].record(stream)
        for ci, (M, name) in enumerate(cases):
            block(M, name)
            evs[st][ci + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    block_ms = np.zeros(len(cases))
    for st in range(args.steps):
        for ci in range(len(cases)):
            block_ms[ci] += evs[st][ci].elapsed_time(evs[st][ci + 1])
    block_ms /= args.steps
    step_ms = float(np.mean([evs[st][0].elapsed_time(evs[st][-1]) for st in range(args.steps)]))

    # replayed outputs equal the eager ones, bit for bit
    for M, name in cases:
        assert torch.equal(outs[(M, name)][0].view(torch.int16), ref[(M, name)].view(torch.int16)), \
            f"replayed output differs from eager output for M={M} {name}"

    step_bytes = sum(LAYERS * alg_bytes(M, *shapes[name], g) for M, name in cases)
    step_flops = sum(LAYERS * alg_flops(M, *shapes[name]) for M, name in cases)
    gbs = step_bytes / (step_ms * 1e-3) / 1e9
    tflops = step_flops / (step_ms * 1e-3) / 1e12

    # ---- roofline of the dominant kernel ----
    per_kernel = {}
    detail = []
    for ci, (M, name) in enumerate(cases):
        N, K = shapes[name]
        kn = kernel_name(M)
        b = LAYERS * alg_bytes(M, N, K, g)
        f = LAYERS * alg_flops(M, N, K)
        d = per_kernel.setdefault(kn, dict(ms=0.0, bytes=0, flops=0, launches=0))
        d["ms"] += block_ms[ci]
        d["bytes"] += b
        d["flops"] += f
        d["launches"] += LAYERS
        us = block_ms[ci] * 1e3 / LAYERS
        detail.append(dict(M=M, shape=name, N=N, K=K, us_per_gemm=round(us, 3),
                           gbs=round(b / LAYERS / (us * 1e-6) / 1e9, 1),
                           tflops=round(f / LAYERS / (us * 1e-6) / 1e12, 2)))
    dom = max(per_kernel, key=lambda k: per_kernel[k]["ms"])
    d = per_kernel[dom]
    avg_us = d["ms"] * 1e3 / d["launches"]
    if wl["key"] == "decode7b" or dom == "gemm_small_m_kernel":
        ach = d["bytes"] / (d["ms"] * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(ach / HBM_PEAK_GBS, 4), traffic=None)
    else:
        ach = d["flops"] / (d["ms"] * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(ach, 2), peak=MFMA_F16_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=round(ach / MFMA_F16_PEAK_TFLOPS, 4), traffic=None)
    roof["kernel"] = dom
    roof["avg_launch_us"] = round(avg_us, 3)
    roof["launches_per_step"] = d["launches"]

    if args.detail:
        for row in detail:
            print(json.dumps(row), file=sys.stderr)

    cpu = None
    if not args.no_cpu_baseline:
        t_cpu, b_cpu, f_cpu, cores = cpu_baseline(wl, args.cpu_sample, args.cpu_layers)
        if wl["key"] == "decode7b":
            cpu = dict(value=round(b_cpu / t_cpu / 1e9, 4), unit="GB/s")
        else:
            cpu = dict(value=round(f_cpu / t_cpu / 1e12, 6), unit="TFLOP/s")
        cpu.update(cores=cores, kind="oracle", seconds=round(t_cpu, 2),
                   sample=f"every (shape, M) of {args.cpu_layers} of the {LAYERS} layers of one step, "
                          f"1 in {args.cpu_sample} weight rows; fp64 C oracle, OpenMP")

    if wl["key"] == "decode7b":
        value, unit = gbs, "GB/s"
    else:
        value, unit = tflops, "TFLOP/s"
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{wl['key']}: {wl['desc']}", "layers": LAYERS,
                   "m": list(ms), "shapes": {k: list(v) for k, v in shapes.items()},
                   "group_size": g, "graphs": use_graph},
        "tflops": round(tflops, 3), "gbs": round(gbs, 1),
        "wall_s_timed": round(wall, 3),
        "roofline": roof, "cpu_baseline": cpu,
        "per_case": detail,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
