"""Benchmark of the W4A16 GEMM on one MI355X.

Default workload ("llama7b"): the linear layers of Llama-2-7B -- 32 layers x
(o_proj 4096x4096, fused qkv 12288x4096, fused gate+up 22016x4096, down
4096x11008), g = 128, asymmetric -- at every M of the metric: the decode
sweep M in {1, 4, 8, 16, 32} (memory-bound) and the prefill sweep M in
{64, 128, 256, 512, 2048} (compute-bound; 1 % of the activation columns
scaled x20 as outliers).  One step runs all of them: 10 x 32 x 4 = 1280
GEMMs over 3.4 GB of distinct int4 weights (one seeded random weight per
shape, copied into 32 per-layer buffers on the device, and per-layer copies
of the activations), so every GEMM reads its operands from HBM and not from
the 256 MB Infinity Cache.

The whole step is captured in one HIP graph; the timed region replays it K
times between events on the launch stream.  Per-(M, shape) times come from a
second pass (ROCm refuses timing events inside a graph): a graph per case
holding its block of 32 launches, replayed back to back between two events.
The cases' times sum to the step time within a fraction of a percent, and
the line reports both.

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
    # the metric's configuration: Llama-2-7B shapes, M = 1..2048
    "llama7b": dict(shapes=workloads.LLAMA7B_SHAPES, ms=workloads.DECODE_M + workloads.PREFILL_M,
                    outliers_from=64,
                    desc="Llama-2-7B linear layers x32, M in {1,4,8,16,32} (decode) and "
                         "{64,128,256,512,2048} (prefill, 1% outlier activation columns x20), "
                         "g=128 asym"),
    "decode7b": dict(shapes=workloads.LLAMA7B_SHAPES, ms=workloads.DECODE_M, outliers_from=None,
                     desc="Llama-2-7B linear layers x32, M in {1,4,8,16,32}, g=128 asym"),
    # the 70B-class GQA configuration (M in {1, 16, 128, 1024}), split by
    # regime: its HBM-bound and its MFMA-bound halves
    "decode70b": dict(shapes=workloads.LLAMA70B_SHAPES, ms=(1, 16), outliers_from=None,
                      desc="70B-class GQA linear layers x32 (fused qkv 10240x8192 with 8 KV "
                           "heads of dim 128, o_proj 8192x8192, fused gate+up 57344x8192, "
                           "down 8192x28672), M in {1,16}, g=128 asym"),
    "prefill70b": dict(shapes=workloads.LLAMA70B_SHAPES, ms=(128, 1024), outliers_from=None,
                       desc="70B-class GQA linear layers x32 (fused qkv 10240x8192 with 8 KV "
                            "heads of dim 128, o_proj 8192x8192, fused gate+up 57344x8192, "
                            "down 8192x28672), M in {128,1024}, g=128 asym"),
    "prefill7b": dict(shapes=workloads.LLAMA7B_SHAPES, ms=workloads.PREFILL_M, outliers_from=0,
                      desc="Llama-2-7B linear layers x32, M in {64,128,256,512,2048}, "
                           "g=128 asym, 1% outlier columns x20"),
    "decodestep7b": dict(shapes=workloads.LLAMA7B_SHAPES, ms=(1, 16), outliers_from=None,
                         desc="GEMM chain of a Llama-2-7B decode step, 32 layers: RMS norms, "
                              "fused q|k|v, o, fused gate|up, SiLU(gate)*up, down, residual adds "
                              "(attention itself not modelled: o reads the q slice), g=128 asym"),
    "quant7b": dict(shapes=workloads.LLAMA7B_SHAPES, ms=(), outliers_from=None,
                    desc="round-to-nearest quantization of the Llama-2-7B linear-layer "
                         "weights x32 (fp16 -> int4 codes, fp16 scales, int4 zeros), g=128 asym"),
}


def quant_alg_bytes(N, K, g):
    """fp16 W read; packed codes, fp16 scales and 4-bit zeros written."""
    G = -(-K // g)
    return 2 * N * K + N * K // 2 + 2 * N * G + N * (-(-G // 2))


def bench_decode_step(args, torch, w4):
    """tok/s proxy: one decode step of a Llama-2-7B-shaped stack of 32 layers
    built from QLinear modules (q, k, v fused into one launch, gate and up
    into another), the whole step captured in one HIP graph."""
    from weight_only_int4_02_amd.qlinear import QLinear, fuse
    wl = WORKLOADS["decodestep7b"]
    g = 128
    dev = torch.device("cuda:0")
    H, I = 4096, 11008
    parts = {"q": (H, H), "k": (H, H), "v": (H, H), "o": (H, H), "gate": (I, H),
             "up": (I, H), "down": (H, I)}
    base = {}
    for name, (N, K) in parts.items():
        c = workloads.draw(1, N, K, g, False,
                           seed=workloads.shape_seed("decodestep7b/" + name, N, K, g, False))
        base[name] = QLinear.from_codes(torch.from_numpy(c.codes).to(dev),
                                        torch.from_numpy(c.scales).to(dev),
                                        torch.from_numpy(c.zeros).to(dev), g)

    def clone(q):
        qp, sc, zp = q.canonical
        return QLinear(qp.clone(), sc.clone(), zp.clone(), q.K, q.g, keep_canonical=True)

    layers = []
    for layer in range(LAYERS):
        qkv = fuse([clone(base["q"]), clone(base["k"]), clone(base["v"])])
        gu = fuse([clone(base["gate"]), clone(base["up"])])
        for m in (qkv.fused, gu.fused):
            m.canonical = None
        o, down = clone(base["o"]), clone(base["down"])
        o.canonical = down.canonical = None
        layers.append((qkv, o, gu, down))
    del base
    torch.cuda.empty_cache()
    results = []
    for M in wl["ms"]:
        x0 = torch.from_numpy(workloads.draw(M, 16, H, g, False, seed=M).X).to(dev)
        h = torch.empty_like(x0)

        def rms(t):
            return (t.float() * torch.rsqrt(t.float().pow(2).mean(-1, keepdim=True) + 1e-6)).to(t.dtype)

        def step():
            h.copy_(x0)
            for qkv, o, gu, down in layers:
                q, _, _ = qkv(rms(h))
                h.add_(o(q.contiguous()))
                gate, up = gu(rms(h))
                h.add_(down(torch.nn.functional.silu(gate) * up))
                h.copy_(rms(h))   # keeps the random-weight activations finite
            return h

        step()
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=s):   # the warmed-up stream: its workspace is cached
            step()
        for _ in range(max(1, args.warmup)):
            gr.replay()
        torch.cuda.synchronize()
        ref = h.clone()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            gr.replay()
        e1.record()
        torch.cuda.synchronize()
        ms_step = e0.elapsed_time(e1) / args.steps
        assert torch.equal(h, ref), "graph replays are not deterministic"
        assert bool(torch.isfinite(h).all())
        # the same step's W4A16 launches alone (fixed inputs, no elementwise
        # work): how much of the step the int4 GEMMs take
        xa = rms(x0)
        xi = torch.nn.functional.silu(layers[0][2](xa)[0]).contiguous()

        def gemms():
            for qkv, o, gu, down in layers:
                qkv(xa)
                o(xa)
                gu(xa)
                down(xi)

        with torch.cuda.stream(s):
            gemms()
        torch.cuda.synchronize()
        gr2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr2, stream=s):
            gemms()
        gr2.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            gr2.replay()
        e1.record()
        torch.cuda.synchronize()
        ms_gemm = e0.elapsed_time(e1) / args.steps
        gemm_bytes = LAYERS * (alg_bytes(M, 3 * H, H, g) + alg_bytes(M, H, H, g) +
                               alg_bytes(M, 2 * I, H, g) + alg_bytes(M, H, I, g))
        results.append(dict(M=M, ms_per_step=round(ms_step, 4),
                            tok_per_s=round(M / (ms_step * 1e-3), 1),
                            gemm_ms_per_step=round(ms_gemm, 4),
                            gemm_only_tok_per_s=round(M / (ms_gemm * 1e-3), 1),
                            gemm_gbs=round(gemm_bytes / (ms_gemm * 1e-3) / 1e9, 1),
                            w4a16_launches_per_step=LAYERS * 4))
    main_r = results[0]
    line = {
        "metric": "decode-step tok/s proxy (GEMM chain, attention not modelled)",
        "value": main_r["tok_per_s"], "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": main_r["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"decodestep7b: {wl['desc']}", "layers": LAYERS,
                   "batch": [r["M"] for r in results], "group_size": g},
        "per_batch": results,
    }
    print(json.dumps(line))


def bench_quant(args, torch, w4):
    """The quantizer over one model's worth of linear-layer weights: 32
    distinct fp16 copies per shape (12.9 GB), one w4a16_quantize per layer
    and shape; a step quantizes all 128."""
    wl = WORKLOADS["quant7b"]
    shapes = wl["shapes"]
    g = 128
    dev = torch.device("cuda:0")
    Ws, outs = {}, {}
    for name, (N, K) in shapes.items():
        W = torch.from_numpy(workloads.draw_weight(N, K, "outliers",
                                                   seed=workloads.shape_seed("quant7b", N, K, g,
                                                                             False))).to(dev)
        Ws[name] = [W] + [W.clone() for _ in range(LAYERS - 1)]
        G = -(-K // g)
        outs[name] = [(torch.empty((N, K // 8), dtype=torch.int32, device=dev),
                       torch.empty((N, G), dtype=torch.float16, device=dev),
                       torch.empty((N, -(-G // 8)), dtype=torch.int32, device=dev))
                      for _ in range(LAYERS)]
    torch.cuda.synchronize()
    def run(name):
        for layer in range(LAYERS):
            w4.quantize(Ws[name][layer], g, out=outs[name][layer])

    for _ in range(max(1, args.warmup)):
        for name in shapes:
            run(name)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    names = list(shapes)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for st in range(args.steps):
        evs[st][0].record(stream)
        for ci, name in enumerate(names):
            run(name)
            evs[st][ci + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    blk = np.zeros(len(names))
    for st in range(args.steps):
        for ci in range(len(names)):
            blk[ci] += evs[st][ci].elapsed_time(evs[st][ci + 1])
    blk /= args.steps
    step_ms = float(np.mean([evs[st][0].elapsed_time(evs[st][-1]) for st in range(args.steps)]))
    step_bytes = sum(LAYERS * quant_alg_bytes(*shapes[n], g) for n in names)
    gbs = step_bytes / (step_ms * 1e-3) / 1e9
    detail = [dict(shape=n, N=shapes[n][0], K=shapes[n][1],
                   us_per_call=round(blk[ci] * 1e3 / LAYERS, 3),
                   gbs=round(quant_alg_bytes(*shapes[n], g) / (blk[ci] * 1e-3 / LAYERS) / 1e9, 1))
              for ci, n in enumerate(names)]
    # the outputs of the last step equal the oracle's on sampled rows
    import oracle
    n0 = names[0]
    N, K = shapes[n0]
    rows = np.arange(0, N, 97)
    Wh = Ws[n0][LAYERS - 1][rows].cpu().numpy()
    codes, s_ref, z_ref = oracle.quantize(Wh, g, False)
    q, sc, z = outs[n0][LAYERS - 1]
    assert np.array_equal(q[rows].cpu().numpy().view(np.uint32), oracle.pack(codes))
    assert np.array_equal(sc[rows].cpu().numpy().view(np.uint16), s_ref.view(np.uint16))
    assert np.array_equal(z[rows].cpu().numpy().view(np.uint32), oracle.pack(z_ref))

    cpu = None
    if not args.no_cpu_baseline:
        t_cpu, b_cpu = 0.0, 0
        cpu_layers = 4
        for n in names:
            N, K = shapes[n]
            for layer in range(cpu_layers):
                Wh = Ws[n][layer].cpu().numpy()
                t1 = time.perf_counter()
                oracle.quantize(Wh, g, False)
                t_cpu += time.perf_counter() - t1
                b_cpu += quant_alg_bytes(N, K, g)
        cpu = dict(value=round(b_cpu / t_cpu / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                   seconds=round(t_cpu, 2),
                   sample=f"every weight row of each shape, {cpu_layers} of the {LAYERS} layers; "
                          "C oracle, one thread")
    roof = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None, kernel="quantize (quantize_kernel)",
                avg_launch_us=round(step_ms * 1e3 / (LAYERS * len(names)), 3),
                launches_per_step=LAYERS * len(names),
                achieved_is="algorithmic bytes of all its launches / their summed event time")
    tr = load_traffic("quantize", "quant7b")
    if tr is not None:
        roof["traffic"] = tr["traffic_bytes_per_launch"]
        roof["alg_bytes_per_launch"] = tr["alg_bytes_per_launch"]
    line = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"quant7b: {wl['desc']}", "layers": LAYERS,
                   "shapes": {k: list(v) for k, v in shapes.items()}, "group_size": g},
        "wall_s_timed": round(wall, 3), "roofline": roof, "cpu_baseline": cpu,
        "per_case": detail,
    }
    print(json.dumps(line))


def alg_bytes(M, N, K, g, sym=False):
    G = -(-K // g)
    return N * K // 2 + 2 * N * G + (0 if sym else N * (-(-G // 2))) + 2 * M * K + 2 * M * N


def alg_flops(M, N, K):
    return 2 * M * N * K



# One w4a16 call runs one main kernel and, where K is split across
# workgroups, the reduce kernel after it.  Per-call times and traffic are
# those of the whole call: the main kernels' dispatches count the calls, and
# the reduce kernel's time and bytes are added to them.
KERNEL_GROUPS = {
    "gemm_small_m": (("gemm_small_m_kernel", "gemm_small_m_lds_kernel"), "splitk_reduce_kernel"),
    "gemm_large_m": (("gemm_large_m_kernel",), "splitk_reduce_kernel"),
    "quantize": (("quantize_kernel",), None),
}
# the kernel groups a workload's calls run (summaries are written per group)
WORKLOAD_GROUPS = {"llama7b": ("gemm_small_m", "gemm_large_m"),
                   "decode7b": ("gemm_small_m",), "prefill7b": ("gemm_large_m",),
                   "quant7b": ("quantize",),
                   "decode70b": ("gemm_small_m",), "prefill70b": ("gemm_large_m",)}
# oracle rows timed by default: every weight row at M <= 32, 1 in CPU_SAMPLE
# rows above, over CPU_LAYERS layers -- about 10-20 s of CPU work on 16 cores
CPU_SAMPLE = {"llama7b": 8, "prefill7b": 4, "prefill70b": 16}
CPU_LAYERS = {"decode7b": 5, "decode70b": 3}


def kernel_name(M, N, K, dtype="f16", g=128):
    """The kernel group the library runs for this call (its own plan, asked
    through w4a16_gemm_kernel)."""
    import weight_only_int4_02_amd as w4
    path, _ = w4.gemm_kernel(M, N, K, g, w4.BF16 if dtype == "bf16" else 0)
    return "gemm_" + path


def group_role(group, name):
    """'main', 'reduce' or None for a kernel name in a profiler record."""
    import re
    mains, red = KERNEL_GROUPS[group]

    def hit(k):
        return re.search(r"(?:^|\W)" + k + r"(?:<|\(|$)", name) is not None
    if any(hit(m) for m in mains):
        return "main"
    if red and hit(red):
        return "reduce"
    return None


# ---------------------------------------------------------------------------
# HBM traffic from rocprofv3 counters.  Two counter runs of this same bench
# (FETCH_SIZE, then WRITE_SIZE, both KiB per dispatch) with --copy-calibration,
# which first runs a device-to-device copy of COPY_MIB MiB: the counters'
# reading for that copy (COPY_MIB MiB read, COPY_MIB MiB written) gives the
# scale factor from counter KiB to bytes.  --pmc-summary turns the two runs
# into a text summary under profiles/ that carries the digest of the kernel
# sources; the bench reports `traffic` only while the sources still match.
# ---------------------------------------------------------------------------
COPY_MIB = 1024  # larger than twice any other copy the workloads make (weight clones)
KERNEL_SOURCES = ("include", "weight_only_int4_02_amd/csrc")


def kernel_source_digest():
    import hashlib
    h = hashlib.sha256()
    for d in KERNEL_SOURCES:
        base = os.path.join(ROOT, d)
        for fn in sorted(os.listdir(base)):
            if fn.endswith((".h", ".hpp", ".hip", ".cpp", ".inc")):
                h.update(fn.encode())
                with open(os.path.join(base, fn), "rb") as f:
                    h.update(f.read())
    return h.hexdigest()[:16]


def profile_tag(workload, dtype):
    return workload + ("_bf16" if dtype == "bf16" else "")


def traffic_summary_path(group, tag):
    return os.path.join(ROOT, "profiles", f"hbm_traffic_{group}_{tag}.txt")


def load_traffic(group, tag):
    """Measured HBM bytes per call of the kernel group, or None when no
    summary exists or the kernel sources changed since the counters were
    taken."""
    path = traffic_summary_path(group, tag)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if line.startswith("data: "):
                rec = json.loads(line[6:])
                if rec.get("source_digest") == kernel_source_digest():
                    return rec
    return None


def _read_counters(csv_dir):
    """{kernel name: [counter value per dispatch]} from a rocprofv3 counter
    collection CSV (one row per dispatch and counter)."""
    import csv
    import glob
    files = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {csv_dir}")
    per = {}
    for fn in files:
        with open(fn, newline="") as f:
            rd = csv.DictReader(f)
            col = {}
            for want in ("kernel_name", "dispatch_id", "counter_name", "counter_value"):
                hits = [c for c in rd.fieldnames if c.lower().replace(" ", "_") == want]
                if not hits:
                    raise SystemExit(f"{fn}: no column {want} in {rd.fieldnames}")
                col[want] = hits[0]
            for row in rd:
                key = (row[col["dispatch_id"]], row[col["counter_name"]])
                d = per.setdefault(row[col["kernel_name"]], {})
                d[key] = d.get(key, 0.0) + float(row[col["counter_value"]])
    return {k: list(v.values()) for k, v in per.items()}


def pmc_summary(fetch_dir, write_dir, workload, dtype, commands):
    """Writes profiles/hbm_traffic_<group>_<workload>.txt from the two runs,
    one file per kernel group the workload runs."""
    fetch, write = _read_counters(fetch_dir), _read_counters(write_dir)
    for group in WORKLOAD_GROUPS[workload]:
        _pmc_summary_group(fetch, write, workload, dtype, commands, group)


def _pmc_summary_group(fetch, write, workload, dtype, commands, group):
    tag = profile_tag(workload, dtype)

    def per_call(d):
        calls = sum(len(vs) for k, vs in d.items() if group_role(group, k) == "main")
        if not calls:
            raise SystemExit(f"no {group} kernel in the counter CSV")
        total = sum(sum(vs) for k, vs in d.items() if group_role(group, k) is not None)
        red = sum(len(vs) for k, vs in d.items() if group_role(group, k) == "reduce")
        return total / calls, calls, red

    def copy_reading(d):
        # the calibration copies are the largest copy dispatches of the run
        # (every weight clone of the workloads is under half of COPY_MIB)
        vals = [v for k, vs in d.items() if "copy" in k.lower() and "w4a16" not in k for v in vs]
        if not vals:
            raise SystemExit("no copy kernel in the counter CSV (run with --copy-calibration)")
        top = max(vals)
        return float(np.mean([v for v in vals if v >= 0.9 * top]))

    copy_f, copy_w = copy_reading(fetch), copy_reading(write)
    kf, nf, rf = per_call(fetch)
    kw, nw, rw = per_call(write)
    copy_bytes = COPY_MIB << 20
    fac_f = copy_bytes / (copy_f * 1024)
    fac_w = copy_bytes / (copy_w * 1024)
    wl = WORKLOADS[workload]
    shapes = wl["shapes"]
    if group == "quantize":
        alg = float(np.mean([quant_alg_bytes(*shapes[n], 128) for n in shapes]))
    else:
        cases = [(M, n) for M in wl["ms"] for n in shapes
                 if kernel_name(M, *shapes[n], dtype) == group]
        alg = float(np.mean([alg_bytes(M, *shapes[n], 128) for M, n in cases]))
    traffic = kf * 1024 * fac_f + kw * 1024 * fac_w
    rec = dict(kernel=group, workload=workload, dtype=dtype, source_digest=kernel_source_digest(),
               fetch_kib_per_call=round(kf, 1), write_kib_per_call=round(kw, 1),
               calls=[nf, nw], reduce_dispatches=[rf, rw], copy_mib=COPY_MIB,
               copy_fetch_kib=round(copy_f, 1),
               copy_write_kib=round(copy_w, 1), fetch_factor=round(fac_f, 4),
               write_factor=round(fac_w, 4), traffic_bytes_per_launch=round(traffic),
               alg_bytes_per_launch=round(alg), traffic_over_alg=round(traffic / alg, 4))
    mains, red = KERNEL_GROUPS[group]
    lines = [f"# HBM traffic of one {group} call ({' / '.join(mains)}"
             + (f", + {red} where K is split" if red else "") + f") -- workload {tag}", "",
             "Commands (repository root, MI355X):", ""]
    lines += ["    " + c for c in commands]
    lines += ["",
              f"Counter KiB per call: the counters of every {group} dispatch of the run"
              + (f" (and of its {red} dispatches)" if red else ""),
              f"summed and divided by the number of calls (FETCH_SIZE run: {nf} calls, "
              f"{rf} reduce dispatches; WRITE_SIZE run: {nw} calls, {rw} reduce dispatches):",
              f"    FETCH_SIZE {kf:.1f} KiB    WRITE_SIZE {kw:.1f} KiB", "",
              f"Calibration: a {COPY_MIB} MiB device-to-device copy reads {copy_f:.1f} KiB "
              f"(FETCH_SIZE) and writes {copy_w:.1f} KiB (WRITE_SIZE) by the counters",
              f"for {COPY_MIB * 1024} KiB each way: factors {fac_f:.4f} (read), {fac_w:.4f} (write).", "",
              f"Scaled HBM bytes per launch: {traffic / 1e6:.3f} MB against "
              f"{alg / 1e6:.3f} MB algorithmic (ratio {traffic / alg:.4f}).", "",
              "data: " + json.dumps(rec)]
    path = traffic_summary_path(group, tag)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)
    print(json.dumps(rec))


def _read_stats(stats_dir):
    """Rows of a rocprofv3 --stats kernel statistics CSV: (name, calls,
    total ns, average ns, min ns, max ns)."""
    import csv
    import glob
    files = glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *kernel_stats.csv under {stats_dir}")
    rows = []
    with open(max(files, key=os.path.getmtime), newline="") as f:
        rd = csv.DictReader(f)
        for r in rd:
            rows.append((r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]),
                         float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"])))
    rows.sort(key=lambda r: -r[2])
    return rows


def prof_summary(stats_dir, bench_log, workload, dtype, commands, plain_log=None):
    """Writes profiles/<group>_<workload>.txt from a rocprofv3 --kernel-trace
    --stats run of the bench, one file per kernel group the workload runs:
    the profiler's kernel table, the group's per-call time from it, and the
    bench's own per-call time of the same run (HIP events) for comparison."""
    rows = _read_stats(stats_dir)
    for group in WORKLOAD_GROUPS[workload]:
        _prof_summary_group(rows, bench_log, workload, dtype, commands, plain_log, group)


def _group_roofline(line, group):
    """The bench line's roofline object of one kernel group."""
    by = line.get("roofline_by_kernel") or {}
    if group in by:
        return by[group]
    return line["roofline"]


def _prof_summary_group(rows, bench_log, workload, dtype, commands, plain_log, group):
    tag = profile_tag(workload, dtype)
    calls = sum(r[1] for r in rows if group_role(group, r[0]) == "main")
    total_ns = sum(r[2] for r in rows if group_role(group, r[0]) is not None)
    red_calls = sum(r[1] for r in rows if group_role(group, r[0]) == "reduce")
    all_ns = sum(r[2] for r in rows)
    bench = None
    with open(bench_log) as f:
        for line in f:
            if line.startswith('{"metric"'):
                bench = json.loads(line)
    if bench is None:
        raise SystemExit(f"no bench line in {bench_log}")
    roof = _group_roofline(bench, group)
    plain = None
    if plain_log:
        with open(plain_log) as f:
            for line in f:
                if line.startswith('{"metric"'):
                    plain = json.loads(line)
    mains, red = KERNEL_GROUPS[group]
    per_call_us = total_ns / calls / 1e3
    lines = [f"# {group} ({' / '.join(mains)}" + (f", + {red} where K is split" if red else "")
             + f") -- workload {tag}", "", "Commands (repository root, MI355X):", ""]
    lines += ["    " + c for c in commands]
    lines += ["", "rocprofv3 kernel statistics (kernel_stats.csv), the 14 kernels with the most time:",
              "", "    Name | Calls | TotalNs | AverageNs | MinNs | MaxNs | Percentage"]
    for name, c, tot, avg, mn, mx in rows[:14]:
        lines.append(f"    {name[:110]} | {c} | {tot:.0f} | {avg:.1f} | {mn:.0f} | {mx:.0f} | "
                     f"{100 * tot / all_ns:.2f}")
    lines += ["",
              f"{group} calls: {calls} (dispatches of {' / '.join(mains)})"
              + (f"; {red} dispatches: {red_calls}" if red else "") + ".",
              f"Profiler time per call (all of the group's kernel time / calls): {per_call_us:.3f} us.",
              f"The bench in the same run (HIP events on the launch stream around graph replays "
              f"of each case): {roof['avg_launch_us']:.3f} us per call ({roof['kernel']}).",
              f"Bench line of the run: value {bench['value']} {bench['unit']}, roofline "
              f"{roof['achieved']} {roof['unit']} = frac {roof['frac']}.",
              "(The profiler adds time around short graph-launched kernels, which the bench's "
              "events see.)"]
    if plain is not None:
        pr = _group_roofline(plain, group)
        lines += [f"The same bench without the profiler (the second command, {plain['steps']} steps, same box): "
                  f"{pr['avg_launch_us']:.3f} us per call, {abs(pr['avg_launch_us'] - per_call_us) / per_call_us * 100:.1f} % "
                  f"from the profiler's kernel time; value {plain['value']} {plain['unit']}, "
                  f"roofline frac {pr['frac']}."]
    lines += ["",
              "data: " + json.dumps(dict(group=group, workload=workload, dtype=dtype,
                                         source_digest=kernel_source_digest(), calls=calls,
                                         reduce_dispatches=red_calls,
                                         profiler_us_per_call=round(per_call_us, 3),
                                         bench_us_per_call=roof["avg_launch_us"],
                                         plain_bench_us_per_call=(plain or {}).get("roofline", {}).get("avg_launch_us"),
                                         bench_value=bench["value"], bench_unit=bench["unit"]))]
    path = os.path.join(ROOT, "profiles", f"{group}_{tag}.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


def cpu_rows(wl_key, M, N, sample):
    """Weight rows the oracle computes for a case: all of them at M <= 32,
    1 in `sample` above."""
    return np.arange(0, N, 1 if M <= 32 else sample, dtype=np.int64)


def cpu_baseline(host, wl, sample, layers, dtype="f16"):
    """The CPU oracle, untuned, on a bounded sample: every (shape, M) of the
    step for `layers` layers, on the rows cpu_rows() names.  Returns (seconds,
    algorithmic bytes, flops, threads, {(M, shape): (rows, y_ref, wnorm2)} of
    layer 0) -- the last for the parity check of the run."""
    import oracle
    t_total, bytes_total, flops_total = 0.0, 0, 0
    refs = {}
    gemm = oracle.gemm_rows_bf16 if dtype == "bf16" else oracle.gemm_rows
    for name, (N, K) in wl["shapes"].items():
        h = host[name]
        G = -(-K // 128)
        for M in wl["ms"]:
            rows = cpu_rows(wl["key"], M, N, sample)
            R = rows.size
            X = np.ascontiguousarray(h["X"][uses_outliers(wl, M)][:M])
            for layer in range(layers):
                t0 = time.perf_counter()
                y_ref, wn2 = gemm(X, h["qp"], h["scales"], h["zp"], K, 128, False, rows=rows)
                t_total += time.perf_counter() - t0
                if layer == 0:
                    refs[(M, name)] = (rows, y_ref, wn2)
                bytes_total += R * (K // 2 + 2 * G + (-(-G // 2))) + 2 * M * K + 2 * M * R
                flops_total += 2 * M * R * K
    return t_total, bytes_total, flops_total, oracle.num_threads(), refs


def cpu_single_thread(host, wl, dtype="f16"):
    """The oracle on one thread: the tiny configuration (M=4, K=N=512, g=128,
    seed 0) and the first shape of the workload at M=1, all rows; best of 3."""
    import oracle
    out = {}
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        c = workloads.tiny_case()
        cases = [("tiny M=4 N=512 K=512", c.X, oracle.pack(c.codes), c.scales,
                  oracle.pack(c.zeros), 512, 512, 4)]
        name = next(iter(wl["shapes"]))
        N, K = wl["shapes"][name]
        if dtype == "f16":
            h = host[name]
            cases.append((f"{name} M=1 N={N} K={K}", np.ascontiguousarray(h["X"][False][:1]),
                          h["qp"], h["scales"], h["zp"], N, K, 1))
        for label, X, qp, sc, zp, N, K, M in cases:
            best = float("inf")
            for _ in range(3):
                t0 = time.perf_counter()
                oracle.gemm_rows(X, qp, sc, zp, K, 128, False)
                best = min(best, time.perf_counter() - t0)
            out[label] = dict(seconds=round(best, 5),
                              gflops=round(2 * M * N * K / best / 1e9, 3))
    finally:
        oracle.set_num_threads(threads)
    return out


def parity_of_run(refs, outs, xs_of, dtype, torch):
    """The run's own outputs (layer 0 of every case) against the oracle on
    the rows the CPU baseline computed: the error bound's worst ratio, and the
    diagnostic max |y - y_ref| / (||x_m|| ||w_n||)."""
    import oracle
    worst, diag, n = 0.0, 0.0, 0
    ok_all = True
    for (M, name), (rows, y_ref, wn2) in refs.items():
        y = outs[(M, name)][0][:, torch.from_numpy(rows).to(outs[(M, name)][0].device)]
        yb = y.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
        xb = xs_of(M, name)[:M].contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
        if dtype == "bf16":
            ok, w = oracle.check_y_bf16(yb, xb, y_ref, wn2)
            yv, xv = oracle.bf16_bits_to_f64_array(yb), oracle.bf16_bits_to_f64_array(xb)
        else:
            ok, w = oracle.check_y(yb.view(np.float16), xb.view(np.float16), y_ref, wn2)
            yv, xv = yb.view(np.float16).astype(np.float64), xb.view(np.float16).astype(np.float64)
        xn = np.sqrt((xv ** 2).sum(1))
        rel = np.abs(yv - y_ref) / np.maximum(xn[:, None] * np.sqrt(wn2)[None, :], 1e-300)
        ok_all &= ok
        worst = max(worst, w)
        diag = max(diag, float(rel.max()) if rel.size else 0.0)
        n += y_ref.size
    return dict(ok=bool(ok_all), outputs_checked=int(n), worst_err_over_bound=round(worst, 4),
                max_err_over_norms=float("%.3g" % diag),
                what="layer 0 of every (M, shape), the CPU baseline's rows, against the oracle")


def _sysfs_card(torch):
    """The sysfs device directory of cuda:0 (matched by PCI bus id), or None."""
    import glob
    try:
        props = torch.cuda.get_device_properties(0)
        bus = "%04x:%02x:%02x" % (getattr(props, "pci_domain_id", 0), props.pci_bus_id,
                                  props.pci_device_id)
    except Exception:
        bus = None
    cards = [d for d in glob.glob("/sys/class/drm/card*/device") if
             os.path.exists(os.path.join(d, "pp_dpm_sclk"))]
    if bus:
        for d in cards:
            if os.path.basename(os.path.realpath(d)).startswith(bus):
                return d
    return cards[0] if len(cards) == 1 else None


class ClockSampler:
    """Reads the current shader and memory clock levels from sysfs every
    `period` seconds on a thread of its own while the timed region runs (a
    file read: no child process, nothing that touches the GPU)."""

    def __init__(self, torch, period=0.02):
        import threading
        self.dir = _sysfs_card(torch)
        self.period = period
        self.samples = {"sclk": [], "mclk": []}
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _current(path):
        with open(path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    return int("".join(ch for ch in line.split(":")[1] if ch.isdigit()))
        return None

    def _run(self):
        while not self._stop.is_set():
            for k in ("sclk", "mclk"):
                try:
                    v = self._current(os.path.join(self.dir, f"pp_dpm_{k}"))
                except Exception:
                    v = None
                if v is not None:
                    self.samples[k].append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.dir:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self.dir:
            self._stop.set()
            self._thread.join()

    def summary(self):
        if not self.dir:
            return None
        out = {"source": os.path.realpath(self.dir) + "/pp_dpm_{sclk,mclk} (level marked *)",
               "period_s": self.period}
        for k, v in self.samples.items():
            if v:
                out[k + "_mhz"] = dict(samples=len(v), min=min(v), median=float(np.median(v)),
                                       max=max(v))
        return out


def read_clocks():
    """Current shader and memory clocks as rocm-smi reports them (a child
    process, after the timed region), or None where it is unavailable."""
    import shutil
    import subprocess
    # Under a profiler every child process inherits its preloaded library,
    # which initialises the GPU before rocm-smi's launcher re-executes
    # itself: no child is started there.
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or \
            any(k.startswith("ROCPROF") for k in os.environ):
        return None
    exe = shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi"
    try:
        r = subprocess.run([exe, "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=30)
        data = json.loads(r.stdout[r.stdout.index("{"):])
    except Exception:
        return None
    out = {}
    for card, vals in data.items():
        if isinstance(vals, dict):
            for k, v in vals.items():
                if any(c in k.lower() for c in ("sclk", "mclk", "fclk")):
                    out[f"{card} {k.strip().rstrip(':')}"] = v
    return out or None



def bf16_tensor(torch, bits, dev):
    """bfloat16 bit patterns (uint16 numpy) -> device bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def fp16_context(torch, w4, shapes, ms, canon, xs_of, detail, args):
    """torch.matmul in fp16 (the vendor GEMM) on each layer's dequantized
    weight, timed like the W4A16 blocks (a graph per (M, shape) block of 32
    launches when graphs are on).  Context only: the W4A16 speedup over fp16
    weights on the same shapes."""
    by_case = {(r["M"], r["shape"]): r for r in detail}
    out = {}
    total_w4 = total_16 = 0.0
    for name, (N, K) in shapes.items():
        qp, sc, zp = canon[name]
        W0 = w4.dequant(qp, sc, zp, K, 128)
        w16 = [W0] + [W0.clone() for _ in range(LAYERS - 1)]
        for M in ms:
            X = xs_of(M, name)[:M]
            ys = [torch.empty((M, N), dtype=torch.float16, device=X.device) for _ in range(LAYERS)]

            def run():
                for layer in range(LAYERS):
                    torch.matmul(X, w16[layer].t(), out=ys[layer])
            run()
            torch.cuda.synchronize()
            if not args.no_graph:
                gr = torch.cuda.CUDAGraph()
                s = torch.cuda.Stream()
                s.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(s):
                    run()
                torch.cuda.current_stream().wait_stream(s)
                with torch.cuda.graph(gr):
                    run()
                fn = gr.replay
            else:
                fn = run
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            reps = max(1, min(args.steps, 10))
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            us16 = e0.elapsed_time(e1) * 1e3 / reps / LAYERS
            usw4 = by_case[(M, name)]["us_per_gemm"]
            total_w4 += usw4
            total_16 += us16
            out[f"M{M}/{name}"] = dict(fp16_us=round(us16, 3), w4a16_us=usw4,
                                       speedup=round(us16 / usw4, 3))
        del w16
        torch.cuda.empty_cache()
    return dict(cases=out, step_speedup=round(total_16 / total_w4, 3),
                note="fp16 weights = the dequantized int4 weights; torch.matmul (hipBLASLt/rocBLAS)")


def uses_outliers(wl, M):
    """Whether the activations of batch M carry the x20 outlier columns."""
    return wl["outliers_from"] is not None and M >= wl["outliers_from"]


def build_inputs(torch, w4, wl, dtype, want_canon):
    """Device inputs of a GEMM workload: per shape one seeded weight cloned
    into LAYERS layer buffers, and per activation kind (plain, outliers) one
    seeded X at the largest M that uses it, cloned per layer.  Also the host
    copies the oracle needs."""
    dev = torch.device("cuda:0")
    g = 128
    weights, xs, host, canon = {}, {}, {}, {}
    for name, (N, K) in wl["shapes"].items():
        seed = workloads.shape_seed(wl["key"], N, K, g, False)
        if dtype == "bf16":
            c = workloads.draw_bf16(1, N, K, g, False, seed=seed)
            scales = bf16_tensor(torch, c.scales, dev)
        else:
            c = workloads.draw(1, N, K, g, False, seed=seed)
            scales = torch.from_numpy(c.scales).to(dev)
        codes = torch.from_numpy(c.codes).to(dev)
        zeros = torch.from_numpy(c.zeros).to(dev)
        base = w4.quantized_weight(codes, scales, zeros, g)
        if want_canon:
            canon[name] = (w4.pack(codes), scales, w4.pack(zeros))
        del codes
        import oracle
        h = dict(qp=oracle.pack(c.codes), zp=oracle.pack(c.zeros), scales=c.scales, X={})
        weights[name] = [base] + [w4.PackedWeight(base.q.clone(), base.s.clone(), base.z.clone(),
                                                  N, K, g, base.flags) for _ in range(LAYERS - 1)]
        for out in (False, True):
            mx = [M for M in wl["ms"] if uses_outliers(wl, M) == out]
            if not mx:
                continue
            xseed = workloads.shape_seed(wl["key"] + ("/x-outliers" if out else "/x"), N, K, g,
                                         False)
            if dtype == "bf16":
                xh = workloads.draw_bf16(max(mx), 16, K, g, False, seed=xseed).X
                x0 = bf16_tensor(torch, xh, dev)
            else:
                xh = workloads.draw(max(mx), 16, K, g, False, seed=xseed, outliers=out).X
                x0 = torch.from_numpy(xh).to(dev)
            h["X"][out] = xh
            xs[(out, name)] = [x0] + [x0.clone() for _ in range(LAYERS - 1)]
        host[name] = h
    torch.cuda.synchronize()
    return weights, xs, host, canon


def time_stream_reads(torch, w4, weights, shapes, args):
    """Context leg: a plain streaming read (w4a16_stream_read, no arithmetic)
    of each layer's weight bytes -- packed codes, scales and zero words, the
    bytes a call must read besides X -- as LAYERS launches captured in a
    graph like the GEMM blocks; also the same graph over 16 bytes per launch
    (the fixed cost of a launch in a graph)."""
    dev = torch.device("cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    s = torch.cuda.Stream()
    out = {}

    def timed(fn):
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=s):
            fn()
        gr.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            gr.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * LAYERS)

    tiny = weights[next(iter(shapes))][0].q[:16]
    floor_us = timed(lambda: [w4.stream_read([tiny], sink) for _ in range(LAYERS)])
    for name in shapes:
        ws = weights[name]
        nbytes = ws[0].q.numel() + ws[0].s.numel() * 2 + ws[0].z.numel() * 4
        us = timed(lambda: [w4.stream_read([w.q, w.s, w.z], sink) for w in ws])
        out[name] = dict(bytes=nbytes, us_per_launch=round(us, 3),
                         gbs=round(nbytes / (us * 1e-6) / 1e9, 1))
    return dict(per_shape=out, launch_floor_us=round(floor_us, 3),
                what="w4a16_stream_read of each layer's q, s and z buffers, "
                     f"{LAYERS} launches per graph; launch_floor_us: the same over 16 bytes")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama7b", choices=sorted(WORKLOADS))
    ap.add_argument("--dtype", default="f16", choices=("f16", "bf16"),
                    help="16-bit format of activations, scales and outputs (GEMM workloads)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-context", action="store_true",
                    help="skip the streaming-read context leg")
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="above M = 32 the oracle runs 1 in this many weight rows "
                         "(default per workload: CPU_SAMPLE)")
    ap.add_argument("--cpu-layers", type=int, default=None,
                    help="layers of the step the oracle computes (default: 5 decode7b, 3 decode70b, else 1)")
    ap.add_argument("--detail", action="store_true", help="print one line per (M, shape) on stderr")
    ap.add_argument("--context", action="store_true",
                    help="also time torch.matmul in fp16 on the dequantized weights (context only)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help=f"first run a {COPY_MIB} MiB device copy (scale for the HBM counters)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the HBM-traffic summaries from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--plain-log", default=None,
                    help="with --prof-summary: output of the same bench run without the profiler")
    ap.add_argument("--prof-summary", nargs=2, metavar=("STATS_DIR", "BENCH_LOG"),
                    help="write the kernel-time summaries from a rocprofv3 --kernel-trace --stats "
                         "run of the bench (its output directory and the bench's output) and exit")
    ap.add_argument("--pmc-command", "--command", dest="command", action="append", default=[],
                    help="command line recorded in a summary (repeat per run)")
    args = ap.parse_args()

    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.workload, args.dtype,
                    args.command)
        return
    if args.prof_summary:
        prof_summary(args.prof_summary[0], args.prof_summary[1], args.workload, args.dtype,
                     args.command, args.plain_log)
        return

    if args.cpu_sample is None:
        args.cpu_sample = CPU_SAMPLE.get(args.workload, 1)
    if args.cpu_layers is None:
        args.cpu_layers = CPU_LAYERS.get(args.workload, 1)
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
    if args.copy_calibration:
        src = torch.ones(COPY_MIB << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload == "quant7b":
        bench_quant(args, torch, w4)
        return
    if args.workload == "decodestep7b":
        bench_decode_step(args, torch, w4)
        return
    shapes = wl["shapes"]
    ms = wl["ms"]
    g = 128

    weights, xs, host, canon = build_inputs(torch, w4, wl, args.dtype, args.context)

    def xs_of(M, name, layer=0):
        return xs[(uses_outliers(wl, M), name)][layer]

    outs = {}
    for name, (N, K) in shapes.items():
        for M in ms:
            outs[(M, name)] = [torch.empty((M, N), dtype=xs_of(M, name).dtype, device=dev)
                               for _ in range(LAYERS)]
    torch.cuda.synchronize()

    cases = [(M, name) for M in ms for name in shapes]

    def run_block(M, name):
        for layer in range(LAYERS):
            w4.gemm(xs_of(M, name, layer)[:M], weights[name][layer], out=outs[(M, name)][layer])

    # eager reference outputs of layer 0 for the graph-replay check
    ref = {}
    for M, name in cases:
        w4.gemm(xs_of(M, name)[:M], weights[name][0], out=outs[(M, name)][0])
        ref[(M, name)] = outs[(M, name)][0].clone()
    torch.cuda.synchronize()

    use_graph = not args.no_graph
    case_timing = None
    step_graph = None
    if use_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for M, name in cases:   # warm the launch path (and the workspace) before capture
                run_block(M, name)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        # the whole step in one graph (the timed region is one replay per
        # step, so host-side graph launches never leave the GPU idle between
        # cases).  Timing events cannot be recorded inside a graph on ROCm
        # (external events are refused there), so each case is timed in a
        # second pass after the timed region; the cases' times sum to the
        # step time within a fraction of a percent.
        step_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(step_graph, stream=s):
            for M, name in cases:
                run_block(M, name)
        torch.cuda.synchronize()

    def one_step():
        if use_graph:
            step_graph.replay()
        else:
            for M, name in cases:
                run_block(M, name)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps ----
    stream = torch.cuda.current_stream()
    ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    eager_ev = None
    if not use_graph:
        eager_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(cases) + 1)]
                    for _ in range(args.steps)]
        case_timing = "events between the cases of the eager step"
    case_ms = np.zeros((args.steps, len(cases)))
    torch.cuda.synchronize()
    with ClockSampler(torch) as clocks:
        t0 = time.perf_counter()
        for st in range(args.steps):
            ev_s[st].record(stream)
            if use_graph:
                step_graph.replay()
            else:
                eager_ev[st][0].record(stream)
                for ci, (M, name) in enumerate(cases):
                    run_block(M, name)
                    eager_ev[st][ci + 1].record(stream)
            ev_e[st].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    step_list = [ev_s[st].elapsed_time(ev_e[st]) for st in range(args.steps)]
    if eager_ev is not None:
        for st in range(args.steps):
            case_ms[st] = [eager_ev[st][i].elapsed_time(eager_ev[st][i + 1])
                           for i in range(len(cases))]
    step_ms = float(np.mean(step_list))
    step_pct = {f"p{q}": round(float(np.percentile(step_list, q)), 4) for q in (10, 50, 90)}

    if use_graph:
        # second pass (after the timed region): each case's block of LAYERS
        # launches, REP times in a graph, replayed back to back
        case_timing = "second pass: a graph per case, replayed after the timed region"
        REP = 4
        reps = max(2, min(args.steps, 5))
        for ci, (M, name) in enumerate(cases):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=s):
                for _ in range(REP):
                    run_block(M, name)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                gr.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            case_ms[:, ci] = e0.elapsed_time(e1) / (reps * REP)
    block_ms = case_ms.mean(0)

    # replayed outputs equal the eager ones, bit for bit
    for M, name in cases:
        assert torch.equal(outs[(M, name)][0].view(torch.int16), ref[(M, name)].view(torch.int16)), \
            f"replayed output differs from eager output for M={M} {name}"

    step_bytes = sum(LAYERS * alg_bytes(M, *shapes[name], g) for M, name in cases)
    step_flops = sum(LAYERS * alg_flops(M, *shapes[name]) for M, name in cases)
    gbs = step_bytes / (step_ms * 1e-3) / 1e9
    tflops = step_flops / (step_ms * 1e-3) / 1e12

    # ---- per case: time, rates, roofline fraction max(t_mem, t_mfma) / t ----
    per_kernel = {}
    detail = []
    for ci, (M, name) in enumerate(cases):
        N, K = shapes[name]
        path, splits = w4.gemm_kernel(M, N, K, g, w4.BF16 if args.dtype == "bf16" else 0)
        kn = "gemm_" + path
        b = alg_bytes(M, N, K, g)
        f = alg_flops(M, N, K)
        us = block_ms[ci] * 1e3 / LAYERS
        t_mem = b / (HBM_PEAK_GBS * 1e9) * 1e6
        t_mfma = f / (MFMA_F16_PEAK_TFLOPS * 1e12) * 1e6
        d = per_kernel.setdefault(kn, dict(ms=0.0, bytes=0, flops=0, launches=0, roof_ms=0.0))
        d["ms"] += block_ms[ci]
        d["bytes"] += LAYERS * b
        d["flops"] += LAYERS * f
        d["launches"] += LAYERS
        d["roof_ms"] += LAYERS * max(t_mem, t_mfma) * 1e-3
        detail.append(dict(M=M, shape=name, N=N, K=K, kernel=kn, splits=splits,
                           us_per_gemm=round(us, 3),
                           gbs=round(b / (us * 1e-6) / 1e9, 1),
                           tflops=round(f / (us * 1e-6) / 1e12, 2),
                           t_mem_us=round(t_mem, 3), t_mfma_us=round(t_mfma, 3),
                           frac=round(max(t_mem, t_mfma) / us, 4)))

    # ---- roofline of each kernel group; the dominant one is `roofline` ----
    roof_by = {}
    for kn, d in per_kernel.items():
        avg_us = d["ms"] * 1e3 / d["launches"]
        if kn == "gemm_small_m":
            ach = d["bytes"] / (d["ms"] * 1e-3) / 1e9
            r = dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                     frac=round(ach / HBM_PEAK_GBS, 4), traffic=None)
        else:
            ach = d["flops"] / (d["ms"] * 1e-3) / 1e12
            r = dict(bound="mfma", achieved=round(ach, 2), peak=MFMA_F16_PEAK_TFLOPS,
                     unit="TFLOP/s", frac=round(ach / MFMA_F16_PEAK_TFLOPS, 4), traffic=None)
        tr = load_traffic(kn, profile_tag(wl["key"], args.dtype))
        if tr is not None:
            r["traffic"] = tr["traffic_bytes_per_launch"]
            r["traffic_unit"] = "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)"
            r["traffic_alg_bytes_per_launch"] = tr["alg_bytes_per_launch"]
        mains, red = KERNEL_GROUPS[kn]
        r["kernel"] = f"{kn} ({' / '.join(mains)}" + (f", + {red} where K is split)" if red else ")")
        r["avg_launch_us"] = round(avg_us, 3)
        r["launches_per_step"] = d["launches"]
        r["alg_bytes_per_launch"] = round(d["bytes"] / d["launches"])
        r["alg_flops_per_launch"] = round(d["flops"] / d["launches"])
        r["share_of_step_time"] = round(d["ms"] / block_ms.sum(), 4)
        r["roofline_frac_max_mem_mfma"] = round(d["roof_ms"] / d["ms"], 4)
        r["achieved_is"] = ("algorithmic bytes" if r["bound"] == "hbm" else "flops") + \
            " of all its calls / their summed case time (split-K reduce included)"
        roof_by[kn] = r
    dom = max(per_kernel, key=lambda k: per_kernel[k]["ms"])
    roof = roof_by[dom]

    # ---- the targets' own regimes ----
    def agg(sel):
        rows = [(ci, r) for ci, r in enumerate(detail) if sel(r["M"])]
        if not rows:
            return None
        t = sum(block_ms[ci] for ci, _ in rows) * 1e-3
        b = sum(LAYERS * alg_bytes(r["M"], r["N"], r["K"], g) for _, r in rows)
        f = sum(LAYERS * alg_flops(r["M"], r["N"], r["K"]) for _, r in rows)
        rf = sum(LAYERS * max(r["t_mem_us"], r["t_mfma_us"]) * 1e-6 for _, r in rows)
        return dict(cases=len(rows), gbs=round(b / t / 1e9, 1), frac_hbm=round(b / t / 1e9 / HBM_PEAK_GBS, 4),
                    tflops=round(f / t / 1e12, 2),
                    frac_mfma=round(f / t / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                    roofline_frac=round(rf / t, 4))
    regimes = {}
    for key, sel, note in (("m_le_16", lambda M: M <= 16, "target: >= 0.70 of HBM peak"),
                           ("m_32_to_256", lambda M: 32 <= M <= 256, "between the regimes"),
                           ("m_ge_512", lambda M: M >= 512, "target: >= 0.50 of dense fp16 MFMA peak"),
                           ("all", lambda M: True, "the whole step")):
        a = agg(sel)
        if a is not None:
            a["note"] = note
            regimes[key] = a

    stream_ctx = None
    if not args.no_stream_context and use_graph:
        stream_ctx = time_stream_reads(torch, w4, weights, shapes, args)
        m1 = {r["shape"]: r["us_per_gemm"] for r in detail if r["M"] == 1}
        for name, v in stream_ctx["per_shape"].items():
            if name in m1:
                v["gemm_m1_us"] = m1[name]
                v["gemm_m1_over_stream"] = round(m1[name] / v["us_per_launch"], 3)

    context = None
    if args.context:
        context = fp16_context(torch, w4, shapes, ms, canon, xs_of, detail, args)

    if args.detail:
        for row in detail:
            print(json.dumps(row), file=sys.stderr)

    small_only = max(ms) <= 32
    cpu = None
    parity = None
    single = None
    if not args.no_cpu_baseline:
        t_cpu, b_cpu, f_cpu, cores, refs = cpu_baseline(host, wl, args.cpu_sample, args.cpu_layers,
                                                         args.dtype)
        parity = parity_of_run(refs, outs, lambda M, name: xs_of(M, name), args.dtype, torch)
        if small_only:
            cpu = dict(value=round(b_cpu / t_cpu / 1e9, 4), unit="GB/s")
        else:
            cpu = dict(value=round(f_cpu / t_cpu / 1e12, 6), unit="TFLOP/s")
        cpu.update(cores=cores, kind="oracle", seconds=round(t_cpu, 2),
                   sample=f"every (shape, M) of {args.cpu_layers} of the {LAYERS} layers of one step; "
                          f"all weight rows at M <= 32, 1 in {args.cpu_sample} above; "
                          "fp64 C oracle, OpenMP")
        single = cpu_single_thread(host, wl, args.dtype)

    if small_only:
        value, unit = gbs, "GB/s"
    else:
        value, unit = tflops, "TFLOP/s"
    clk = clocks.summary()
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl['key']}: {wl['desc']}"
                               + (", bf16 activations/scales/outputs" if args.dtype == "bf16" else ""),
                   "layers": LAYERS,
                   "m": list(ms), "shapes": {k: list(v) for k, v in shapes.items()},
                   "group_size": g, "graphs": use_graph},
        "tflops": round(tflops, 3), "gbs": round(gbs, 1),
        "wall_s_timed": round(wall, 3),
        "ms_per_step_percentiles": step_pct,
        "case_timing": case_timing,
        "case_ms_sum": round(float(block_ms.sum()), 4),
        "clocks_during_run": clk,
        "roofline": roof, "roofline_by_kernel": roof_by, "regimes": regimes,
        "cpu_baseline": cpu, "cpu_single_thread": single, "parity": parity,
        "stream_read_context": stream_ctx,
        "per_case": detail,
    }
    if clk is None:
        line["clocks_after_run"] = read_clocks()
    if context is not None:
        line["context_fp16_matmul"] = context
    print(json.dumps(line))


if __name__ == "__main__":
    main()
