#!/usr/bin/env python3
"""Benchmark of the fused WUSH transform + MXFP4 quantization on one MI355X.

One step is one pass of the whole online path over one batch: every token's
bf16 row is transformed block by block with T_wush and quantized to E2M1
codes plus E8M0 scales.  That is one wush_quant_mxfp4 call on the
4096-token x 4096-channel workload (G = 32, 128 blocks, Student-t(3)
activations with 1% outlier channels).  The inputs are synthetic, seeded, and
resident in HBM before the timed region starts.

Metric: algorithmic HBM bytes per step (X read once, T once, codes and
scales written once) divided by the time per step, in GB/s.  Cold cache:
the steps rotate through buffer sets whose total footprint is more than
twice the 256 MB Infinity Cache, so each step reads its inputs from HBM.

Printed: one JSON line.  It carries the roofline of the kernel (its
average duration over the timed region, HIP events on the launch stream),
HBM traffic from the counter profile when one matches the kernel source,
context numbers (the same kernel with hot caches, a plain device copy of
the same bytes), and the CPU oracle timed on the host as a reported
baseline.
"""

from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MALL_BYTES = 256 << 20


TRANSFORMS = ("wush", "wus", "hadamard", "identity")


def workload_layer(wl, dev):
    """The workload's weight and calibration activations as bf16 device
    tensors (seeded synthetic data, rounded to bf16 by the generator)."""
    import numpy as np
    import torch

    from synthetic import f64_to_bf16_bits, gen_calibration, gen_weight

    def dev_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    wb, xb = f64_to_bf16_bits(gen_weight(wl)), f64_to_bf16_bits(gen_calibration(wl))
    return wb, xb, dev_bf16(wb), dev_bf16(xb)


def build_bank(name, wl, dev):
    """bf16 transform bank [C][G][G] on the device for a workload.  WUSH and
    WUS come from the workload's weight and calibration statistics, built by
    the library (wush_build_transforms); the blockwise Hadamard and the
    identity are the pages' data-agnostic comparators (RTN-H and plain RTN,
    wush_fixed_transforms)."""
    from mxfp4_activation_amd import transforms

    C, G = wl.K // wl.G, wl.G
    if name in ("wush", "wus"):
        _, _, Wd, Xd = workload_layer(wl, dev)
        return transforms.wush_bank(Wd, Xd, G, use_hadamard=(name == "wush"))[0]
    if name == "hadamard":
        return transforms.hadamard_bank(C, G, dev)
    return transforms.identity_bank(C, G, dev)


def algorithmic_bytes(fmt: str, M: int, K: int, G: int) -> int:
    scale_bytes = 2 if fmt == "int4" else 1
    return M * K * 2 + M * K // 2 + M * (K // G) * scale_bytes + (K // G) * G * G * 2


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=320)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", default="llama8b_mxfp4",
                    help="llama8b_mxfp4 (default), downproj_mxfp4, nvfp4, int4, tiny_mxfp4")
    ap.add_argument("--sets", type=int, default=0, help="rotating buffer sets (0: > 2x MALL)")
    ap.add_argument("--mode", choices=["eager", "graph"], default="eager",
                    help="timed steps as back-to-back launches (eager, default) or as one HIP graph; a graph "
                         "replay costs about 10 us more to start than the first eager launch, which is 2%% of "
                         "a 20-step run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the hot-cache and device-copy context runs (for counter profiles)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="instead of the path, run a plain device copy of this many MiB --steps times "
                         "(reference for the HBM byte counters)")
    ap.add_argument("--transform", choices=list(TRANSFORMS), default="wush",
                    help="transform bank fed to the same kernel: wush (default), wus (no Hadamard), "
                         "hadamard (blockwise H, the RTN-H comparator), identity (plain RTN)")
    ap.add_argument("--compare-transforms", action="store_true",
                    help="instead of the step benchmark, time all transform banks through the same kernel, "
                         "interleaved in one process, and print one JSON line")
    ap.add_argument("--gemm-layers", action="store_true",
                    help="per-layer Eq. 10 forward (transform + quantize + MXFP4 GEMM) against the bf16 GEMM "
                         "on Qwen3-8B layer shapes at 1024 tokens, instead of the headline measurement")
    ap.add_argument("--gemm-fused", action="store_true",
                    help="with --gemm-layers: measure the fused projections instead (q|k|v as one 6144 x 4096 "
                         "layer, gate|up as one 24576 x 4096 layer, each with one transform bank built from the "
                         "concatenated weight)")
    ap.add_argument("--gemm-model", default="qwen3-8b", choices=["qwen3-8b", "qwen3-14b", "llama3.1-70b"],
                    help="with --gemm-layers: whose linear-layer shapes to measure")
    ap.add_argument("--gemm-tokens", type=int, default=0,
                    help="with --gemm-layers: token batch M (default 1024)")
    ap.add_argument("--layer-loss", action="store_true",
                    help="layerwise loss (Eq. 5) of I / H / WUS / WUSH in MXFP4, NVFP4 and INT4 on synthetic "
                         "Qwen3-8B-shaped layers, computed by the kernels, instead of the headline measurement")
    ap.add_argument("--build-transforms", action="store_true",
                    help="time the GPU transform construction (wush_build_transforms) on each workload's layer, "
                         "builder on each workload's layer, instead of the headline measurement")
    ap.add_argument("--gptq-wush", action="store_true",
                    help="GPTQ-WUSH (Algorithm 1) on synthetic 4096-wide layers: calibration time on the GPU and the "
                         "Eq. 10 output error against RTN, instead of the headline measurement")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="instead of running, read four rocprofv3 --pmc output folders (FETCH_SIZE and "
                         "WRITE_SIZE of the path, then of --copy-probe-mib) and write "
                         "profiles/traffic_<workload>.json")
    ap.add_argument("--traffic-cmds", default="", help="the commands that made the --traffic-from folders")
    return ap.parse_args()


def copy_probe(mib: int, steps: int) -> None:
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "steps": steps,
                      "ms_per_copy": round(ms, 6), "GBps_read_plus_write": round(2 * n / ms / 1e6, 2)}),
          flush=True)


def _pmc_rows(folder: str, counter: str):
    """(kernel name, value) of every dispatch in a rocprofv3 --pmc output
    folder (SQLite results database or counter_collection.csv)."""
    import csv
    import glob

    rows = []
    dbs = glob.glob(os.path.join(folder, "**", "*_results.db"), recursive=True)
    if dbs:  # rocprofv3's default SQLite output: the counters_collection view
        import sqlite3

        for fn in dbs:
            con = sqlite3.connect(fn)
            rows += [(k, float(v)) for k, v in con.execute(
                "select kernel_name, value from counters_collection where counter_name = ?", (counter,))]
            con.close()
        return rows
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no rocprofv3 output under %s" % folder)
    for fn in files:
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def _median_for(rows, pick):
    import statistics

    vals = [v for k, v in rows if pick(k)]
    if not vals:
        raise SystemExit("no matching dispatches")
    return statistics.median(vals), len(vals)


def ingest_traffic(args) -> None:
    """HBM bytes per launch of the quant kernel from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by what the same counter reads for a
    plain device copy of known size."""
    from synthetic import CONFIGS

    wl = CONFIGS[args.workload]
    fdir, wdir, cfdir, cwdir = args.traffic_from
    is_quant = lambda k: "quant_kernel" in k
    is_copy = lambda k: "copy" in k.lower()
    f_kib, nf = _median_for(_pmc_rows(fdir, "FETCH_SIZE"), is_quant)
    w_kib, nw = _median_for(_pmc_rows(wdir, "WRITE_SIZE"), is_quant)
    cf_kib, _ = _median_for(_pmc_rows(cfdir, "FETCH_SIZE"), is_copy)
    cw_kib, _ = _median_for(_pmc_rows(cwdir, "WRITE_SIZE"), is_copy)
    copy_bytes = args.copy_probe_mib << 20
    if copy_bytes <= 0:
        raise SystemExit("--copy-probe-mib must give the size of the calibration copy")
    ff = copy_bytes / (cf_kib * 1024.0)
    fw = copy_bytes / (cw_kib * 1024.0)
    rd = f_kib * 1024.0 * ff
    wr = w_kib * 1024.0 * fw
    alg = algorithmic_bytes(wl.fmt, wl.M, wl.K, wl.G)
    alg_rd = wl.M * wl.K * 2 + (wl.K // wl.G) * wl.G * wl.G * 2
    out = {
        "workload": wl.name,
        "kernel": "quant_kernel<%s>" % wl.fmt,
        "kernel_source_sha": _kernel_source_sha(),
        "hbm_bytes_per_launch": round(rd + wr),
        "read_bytes_per_launch": round(rd),
        "write_bytes_per_launch": round(wr),
        "algorithmic_bytes_per_launch": alg,
        "algorithmic_read_bytes": alg_rd,
        "algorithmic_write_bytes": alg - alg_rd,
        "traffic_over_algorithmic": round((rd + wr) / alg, 4),
        "raw_FETCH_SIZE_KiB_median": f_kib,
        "raw_WRITE_SIZE_KiB_median": w_kib,
        "dispatches": [nf, nw],
        "calibration": {"copy_bytes_each_way": copy_bytes, "copy_FETCH_SIZE_KiB": cf_kib,
                        "copy_WRITE_SIZE_KiB": cw_kib, "fetch_factor": round(ff, 4),
                        "write_factor": round(fw, 4)},
        "commands": args.traffic_cmds,
    }
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % wl.name)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def cpu_baseline(wl, x_bits_np, transform: str, seconds: float):
    """The oracle as it stands, on the host cores: first its construction of
    the workload's transform bank (float64 Cholesky and SVD per block, timed
    on its own), then whole passes of the online path over the same
    activations until at least `seconds` have elapsed.  The oracle builds its
    bank from the same bf16 weight and calibration values the library's
    builder takes; nothing it computes comes from the GPU path."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import codecs, quant
    from oracle import transform as tr

    cores = len(os.sched_getaffinity(0))
    C, G = wl.K // wl.G, wl.G
    t_build = None
    with threadpool_limits(limits=cores):
        if transform in ("wush", "wus"):
            wb, xb, _, _ = workload_layer(wl, "cpu")
            W = codecs.bf16_bits_to_f32(wb).astype(np.float64)
            Xc = codecs.bf16_bits_to_f32(xb).astype(np.float64)
            tb0 = time.perf_counter()
            T64, _ = tr.build_transforms(W, Xc, G, H=None if transform == "wush" else np.eye(G))
            t_build = time.perf_counter() - tb0
        elif transform == "hadamard":
            T64 = np.broadcast_to(tr.hadamard(G), (C, G, G)).copy()
        else:
            T64 = np.broadcast_to(np.eye(G), (C, G, G)).copy()
        t_bits_np = tr.transforms_to_bf16_bits(T64)
        g = None
        passes = 0
        t0 = time.perf_counter()
        while True:
            if wl.fmt == "nvfp4" and g is None:
                y = quant.transform_ref(x_bits_np, t_bits_np)
                g = quant.nvfp4_global_scale(quant.tensor_amax_ref(y))
            quant.run_path(wl.fmt, x_bits_np, t_bits_np, g)
            passes += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    nbytes = algorithmic_bytes(wl.fmt, wl.M, wl.K, wl.G)
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    out = {
        "value": round(nbytes * passes / el / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "%d full pass(es) of the %dx%d workload in %.1f s (NumPy float64 oracle, "
                  "BLAS threads=%d, rest single-threaded; %s)" % (passes, wl.M, wl.K, el, cores, cpu_model),
        "elements_per_s": round(wl.M * wl.K * passes / el, 1),
    }
    if t_build is not None:
        out["transform_construction"] = {
            "seconds": round(t_build, 3), "blocks": C, "G": G, "d_out": wl.d_out, "n_cal": wl.n_cal,
            "what": "oracle build of the %s bank (moments, damping, Cholesky, SVD, products per block, "
                    "float64), once, same host and threads" % transform}
    return out


def context_runs(graph_ms, launch, sets, n_sets, nbytes, M, K, dev):
    """The kernel on one buffer set (inputs served from the Infinity Cache),
    and a plain device copy moving the same bytes, cold.  The copy moves the
    activation bytes themselves (the first half of each set's X), since
    bandwidth on this part depends on the data."""
    import torch

    hot_ms = graph_ms(lambda i: launch(0), 64, 4)
    half = min(nbytes // 2, M * K * 2) // 16 * 16
    csets = [(X.view(torch.uint8).view(-1)[:half], torch.empty(half, dtype=torch.uint8, device=dev))
             for X, _, _, _ in sets]
    copy_ms = graph_ms(lambda i: csets[i % n_sets][1].copy_(csets[i % n_sets][0]), n_sets * 4, 4)
    del csets
    torch.cuda.synchronize()
    return hot_ms, copy_ms


def compare_transforms(args) -> None:
    """WUSH against the comparators through the same kernel: the same cold
    rotating buffer sets, one HIP graph per transform, replays interleaved
    so drift affects all alike; median over repetitions."""
    import statistics

    import numpy as np
    import torch

    import mxfp4_activation_amd as wush
    from mxfp4_activation_amd import _lib
    from synthetic import CONFIGS, gen_x_bits

    wl = CONFIGS[args.workload]
    M, K, G, fmt = wl.M, wl.K, wl.G, wl.fmt
    lib = wush.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    X0 = torch.from_numpy(gen_x_bits(wl).view(np.int16)).view(torch.bfloat16).to(dev)
    banks = {name: build_bank(name, wl, dev) for name in TRANSFORMS}
    nbytes = algorithmic_bytes(fmt, M, K, G)
    n_sets = args.sets or max(2, -(-2 * MALL_BYTES // nbytes) + 1)
    sdt = torch.float16 if fmt == "int4" else torch.uint8
    xs = [X0.clone() if i else X0 for i in range(n_sets)]
    outs = [(torch.empty((M, K // 2), dtype=torch.uint8, device=dev), torch.empty((M, K // G), dtype=sdt, device=dev))
            for _ in range(n_sets)]
    tsets = {name: [T.clone() for _ in range(n_sets)] for name, T in banks.items()}
    gscale = torch.zeros(1, dtype=torch.float32, device=dev)
    counts = torch.zeros(len(TRANSFORMS), dtype=torch.int32, device=dev)
    fmt_id = _lib.FMT[fmt]
    cap = torch.cuda.Stream()
    graphs = {}
    # Each bank's tensor scale stays referenced while its graph exists:
    # torch.cuda.graph() empties the allocator cache at every capture, so a
    # dropped tensor could be unmapped under an earlier graph.
    g_keep = []
    for ti, name in enumerate(TRANSFORMS):
        if fmt == "nvfp4":
            g = torch.zeros(1, dtype=torch.float32, device=dev)
            wush.nvfp4_global_scale(X0, banks[name], out=g)
        else:
            g = gscale
        g_keep.append(g)

        def launch(i, name=name, g=g, cnt=None):
            c, s = outs[i % n_sets]
            st = lib.wush_quant(fmt_id, xs[i % n_sets].data_ptr(), tsets[name][i % n_sets].data_ptr(), M, K,
                                g.data_ptr() if fmt == "nvfp4" else None, c.data_ptr(), s.data_ptr(),
                                None if cnt is None else cnt, torch.cuda.current_stream().cuda_stream)
            if st:
                _lib.check(st, "wush_quant")

        launch(0, cnt=counts[ti:ti + 1].data_ptr())  # exact recomputations of one launch
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=cap):
            for i in range(n_sets * 4):
                launch(i)
        gr.replay()
        graphs[name] = gr
    torch.cuda.synchronize()
    times = {name: [] for name in TRANSFORMS}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(max(3, args.steps // 40)):
        for name in TRANSFORMS:
            torch.cuda.synchronize()
            e0.record()
            graphs[name].replay()
            e1.record()
            torch.cuda.synchronize()
            times[name].append(e0.elapsed_time(e1) * 1e3 / (n_sets * 4))
    cnt = counts.cpu().tolist()
    res = {}
    for ti, name in enumerate(TRANSFORMS):
        us = statistics.median(times[name])
        res[name] = {"us_per_step": round(us, 3), "GBps": round(nbytes / us / 1e3, 2),
                     "exact_groups_per_launch": cnt[ti]}
    gap = 100.0 * (res["wush"]["us_per_step"] / res["hadamard"]["us_per_step"] - 1.0)
    print(json.dumps({
        "comparison": "transform banks through the same fused kernel (cold, interleaved graphs, median)",
        "workload": wl.name, "format": fmt, "tokens": M, "d": K, "G": G,
        "algorithmic_bytes_per_step": nbytes, "results": res,
        "wush_vs_hadamard_time_pct": round(gap, 2),
        "pages": "WUSH+Quant within about 1.3% of H+Quant on average (papernotes results; deep dive 3.4.7, 5)",
    }), flush=True)


def gemm_layers(args) -> None:
    """Per-layer forward of Eq. 10 on the linear-layer shapes of Qwen3-8B
    (or, with --gemm-model, Qwen3-14B or Llama-3.1-70B) at 1024 tokens,
    against the bf16 GEMM (deep dive, section 3.4.7 and the
    results: speedup of transform + quantization + FP4 MatMul over BF16,
    with "None" = the FP4 MatMul alone).  Weights are random N(0, 0.02) in
    nn.Linear order, pre-quantized offline with the weight-side transform
    (T_xvsh for WUSH, H for H+Quant); activations are Student-t(3)-like
    with 1% outlier channels.  Hot caches (the same buffers every step),
    one HIP graph per variant, replays interleaved, median."""
    import statistics

    import torch

    from mxfp4_activation_amd import ops, transforms
    from synthetic.gemm_operands import GEMM_TOKENS, MODEL_LAYERS, QWEN3_8B_FUSED

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    M, G = (args.gemm_tokens or GEMM_TOKENS), 32
    if M < 1:
        raise SystemExit("--gemm-tokens must be positive")
    gen = torch.Generator(device="cpu").manual_seed(2024)
    shapes = {}
    if args.gemm_fused and args.gemm_model != "qwen3-8b":
        raise SystemExit("--gemm-fused measures the Qwen3-8B projections only")
    for name, nk in (QWEN3_8B_FUSED if args.gemm_fused else MODEL_LAYERS[args.gemm_model]).items():
        shapes.setdefault(nk, []).append(name)
    rows = []
    for (N, K), names in shapes.items():
        C = K // G
        out_ch = torch.randperm(K, generator=gen)[: max(1, K // 100)]
        def acts(n):
            x = torch.distributions.StudentT(3.0).sample((n, K)) * 0.5
            x[:, out_ch] *= 30.0
            return x
        torch.manual_seed(K * 7 + N)
        Xcal = acts(2048).to(torch.bfloat16).to(dev)
        W = (torch.randn(N, K, generator=gen, dtype=torch.float64) * 0.02)
        X = acts(M).to(torch.bfloat16).to(dev)
        Wb = W.to(torch.bfloat16).to(dev)
        Tw, Tx, _, _ = transforms.wush_bank(Wb, Xcal, G)
        Hb = transforms.hadamard_bank(C, G, dev)
        banks = {"wush": (Tw, Tx), "hadamard": (Hb, Hb)}
        wq = {k: ops.quant("mxfp4", Wb, tb[1]) for k, tb in banks.items()}
        # Weights are quantized offline, and re-laid once (offline too) in
        # the order the GEMM kernel stages them.
        wp = {k: ops.gemm_pack_b(*wq[k]) for k in wq}
        xc = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        xs = torch.empty((M, K // G), dtype=torch.uint8, device=dev)
        # The activations' codes and scales in the GEMM's packed layout,
        # written there by the quantizer itself.
        xp = ops.quant_mxfp4_packed(X, banks["wush"][0])
        Cout = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        Wt = Wb.t()

        def v_bf16():
            torch.matmul(X, Wt, out=Cout)

        def v_q(k):
            def f():
                ops.quant_mxfp4_packed(X, banks[k][0], out=xp)
                ops.gemm_mxfp4_packed(xp, wp[k], out_dtype=torch.bfloat16, out=Cout)
            return f

        def v_none():
            ops.gemm_mxfp4_packed(xp, wp["wush"], out_dtype=torch.bfloat16, out=Cout)

        def v_q_rows():
            ops.quant("mxfp4", X, banks["wush"][0], codes=xc, scales=xs)
            ops.gemm_mxfp4(xc, xs, wq["wush"][0], wq["wush"][1], out_dtype=torch.bfloat16, out=Cout)

        def v_none_rows():
            ops.gemm_mxfp4(xc, xs, wq["wush"][0], wq["wush"][1], out_dtype=torch.bfloat16, out=Cout)

        variants = {"bf16": v_bf16, "wush_quant_fp4": v_q("wush"), "h_quant_fp4": v_q("hadamard"),
                    "none_fp4": v_none, "wush_quant_fp4_row_major": v_q_rows, "none_fp4_row_major": v_none_rows}
        reps = 40
        cap = torch.cuda.Stream()
        graphs = {}
        for vn, fn in variants.items():
            with torch.cuda.stream(cap):
                for _ in range(3):
                    fn()
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=cap):
                for _ in range(reps):
                    fn()
            gr.replay()
            graphs[vn] = gr
        torch.cuda.synchronize()
        times = {vn: [] for vn in variants}
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(7):
            for vn in variants:
                torch.cuda.synchronize()
                e0.record()
                graphs[vn].replay()
                e1.record()
                torch.cuda.synchronize()
                times[vn].append(e0.elapsed_time(e1) * 1e3 / reps)
        us = {vn: statistics.median(t) for vn, t in times.items()}
        flop = 2.0 * M * N * K
        row = {"layers": names, "N": N, "K": K, "M": M,
               "us": {vn: round(t, 2) for vn, t in us.items()},
               "speedup_vs_bf16": {vn: round(us["bf16"] / t, 2) for vn, t in us.items() if vn != "bf16"},
               "fp4_gemm_tflops": round(flop / us["none_fp4"] / 1e6, 1),
               "bf16_gemm_tflops": round(flop / us["bf16"] / 1e6, 1)}
        rows.append(row)
        print(json.dumps(row), flush=True)
    what = "fused Qwen3-8B projections" if args.gemm_fused else "%s layer shape" % args.gemm_model
    print(json.dumps({"comparison": "Eq. 10 forward per %s, %d tokens, bf16 output, hot caches" % (what, M),
                      "variants": {"bf16": "torch.matmul (hipBLASLt)",
                                   "wush_quant_fp4": "wush_quant_mxfp4_packed (T_wush) + wush_gemm_mxfp4_packed: "
                                                     "activations quantized into the GEMM's operand layout, weights "
                                                     "packed offline",
                                   "h_quant_fp4": "same kernels with the blockwise Hadamard bank",
                                   "none_fp4": "wush_gemm_mxfp4_packed alone",
                                   "wush_quant_fp4_row_major": "wush_quant_mxfp4 + wush_gemm_mxfp4, both operands "
                                                               "row-major",
                                   "none_fp4_row_major": "wush_gemm_mxfp4 alone, both operands row-major"},
                      "layers": rows}), flush=True)


def layer_loss(args) -> None:
    """Table 1 analogue (deep dive, section 5, "Per-Layer Quantization
    Loss"): Eq. 5 for the transform pairs I, H, WUS and WUSH in the three
    formats, on one synthetic linear layer per Qwen3-8B block shape (random
    N(0, 0.02) weights, Student-t(3) activations with 1% outlier channels,
    2048 calibration and 2048 evaluation tokens).  Transform, quantization
    and dequantization run in the kernels; the products are fp32 GEMMs.
    Printed per layer and format: the loss and the loss relative to the
    mean squared unquantized output."""
    import numpy as np
    import torch

    from mxfp4_activation_amd import layerwise
    from synthetic import f64_to_bf16_bits
    from synthetic.gemm_operands import QWEN3_8B_LAYERS
    from synthetic.layers import gen_linear_layer

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf16(a):
        return torch.from_numpy(f64_to_bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(dev)

    table = {}
    for li, (name, (N, K)) in enumerate(QWEN3_8B_LAYERS.items()):
        W, Xc, Xe = gen_linear_layer(K, N, 2048, 2048, seed=7000 + li, n_outlier=max(1, K // 100))
        X, Wd = bf16(Xe), bf16(W)
        ref_ms = float((X.float() @ Wd.float().t()).double().pow(2).mean().item())
        Xcd = bf16(Xc)
        for fmt in ("mxfp4", "nvfp4", "int4"):
            G = 16 if fmt == "nvfp4" else 32
            banks = layerwise.transform_pairs(Wd, Xcd, G)
            losses = {k: layerwise.layerwise_loss(fmt, X, Wd, a, b) for k, (a, b) in banks.items()}
            row = {"layer": name, "d_in": K, "d_out": N, "format": fmt,
                   "loss": {k: float("%.6g" % v) for k, v in losses.items()},
                   "relative": {k: float("%.4g" % (v / ref_ms)) for k, v in losses.items()}}
            table.setdefault(fmt, {})[name] = row["relative"]
            print(json.dumps(row), flush=True)
    print(json.dumps({"comparison": "layerwise loss (Eq. 5) relative to the mean squared output, synthetic "
                                    "Qwen3-8B-shaped layers", "relative": table}), flush=True)


def build_transforms_timing(args) -> None:
    """Offline construction of T_wush and T_xvsh for each workload's layer
    (Eq. 7, Eq. 8) in the library: moments, damping, Cholesky, Jacobi SVD and
    the products, one workgroup per block, float64 on the device.  Its
    agreement with the oracle is a test (tests/test_gpu_build.py); the
    oracle's own construction time on the host is part of the default
    run's cpu_baseline."""
    import statistics

    import torch

    from mxfp4_activation_amd import ops
    from synthetic import CONFIGS

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    for name in ("llama8b_mxfp4", "downproj_mxfp4", "nvfp4", "int4"):
        wl = CONFIGS[name]
        _, _, Wd, Xd = workload_layer(wl, dev)
        for _ in range(2):
            ops.build_transforms(Wd, Xd, wl.G)
        torch.cuda.synchronize()
        gpu = []
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(5):
            e0.record()
            ops.build_transforms(Wd, Xd, wl.G)
            e1.record()
            torch.cuda.synchronize()
            gpu.append(e0.elapsed_time(e1))
        print(json.dumps({"workload": name, "d_out": wl.d_out, "n_cal": wl.n_cal, "d_in": wl.K, "G": wl.G,
                          "blocks": wl.K // wl.G, "gpu_ms": round(statistics.median(gpu), 3)}), flush=True)


def gptq_wush_bench(args) -> None:
    """GPTQ-WUSH (deep dive, section 3.4.6, Algorithm 1) against round-to-
    nearest on synthetic layers (Student-t(3) activations with 1% outlier
    channels, N(0, 0.02) weights; 8192 calibration tokens, 2048 held-out
    tokens).  The weights are calibrated on the device (float64); the
    held-out tokens then go through the Eq. 10 forward in the kernels (fused
    transform + MXFP4 quantization, MXFP4 GEMM).  Printed: calibration time
    and the output error relative to the mean squared exact output, for
    GPTQ-WUSH, RTN inside Algorithm 1, and RTN with the blockwise Eq. 8
    transforms."""
    import numpy as np
    import torch

    from mxfp4_activation_amd import gptq as pg
    from mxfp4_activation_amd import ops, transforms
    from synthetic import f64_to_bf16_bits
    from synthetic.layers import gen_linear_layer

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    for name, d_in, d_out in (("q_proj-like", 4096, 4096), ("down_proj-like", 12288, 4096)):
        W, Xc, Xe = gen_linear_layer(d_in, d_out, 8192, 2048, seed=9000 + d_in, n_outlier=d_in // 100)
        Wd, Xcd = torch.from_numpy(W).to(dev), torch.from_numpy(Xc).to(dev)
        Xb = torch.from_numpy(f64_to_bf16_bits(Xe).view(np.int16)).to(dev).view(torch.bfloat16)
        exact = torch.from_numpy(Xe).to(dev) @ Wd.t()
        den = float((exact ** 2).mean())

        def forward(bank, wc, ws):
            xc, xs = ops.quant("mxfp4", Xb, bank)
            out = ops.gemm_mxfp4(xc, xs, wc, ws, out_dtype=torch.float32)
            return float(((out.double() - exact) ** 2).mean()) / den

        row = {"layer": name, "d_in": d_in, "d_out": d_out, "n_cal": 8192, "n_eval": 2048}
        for mode in (True, False):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            r = pg.gptq_wush(Wd, Xcd, 32, "mxfp4", gptq=mode)
            torch.cuda.synchronize()
            key = "gptq_wush" if mode else "rtn_alg1"
            row[key + "_calib_s"] = round(time.perf_counter() - t0, 2)
            row[key + "_rel_err"] = float("%.5g" % forward(transforms.to_kernel_layout(r.T_x), r.codes, r.scales))
        Wb = torch.from_numpy(f64_to_bf16_bits(W).view(np.int16)).to(dev).view(torch.bfloat16)
        Xcb = torch.from_numpy(f64_to_bf16_bits(Xc).view(np.int16)).to(dev).view(torch.bfloat16)
        Tw, Tx, _, _ = transforms.wush_bank(Wb, Xcb, 32)
        wq_c, wq_s = ops.quant("mxfp4", Wb, Tx)
        row["rtn_eq8_rel_err"] = float("%.5g" % forward(Tw, wq_c, wq_s))
        print(json.dumps(row), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the path needs no cross-GPU exchange (token rows are "
              "independent), so --gpus must be 1 (got --gpus %d, WORLD_SIZE %d)." % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    if args.traffic_from:
        ingest_traffic(args)
        return
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib, args.steps)
        return
    if args.compare_transforms:
        compare_transforms(args)
        return
    if args.gemm_layers:
        gemm_layers(args)
        return
    if args.layer_loss:
        layer_loss(args)
        return
    if args.build_transforms:
        build_transforms_timing(args)
        return
    if args.gptq_wush:
        gptq_wush_bench(args)
        return

    import numpy as np
    import torch

    import mxfp4_activation_amd as wush
    from mxfp4_activation_amd import _lib
    from synthetic import CONFIGS, gen_x_bits

    wl = CONFIGS[args.workload]
    M, K, G, fmt = wl.M, wl.K, wl.G, wl.fmt
    lib = wush.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("bench: workload %s (%s, M=%d, K=%d, G=%d)" % (wl.name, fmt, M, K, G), file=sys.stderr, flush=True)

    # Inputs: seeded activations and the offline transform bank.
    x_np = gen_x_bits(wl)
    T0 = build_bank(args.transform, wl, dev)
    X0 = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)

    nbytes = algorithmic_bytes(fmt, M, K, G)
    per_set = nbytes
    n_sets = args.sets or max(2, -(-2 * MALL_BYTES // per_set) + 1)
    sets = []
    sdt = torch.float16 if fmt == "int4" else torch.uint8
    for i in range(n_sets):
        X = X0.clone() if i else X0
        T = T0.clone() if i else T0
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((M, K // G), dtype=sdt, device=dev)
        sets.append((X, T, codes, scales))
    gscale = torch.zeros(1, dtype=torch.float32, device=dev)
    if fmt == "nvfp4":
        wush.nvfp4_global_scale(X0, T0, out=gscale)
    torch.cuda.synchronize()

    fmt_id = _lib.FMT[fmt]
    gs_ptr = gscale.data_ptr() if fmt == "nvfp4" else None
    ptrs = [(X.data_ptr(), T.data_ptr(), c.data_ptr(), s.data_ptr()) for X, T, c, s in sets]
    quant_fn = lib.wush_quant

    # The launch stream: the device's current stream, looked up once for
    # eager launches, and per call while a graph is being captured.
    eager_stream = torch.cuda.current_stream().cuda_stream
    capturing = [False]

    def launch(i):
        xp, tp, cp, sp = ptrs[i % n_sets]
        strm = torch.cuda.current_stream().cuda_stream if capturing[0] else eager_stream
        st = quant_fn(fmt_id, xp, tp, M, K, gs_ptr, cp, sp, None, strm)
        if st:
            _lib.check(st, "wush_quant")

    for i in range(min(args.warmup, 8)):  # first launches: code upload, clocks
        launch(i)
    torch.cuda.synchronize()

    # Per-launch kernel durations from HIP events on the launch stream, a
    # diagnostic: the events between launches add their own cost.
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        evs[i][0].record(stream)
        launch(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    kern_ms = np.array([a.elapsed_time(b) for a, b in evs])

    # Timed region: exactly K steps back to back, each launch on the next
    # buffer set.  Eager launches (the default) keep the device busy: the
    # host enqueues a launch in a few microseconds, the kernel runs about
    # ten.  In graph mode the K steps are one HIP graph.
    if args.mode == "graph":
        cap = torch.cuda.Stream()

        def capture(n, first=0):
            g = torch.cuda.CUDAGraph()
            capturing[0] = True
            with torch.cuda.graph(g, stream=cap):
                for i in range(first, first + n):
                    launch(i)
            capturing[0] = False
            return g

        g_timed = capture(args.steps)
        g_timed.replay()  # uploads the graph; not counted as steps
        torch.cuda.synchronize()
    # Warmup: W untimed steps, directly before the timed region, on the
    # buffer sets that precede set 0 in the rotation, so the timed steps
    # continue the rotation and each reads a set that left the caches
    # n_sets - 1 steps earlier.
    wfirst = (-args.warmup) % n_sets
    if args.mode == "graph" and args.warmup:
        wg = capture(args.warmup, wfirst)
        wg.replay()
    else:
        for i in range(wfirst, wfirst + args.warmup):
            launch(i)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # No garbage collection pass may stall the host between eager launches.
    gc_was_on = gc.isenabled()
    gc.disable()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    if args.mode == "graph":
        g_timed.replay()
    else:
        for i in range(args.steps):
            launch(i)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    if gc_was_on:
        gc.enable()
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / args.steps

    value = nbytes / (ms_per_step * 1e-3) / 1e9
    # The roofline uses the kernel's average duration over the timed region:
    # back-to-back launches of the one kernel, HIP events on the launch
    # stream.  rocprofv3 --kernel-trace on the same command reports the
    # per-dispatch duration without the fixed inter-kernel gap (about
    # 1.5 us on this platform, measured with an empty kernel).  The
    # profile summaries under profiles/ record both.
    kern_avg_ms = ms_per_step
    achieved = nbytes / (kern_avg_ms * 1e-3) / 1e9

    # Context, not the metric: hot caches and a plain device copy.
    def graph_ms(fn, n, reps):
        cap = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        capturing[0] = True
        with torch.cuda.graph(g, stream=cap):
            for i in range(n):
                fn(i)
        capturing[0] = False
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (n * reps)

    hot_ms = copy_ms = packed_ms = float("nan")
    if not args.no_context:
        hot_ms, copy_ms = context_runs(graph_ms, launch, sets, n_sets, nbytes, M, K, dev)
        # The same codes and scales in the GEMM's packed operand layout
        # (wush_quant_mxfp4_packed), cold, on the same sets; its buffers are
        # the sets' own when M is a multiple of 128.
        if fmt == "mxfp4" and K % 256 == 0 and M % 128 == 0:
            def launch_packed(i):
                xp, tp, cp, sp = ptrs[i % n_sets]
                strm = torch.cuda.current_stream().cuda_stream
                _lib.check(lib.wush_quant_mxfp4_packed(xp, tp, M, K, cp, sp, strm), "wush_quant_mxfp4_packed")

            packed_ms = graph_ms(launch_packed, n_sets * 4, 4)
            row_major_ms = graph_ms(launch, n_sets * 4, 4)

    # NVFP4 with its per-tensor scale computed in the same step: the AbsMax
    # pre-pass (transform of the whole tensor, max |y|, g = max / (6 * 448))
    # and then the quantize kernel with that g, each set with its own g.
    prepass = None
    if fmt == "nvfp4" and not args.no_context:
        gs_sets = [torch.zeros(1, dtype=torch.float32, device=dev) for _ in range(n_sets)]

        def launch_with_prepass(i):
            xp, tp, cp, sp = ptrs[i % n_sets]
            g_ptr = gs_sets[i % n_sets].data_ptr()
            strm = torch.cuda.current_stream().cuda_stream
            _lib.check(lib.wush_nvfp4_global_scale(xp, tp, M, K, g_ptr, strm), "wush_nvfp4_global_scale")
            _lib.check(quant_fn(fmt_id, xp, tp, M, K, g_ptr, cp, sp, None, strm), "wush_quant")

        pp_ms = graph_ms(launch_with_prepass, n_sets * 4, 4)
        # The pre-pass reads X and T once more.
        pp_bytes = nbytes + M * K * 2 + (K // G) * G * G * 2
        same = torch.equal(gs_sets[0], gscale)
        prepass = {"us_per_step": round(pp_ms * 1e3, 3), "algorithmic_bytes": pp_bytes,
                   "GBps": round(pp_bytes / (pp_ms * 1e-3) / 1e9, 2),
                   "pct_of_hbm_peak": round(100.0 * pp_bytes / (pp_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                   "global_scale_matches_setup": bool(same)}
        del gs_sets

    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic_%s.json" % wl.name)
    if os.path.exists(tpath):
        with open(tpath) as f:
            tr = json.load(f)
        if tr.get("kernel_source_sha") == _kernel_source_sha():
            traffic = tr.get("hbm_bytes_per_launch")

    out = {
        "metric": "fused WUSH+%s quant: HBM GB/s and %% of peak at d=%d, %d tokens" % (fmt.upper(), K, M),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "%s: X bf16 [%d x %d], G=%d, %s, %d outlier channels x%g; T_wush per block from "
                        "W [%d x %d] N(0,0.02) and %d calibration tokens" % (
                            wl.name, M, K, G, wl.dist, wl.n_outlier, wl.outlier_mult, wl.d_out, K, wl.n_cal),
            "format": fmt,
            "transform": args.transform,
            "tokens": M,
            "d": K,
            "G": G,
            "algorithmic_bytes_per_step": nbytes,
            "cold_cache_sets": n_sets,
            "timing": args.mode,
            "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
            "elements_per_s": round(M * K / (ms_per_step * 1e-3), 1),
            "host_wall_s": round(wall, 4),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "quant_kernel<%s>" % fmt,
            "kernel_avg_us": round(kern_avg_ms * 1e3, 3),
            "per_launch_event_avg_us": round(float(kern_ms.mean()) * 1e3, 3),
            "per_launch_event_p10_p90_us": [round(float(np.percentile(kern_ms, 10)) * 1e3, 3),
                                            round(float(np.percentile(kern_ms, 90)) * 1e3, 3)],
        },
    }
    half = min(nbytes // 2, M * K * 2) // 16 * 16
    out["context"] = None if args.no_context else {
        "hot_cache_us_per_step": round(hot_ms * 1e3, 3),
        "hot_cache_GBps": round(nbytes / (hot_ms * 1e-3) / 1e9, 2),
        "device_copy_cold": {"bytes_read_plus_written": 2 * half, "us": round(copy_ms * 1e3, 3),
                             "GBps": round(2 * half / (copy_ms * 1e-3) / 1e9, 2)},
    }
    if out["context"] is not None and packed_ms == packed_ms:
        out["context"]["gemm_packed_layout_cold"] = {
            "entry": "wush_quant_mxfp4_packed", "us": round(packed_ms * 1e3, 3),
            "GBps": round(nbytes / (packed_ms * 1e-3) / 1e9, 2),
            "row_major_same_graphs_us": round(row_major_ms * 1e3, 3)}
    if prepass is not None:
        out["context"]["nvfp4_with_absmax_prepass"] = prepass
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle (~%.0f s)" % args.cpu_seconds, file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, x_np, args.transform, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def _code_only(src: bytes) -> bytes:
    """C/C++ source without comments, trailing blanks and empty lines, so
    that an edit to a comment does not change the hash of the code."""
    import re

    text = re.sub(rb"/\*.*?\*/", b"", src, flags=re.S)
    text = re.sub(rb"//[^\n]*", b"", text)
    return b"\n".join(line.rstrip() for line in text.split(b"\n") if line.strip())


def _kernel_source_sha() -> str:
    import hashlib

    h = hashlib.sha256()
    # The quantization kernel's code and its launch planner (plan_quant in
    # the ABI file); the other entry points of the library do not enter.
    csrc = os.path.join(ROOT, "mxfp4_activation_amd", "csrc")
    for name in ("wush_kernels.hip", "wush_kernels.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(_code_only(f.read()))
    with open(os.path.join(csrc, "wush_abi.cpp"), "rb") as f:
        abi = f.read()
    start = abi.find(b"void plan_quant(")
    h.update(_code_only(abi[start:abi.find(b"\n}\n", start) + 3] if start >= 0 else abi))
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
