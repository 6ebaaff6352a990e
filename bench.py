"""Benchmark: SubMConv3d ms/layer and effective TFLOP/s on one MI355X.

Workload: SubMConv3d 3x3x3, batch 1, 128^3 grid, 209,715 uniform voxels (10 %
occupancy), Cin = Cout = 128, fp16 features and weights, fp32 accumulation,
no bias; the kernel map is built once and reused (warm cache), as in the
"Performance" table of the trellis_sparse_mlx README.

A step is one layer through the C ABI's submconv_forward on the layer's own
weights W [27,128,128] (the call rearranges W into the MFMA fragment order,
then runs the fused gather-GEMM), inputs resident in HBM. Effective TFLOP/s =
2 * active_pairs * Cin * Cout / time. The JSON line also carries:
  * the roofline of the dominant kernel: the forward on prepared weights
    (submconv_forward_prepared), launched back to back inside one event pair
    on the launch stream, as the steps are timed; its algorithmic bytes are
    the structures it reads and writes (features, output, the per-tile lists
    and counts, weights);
  * measured ceilings from the same process: a 512 MiB device copy's GB/s and
    a dense fp16 GEMM's TFLOP/s (torch.matmul), with the kernel's fractions
    of both;
  * the kernel-map build time, the CPU oracle (C twin, all host threads, the
    host CPU's model) timed on the same workload, and for context the pages'
    own figures for this workload (other hardware: not a target).

With --op backward_input or backward_weight the same workload times the
layer's input gradient (submconv_backward_input on W: the forward with the
flipped, transposed kernel on the same map) or weight gradient (the MFMA pair
contraction + the fixed-order reduction of its partials), each with its own
roofline and oracle baseline. --op downsample / subdivide time the x2
coordinate operations on the workload's sites and first-layer features
(sites per second; the downsample step includes its plan and one host wait,
its roofline covers the max-pool kernel on a built plan).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--op OP]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, TFLOP/s
CSRC = os.path.join(ROOT, "submanifold_sparse_convolution_hash_amd", "csrc")

# HBM traffic of one launch of an op's dominant kernel from rocprofv3 counter
# runs of this script (FETCH_SIZE and WRITE_SIZE, KiB per dispatch, averaged
# over its launches), keyed by (workload, op) and by the SHA-256 of the kernel
# source's code (comments stripped) they were taken on. Scale factors come from a plain 512 MiB device
# copy measured in the same runs (--calib-copy-mib 512, and the measured-ceiling
# copies): its FETCH_SIZE read 262,156 KiB and its WRITE_SIZE 524,288 KiB for
# 524,288 KiB moved each way.
# A changed kernel source makes the entry stale and the reported traffic null.
MEASURED_TRAFFIC = {
    ("c3_128_128", "forward"): {
        "src": ["forward.hip", "map_build.hip"],  # the kernel, and the map's tile size
        "sha256": "58379b2e89bb43ddf2c4f318803e671165dc532190e1195c6cd804526e716e00",
        "fetch_kib": 49377.4, "write_kib": 52430.7,
        "fetch_factor": 524288.0 / 262170.9, "write_factor": 524288.0 / 524288.0},
    ("c5_512_chain", "forward"): {
        "src": ["staged.hip", "map_build.hip"],  # the staged kernel (64 -> 32), and its plan
        "sha256": "59d85ecd7a57ae395b215df26e4b960f1191677160ce4c408c1fd486515174df",
        "fetch_kib": 168751.0, "write_kib": 95630.5,
        "fetch_factor": 524288.0 / 262170.0, "write_factor": 524288.0 / 524288.0},
    ("c5_512_chain", "backward_weight"): {
        # the staged weight gradient (64 -> 32) and its reduce: the call bench.py times
        "src": ["staged_bwd.hip", "map_build.hip"],
        "sha256": "ee68c00cb7a9fa3ce43ce3c826da56166e4d758d23e519adef566fae22430577",
        "fetch_kib": 195501.9 + 27656.5, "write_kib": 55296.0 + 216.0,
        "fetch_factor": 524288.0 / 262159.1, "write_factor": 524288.0 / 524288.0},
    ("c4_256_shell", "forward"): {
        "src": ["staged_wide.hip", "map_build.hip"],  # the staged kernel (256 -> 256), and its plan
        "sha256": "057d7490056cdcf9fa2e8abef00a7b3dd37286e31b8181b3325c9bef842de8b5",
        "fetch_kib": 2059962.6, "write_kib": 372321.9,
        "fetch_factor": 524288.0 / 262160.9, "write_factor": 524288.0 / 524288.0},
}

METRICS = {
    "forward": "SubMConv3d ms/layer + effective TFLOP/s (128^3 grid, C=128, 10% occ)",
    "backward_input": "SubMConv3d input-gradient ms/layer + effective TFLOP/s",
    "backward_weight": "SubMConv3d weight-gradient ms/layer + effective TFLOP/s",
    "forward_masked": "SubMConv3d masked implicit-GEMM ms/layer + effective TFLOP/s",
    "downsample": "x2 sparse downsample (max) input sites/s",
    "subdivide": "x2 sparse subdivide input sites/s",
}
KERNELS = {"forward": "k_fwd_pp", "backward_input": "k_fwd_pp", "backward_weight": "k_bwd_weight",
           "forward_masked": "k_fwd_masked",
           "downsample": "k_down_max", "subdivide": "k_subdivide"}


def algorithmic_bytes(op, n, cin, cout, ksize, has_order, has_bias, pairs, tile_rows, staged=None):
    """Compulsory HBM bytes of one launch of the op's dominant kernel: its row
    inputs read once and its output written once; for a 3x3x3 forward (or
    input gradient) the per-tile lists it streams (8 bytes per active pair,
    plus the terminating entry) with the tiles' counts (27 x 2 bytes) and
    offsets (4 bytes), or with the staged kernel (staged = (units, staged
    rows)) the staged plan it reads (16 bytes per unit, 4 per staged row, a
    2-byte table entry per (tap, row)); for the weight gradient the lists;
    the processing order when there is one; the weights (fp16 in, or the
    fp32 weight gradient out) and the bias."""
    K = 27 if ksize == 3 else 1
    b = n * cin * 2 + n * cout * 2
    b += K * cin * cout * (4 if op == "backward_weight" else 2)
    if ksize == 3:
        if staged:
            b += staged[0] * 16 + staged[1] * 4 + 27 * 2 * (n + (n & 1))
        else:
            n_tiles = -(-n // tile_rows)
            b += (pairs + 1) * 8 + n_tiles * (27 * 2 + 4) + 4
        if has_order:
            b += n * 4
    if has_bias and op in ("forward", "forward_masked"):
        b += cout * 4
    return b


def code_sha256(*paths):
    """SHA-256 of source files' code: // comments and blank lines removed,
    so that editing a comment does not invalidate counters taken on the code."""
    lines = []
    for path in paths:
        with open(path) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def measured_traffic(config, op, morton):
    """HBM bytes per launch from the counter table, or None when no entry
    matches this workload, op and the current kernel code."""
    t = MEASURED_TRAFFIC.get((config, op))
    if t is None or morton:
        return None
    if code_sha256(*(os.path.join(CSRC, f) for f in t["src"])) != t["sha256"]:
        return None
    return round((t["fetch_kib"] * t["fetch_factor"] + t["write_kib"] * t["write_factor"]) * 1024)


def _time(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / steps * 1e3  # us


def measured_ceilings(torch, dev):
    """Achievable ceilings measured in this process: a 512 MiB device copy
    (GB/s counting the bytes read and written) and a dense fp16 GEMM,
    torch.matmul 8192^3 on the vendor library (TFLOP/s), each the best of
    three back-to-back batches."""
    nb = 512 * 1024 * 1024
    a = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)

    def best(fn, reps):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / reps * 1e-3)
        return min(ts)

    copy_s = best(lambda: b.copy_(a), 10)
    del a, b
    m = 8192
    x = torch.randn((m, m), device=dev).to(torch.float16)
    y = torch.randn((m, m), device=dev).to(torch.float16)
    gemm_s = best(lambda: torch.matmul(x, y), 10)
    del x, y
    return {"copy_gbs": round(2 * nb / copy_s / 1e9, 1),
            "gemm_f16_tflops": round(2.0 * m ** 3 / gemm_s / 1e12, 1),
            "how": "512 MiB device copy (read + write bytes); torch.matmul fp16 8192^3; best of 3x10"}


def cpu_model():
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def python_oracle_times():
    """Wall-clock seconds of the pure-Python oracle (dictionary map, fp64
    per-pair products), one thread, on the three uniform workloads."""
    from threadpoolctl import threadpool_limits

    import workloads
    from oracle import oracle as O
    res = []
    with threadpool_limits(limits=1):
        for name in ("c1_16_8", "c2_64_64", "c3_128_128"):
            wl = workloads.make(name)
            L = wl.layers[0]
            t = time.perf_counter()
            kmap = O.kernel_map(wl.coords, wl.grid, L.ksize, wl.batch)
            map_s = time.perf_counter() - t
            t = time.perf_counter()
            O.submconv(wl.coords, wl.feats, L.W, L.bias, wl.grid, L.ksize, wl.batch, kmap=kmap)
            conv_s = time.perf_counter() - t
            pairs = O.active_pairs(kmap)
            res.append({"workload": name, "rows": wl.n, "active_pairs": pairs, "map_s": round(map_s, 3),
                        "conv_s": round(conv_s, 3),
                        "conv_tflops": round(2.0 * pairs * L.cin * L.cout / conv_s / 1e12, 7)})
            print(f"[bench] python oracle {name}: map {map_s:.2f} s, conv {conv_s:.2f} s",
                  file=sys.stderr, flush=True)
    return {"threads": 1, "runs": res}


def coord_op_bench(args, sc, wl, coords, feats, dev):
    import ctypes
    import numpy as np
    import torch
    op = args.op
    n, C = wl.n, feats.shape[1]
    lib = sc.load_library()
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    if op == "downsample":
        def step():
            sc.downsample(coords, feats, wl.grid, wl.batch)
        t = time.perf_counter()
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        steps = max(3, args.steps // 10)
        t = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        step_us = (time.perf_counter() - t) / steps * 1e6
        g = (ctypes.c_int32 * 3)(*wl.grid)
        h = ctypes.c_void_p()
        sc._check(lib.submconv_downsample_plan(sc._ptr(coords), n, wl.batch, g, st, ctypes.byref(h)))
        m = int(lib.submconv_downsample_rows(h))
        pf = torch.empty((m, C), dtype=torch.float16, device=dev)
        k_us = _time(lambda: sc._check(lib.submconv_downsample_max(h, sc._ptr(feats), C, sc._ptr(pf), st)),
                     args.steps, args.warmup, torch)
        lib.submconv_downsample_free(h)
        alg = n * C * 2 + m * C * 2 + n * 4 + (m + 1) * 4
        detail = {"parents": m}
    else:
        cc = torch.empty((8 * n, 4), dtype=torch.int32, device=dev)
        cf = torch.empty((8 * n, C), dtype=torch.float16, device=dev)

        def step():
            sc._check(lib.submconv_subdivide(sc._ptr(coords), n, sc._ptr(feats), C, sc._ptr(cc),
                                             sc._ptr(cf), st))
        k_us = _time(step, args.steps, args.warmup, torch)
        step_us = k_us
        alg = n * 16 + n * C * 2 + 8 * n * 16 + 8 * n * C * 2
        detail = {"children": 8 * n}
    gbs = alg / (k_us * 1e-6) / 1e9
    print(f"[bench] {op}: step {step_us:.1f} us, kernel {k_us:.1f} us, {gbs:.0f} GB/s", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        if op == "downsample":
            ns = n
            t = time.perf_counter()
            O.downsample_np(wl.coords, wl.feats, wl.grid)
            what = "all sites, numpy sorting unique + maximum scatter"
        else:
            ns = min(n, 50000)
            t = time.perf_counter()
            O.subdivide(wl.coords[:ns], wl.feats[:ns], wl.grid)
            what = f"first {ns} sites, per-site loop"
        cpu_s = time.perf_counter() - t
        cpu = {"value": round(ns / cpu_s / 1e6, 4), "unit": "Msites/s", "cores": 1, "kind": "oracle",
               "sample": f"{args.config}: {what} ({cpu_s * 1e3:.0f} ms)"}
    rec = {
        "metric": METRICS[op], "value": round(n / (step_us * 1e-6) / 1e6, 3), "unit": "Msites/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_us / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16 / int32",
        "data": "synthetic",
        "config": dict({"workload": f"{args.config}: {n} sites, grid {wl.grid[0]}^3, batch {wl.batch}, C={C}",
                        "op": op}, **detail),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": KERNELS[op],
                     "kernel_us": round(k_us, 2), "algorithmic_bytes": alg},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c3_128_128")
    ap.add_argument("--op", default="forward", choices=list(METRICS))
    ap.add_argument("--dtype", default="fp16", choices=["fp16", "bf16"],
                    help="element type of features and weights (forward and input gradient)")
    ap.add_argument("--morton", action="store_true")
    ap.add_argument("--sorted-keys", action="store_true",
                    help="build the map with the sorted-key lookup instead of the hash table")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a device copy of this many MiB (counter calibration)")
    ap.add_argument("--scrub-mib", type=int, default=512,
                    help="also time the op's kernels with a device copy of this many MiB before "
                         "each launch, which evicts the L2s and the 256 MiB MALL (0: skip)")
    ap.add_argument("--python-oracle", action="store_true",
                    help="also time the pure-Python oracle, single-threaded, on c1_16_8, "
                         "c2_64_64 and c3_128_128 (tens of seconds)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import submanifold_sparse_convolution_hash_amd as sc
    import workloads

    sc.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.make(args.config)
    L = wl.layers[0]
    op = args.op
    coords = torch.from_numpy(wl.coords).to(dev)
    feats = torch.from_numpy(wl.feats).to(dev)
    W = torch.from_numpy(L.W).to(dev)
    if args.dtype == "bf16":
        if op not in ("forward", "backward_input"):
            raise SystemExit("--dtype bf16 applies to the forward and the input gradient")
        feats, W = feats.to(torch.bfloat16), W.to(torch.bfloat16)
    bias = None if L.bias is None else torch.from_numpy(L.bias).to(dev)
    g_np = np.random.default_rng(12345).standard_normal((wl.n, L.cout)).astype(np.float16)
    grad_out = torch.from_numpy(g_np).to(dev).to(feats.dtype)
    torch.cuda.synchronize()
    print(f"[bench] {args.config} {op}: N={wl.n} {L.cin}->{L.cout} ksize={L.ksize}", file=sys.stderr, flush=True)

    if op in ("downsample", "subdivide"):
        return coord_op_bench(args, sc, wl, coords, feats, dev)

    # kernel-map build (cold, including allocation and the one host wait)
    build_ms = []
    km = None
    for _ in range(5):
        if km is not None:
            km.free()
        torch.cuda.synchronize()
        t = time.perf_counter()
        km = sc.build_map(coords, wl.grid, wl.batch, morton=args.morton, sorted_keys=args.sorted_keys)
        torch.cuda.synchronize()
        build_ms.append((time.perf_counter() - t) * 1e3)
    pairs = km.active_pairs(L.ksize)
    flops = 2.0 * pairs * L.cin * L.cout
    # the kernel the op's forward takes: the staged one on a map with a plan
    cin_t, cout_t = (L.cout, L.cin) if op == "backward_input" else (L.cin, L.cout)
    staged = None
    if op in ("forward", "backward_input") and L.ksize == 3 and km.staged()[0] > 0 and \
            sc.forward_kernel(wl.n, pairs, cin_t, cout_t, 3) == 2:
        staged = km.staged()
    kname = ("k_fwd_staged_wide" if cout_t == 256 else "k_fwd_staged") if staged else KERNELS[op]
    # the weight gradient on the staged plan (dense maps, these shapes)
    if op == "backward_weight" and L.ksize == 3 and km.staged()[0] > 0 and \
            (L.cin, L.cout) in ((32, 32), (64, 32), (32, 64)):
        staged = km.staged()
        kname = "k_bwd_weight_staged"

    # Steps and kernels call the C ABI directly (ctypes, arguments built
    # once): the Python binding's checks would add host time to every launch.
    import ctypes
    lib = sc.load_library()
    st = sc._stream(dev)
    P = ctypes.c_void_p
    dt = sc._DTYPES[feats.dtype]
    if op == "forward":
        out = torch.empty((wl.n, L.cout), dtype=feats.dtype, device=dev)
        wp = sc.prepare_weights(W)
        a_step = (km.handle, P(feats.data_ptr()), P(W.data_ptr()), sc._ptr(bias),
                  P(out.data_ptr()), L.cin, L.cout, L.ksize, dt, st)
        a_kern = (km.handle, P(feats.data_ptr()), wp.handle, sc._ptr(bias), P(out.data_ptr()), st)

        def step():
            sc._check(lib.submconv_forward_dtype(*a_step))

        def kernel():
            sc._check(lib.submconv_forward_prepared(*a_kern))
    elif op == "backward_input":
        out = torch.empty((wl.n, L.cin), dtype=feats.dtype, device=dev)
        wp = sc.prepare_weights(W, input_grad=True)
        a_step = (km.handle, P(grad_out.data_ptr()), P(W.data_ptr()), P(out.data_ptr()), L.cin,
                  L.cout, L.ksize, dt, st)
        a_kern = (km.handle, P(grad_out.data_ptr()), wp.handle, P(out.data_ptr()), st)

        def step():
            sc._check(lib.submconv_backward_input_dtype(*a_step))

        def kernel():
            sc._check(lib.submconv_backward_input_prepared(*a_kern))
    elif op == "forward_masked":
        out = torch.empty((wl.n, L.cout), dtype=torch.float16, device=dev)
        wp = sc.prepare_weights(W)
        mplan = sc.masked_plan(km)
        print(f"[bench] masked plan: {mplan.row_taps} row-taps executed for {pairs} pairs "
              f"({mplan.row_taps / pairs:.2f}x)", file=sys.stderr, flush=True)
        a_kern = (mplan.handle, P(feats.data_ptr()), wp.handle, sc._ptr(bias), P(out.data_ptr()), st)

        def step():
            wp.set(W)
            sc._check(lib.submconv_forward_masked(*a_kern))

        def kernel():
            sc._check(lib.submconv_forward_masked(*a_kern))
    else:
        out = torch.empty((27 if L.ksize == 3 else 1, L.cin, L.cout), dtype=torch.float32, device=dev)
        ws = int(lib.submconv_backward_weight_workspace_bytes(km.handle, L.cin, L.cout, L.ksize))
        work = torch.empty((max(ws, 1),), dtype=torch.uint8, device=dev)
        a_kern = (km.handle, P(feats.data_ptr()), P(grad_out.data_ptr()), P(out.data_ptr()),
                  P(work.data_ptr()), L.cin, L.cout, L.ksize, st)

        def step():
            sc._check(lib.submconv_backward_weight(*a_kern))

        kernel = step

    for _ in range(args.warmup):
        step()
    # The K timed steps, then K launches of the op's dominant kernel alone,
    # each run back to back inside one event pair on the launch stream
    # (torch's current stream), with a synchronisation before the steps and
    # after the kernels and no idle time between the two runs.
    torch.cuda.synchronize()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    t = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    for _ in range(args.steps):
        kernel()
    e2.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t) * 1e3 / args.steps
    step_us = e0.elapsed_time(e1) / args.steps * 1e3
    k_us = e1.elapsed_time(e2) / args.steps * 1e3
    ms_step = step_us / 1e3
    print(f"[bench] step {step_us:.1f} us (wall of steps and kernels {wall_ms * 1e3:.1f} us)",
          file=sys.stderr, flush=True)
    alg_bytes = algorithmic_bytes(op, wl.n, L.cin, L.cout, L.ksize, args.morton, bias is not None,
                                  pairs, km.tile_rows, staged)
    achieved_gbs = alg_bytes / (k_us * 1e-6) / 1e9
    print(f"[bench] {op} kernels {k_us:.1f} us, {achieved_gbs:.0f} GB/s algorithmic", file=sys.stderr, flush=True)

    cold = None
    if args.scrub_mib > 0:
        # the same launches with every cache cold: a copy of scrub_mib MiB
        # between launches, outside the event pair
        nb = args.scrub_mib * 1024 * 1024 // 2
        sa = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(3)
        sb = torch.empty_like(sa)
        n_cold = max(1, min(args.steps, 50))
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_cold)]
        torch.cuda.synchronize()
        for a, b in evs:
            sb.copy_(sa)
            a.record()
            kernel()
            b.record()
        torch.cuda.synchronize()
        cold_us = sorted(a.elapsed_time(b) for a, b in evs)[n_cold // 2] * 1e3
        del sa, sb
        cold = {"kernel_us_median": round(cold_us, 2), "launches": n_cold, "scrub_mib": args.scrub_mib,
                "achieved_gbs": round(alg_bytes / (cold_us * 1e-6) / 1e9, 1)}
        print(f"[bench] {op} kernels after a {args.scrub_mib} MiB scrub: {cold_us:.1f} us (median of "
              f"{n_cold})", file=sys.stderr, flush=True)

    if args.calib_copy_mib > 0:
        # one plain device copy of known size, for scaling the HBM counters
        nb = args.calib_copy_mib * 1024 * 1024
        a = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    ceil = measured_ceilings(torch, dev)
    print(f"[bench] ceilings: copy {ceil['copy_gbs']:.0f} GB/s, fp16 GEMM {ceil['gemm_f16_tflops']:.0f} "
          f"TFLOP/s", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import cpu as oc
        t = time.perf_counter()
        kmap = oc.kernel_map(wl.coords, wl.grid, wl.batch, L.ksize)
        map_s = time.perf_counter() - t
        times = []
        for _ in range(2):
            t = time.perf_counter()
            if op in ("forward", "forward_masked"):
                oc.submconv_rows(kmap, wl.feats, L.W, L.bias)
            elif op == "backward_input":
                oc.backward_input_rows(wl.coords, wl.grid, wl.batch, L.ksize, g_np, L.W)
            else:
                oc.backward_weight(kmap, wl.feats, g_np)
            times.append(time.perf_counter() - t)
        conv_s = min(times)
        what = {"forward": "conv", "forward_masked": "conv", "backward_input": "input gradient",
                "backward_weight": "weight gradient"}[op]
        cpu = {"value": round(flops / conv_s / 1e12, 6), "unit": "TFLOP/s", "cores": oc.num_threads(),
               "kind": "oracle", "cpu_model": cpu_model(),
               "sample": f"full {args.config} layer, all {wl.n} rows: C oracle (fp64, sort+bsearch map, "
                         f"naive loops, OpenMP); {what} {conv_s * 1e3:.0f} ms (best of 2), "
                         f"map {map_s * 1e3:.0f} ms"}
        print(f"[bench] cpu oracle {what} {conv_s:.2f} s", file=sys.stderr, flush=True)

    py_oracle = None
    if args.python_oracle:
        py_oracle = python_oracle_times()

    # The bound is the larger of the two floors: the compulsory bytes at peak
    # HBM bandwidth, or the compulsory FLOPs (2 x active pairs x Cin x Cout)
    # at the dense fp16 MFMA peak, i.e. whether the layer's FLOPs per
    # algorithmic byte exceed the ridge of 2500 TFLOP/s / 8 TB/s = 312.5.
    k_tflops = flops / (k_us * 1e-6) / 1e12
    if flops / alg_bytes > MFMA_F16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        bound_fields = {"bound": "mfma", "achieved": round(k_tflops, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(k_tflops / MFMA_F16_PEAK_TFLOPS, 4)}
    else:
        bound_fields = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4)}

    extra = {}
    if op == "forward_masked":
        extra = {"masked_row_taps": mplan.row_taps, "padding_factor": round(mplan.row_taps / pairs, 3)}
    rec = {
        "metric": METRICS[op],
        "value": round(flops / (ms_step * 1e-3) / 1e12, 4),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{args.dtype} (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: SubMConv3d {L.ksize}x{L.ksize}x{L.ksize}, grid {wl.grid[0]}^3, "
                               f"batch {wl.batch}, N={wl.n}, Cin={L.cin}, Cout={L.cout}, warm kernel map",
                   "op": op, "active_pairs": pairs, "morton": bool(args.morton), **extra,
                   "map_lookup": "sorted keys" if args.sorted_keys else "hash"},
        "roofline": dict(bound_fields, **{
                     "traffic": measured_traffic(args.config, op, args.morton),
                     "kernel": kname, "kernel_us": round(k_us, 2),
                     "algorithmic_bytes": alg_bytes,
                     "hbm_frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                     "mfma_effective_frac": round(k_tflops / MFMA_F16_PEAK_TFLOPS, 4),
                     "measured_ceilings": dict(ceil, **{
                         "frac_of_copy": round(achieved_gbs / ceil["copy_gbs"], 4),
                         "mfma_effective_frac_of_gemm": round(
                             flops / (k_us * 1e-6) / 1e12 / ceil["gemm_f16_tflops"], 4)})}),
        "map_build_ms": round(float(np.median(build_ms)), 3),
        "mall_cold": cold,
        "cpu_baseline": cpu,
    }
    if op == "forward" and args.config == "c3_128_128":
        rec["context"] = {
            "source": "trellis_sparse_mlx README, Performance table (MLX on Apple GPUs; other "
                      "hardware, context only, not a target)",
            "conv_ms": {"M3 Ultra (80 GPU cores)": 13.8, "M4 Pro (~20 GPU cores)": 55.1},
            "this_step_ms": round(ms_step, 5)}
    if py_oracle is not None:
        rec["python_oracle"] = py_oracle
    print(json.dumps(rec), flush=True)
    if op == "forward_masked":
        mplan.free()
    km.free()
    return 0


if __name__ == "__main__":
    sys.exit(main())
