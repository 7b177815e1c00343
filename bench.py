"""Benchmark: int4 group-64 decode GEMV over the full weight stream of a
13.3B-shaped RWKV-7 model (61 layers x 6 quantized matrices at width 4096,
FFN 16384), on one MI355X.

One step = one pass of the decode hot path: every one of the 366 layer
matrices is multiplied by its own activation row (M = 1), in dependency order,
on one stream (gemm_rwkv_decode_amd.step, kind "layer": receptance/key/value
of a layer in one rq_gemv_batched launch, the rest through rq_gemv).  The same
step followed by the 65536x4096 vocabulary head (6.68 GB) is reported beside
it.  Inputs (packed codes and scales, the activations) are generated on the
GPU from their seeds and are resident in HBM before the timed region.  The
same step at M = 16, 32 and 64 (rq_gemm_smallm, matrix cores) gives the
TFLOP/s figures; M = 32 is the headline one.

Prints one JSON line (rank 0):
  value       algorithmic bytes per step / step time, GB/s (M = 1, no head)
  roofline    the dominant kernel (FFN 4096x16384 or 16384x4096) against 8 TB/s:
              algorithmic bytes of one launch / its average time, from events
              around back-to-back launches of that shape (the per-shape leg;
              `--roofline-only` runs that leg alone, for the kernel trace)
  cpu_baseline the CPU oracle, single-threaded, on a bounded sample of the same
              step (its first layers), GB/s of algorithmic bytes
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "int4-g64 GEMV HBM GB/s (% of peak) at D=4096 M=1; TFLOP/s at M=32"
# The dominant kernel's record from rocprofv3 (its duration in a trace of the
# per-shape leg alone, and HBM bytes per launch from the memory counters);
# valid only while the kernel's sources hash to the recorded value.
RECORD_FILE = os.path.join(ROOT, "profiles", "rq_gemv_int4g64_4096x16384_m1_roofline.json")
# matrix-core busy fractions of the M = 64 step from rocprofv3 counters; valid
# only while the matrix-core kernel's sources hash to the recorded value
MFMA_RECORD_FILE = os.path.join(ROOT, "profiles", "rq_gemm_int4g64_m64_mfma_record.json")
MM_SOURCES = ["gemm_rwkv_decode_amd/csrc/rq_gemm_impl.h",
              "gemm_rwkv_decode_amd/csrc/rq_gemm_plan.h",
              "gemm_rwkv_decode_amd/csrc/rq_common.h"]
KERNEL_SOURCES = ["gemm_rwkv_decode_amd/csrc/rq_gemv.hip",
                  "gemm_rwkv_decode_amd/csrc/rq_common.h"]


def kernel_source_hash(files=None):
    import hashlib
    h = hashlib.sha256()
    for f in files or KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded(shape):
    """The rocprofv3 record of the dominant kernel for `shape`, or {} if absent
    or the kernel has changed since it was taken."""
    try:
        with open(RECORD_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return {}
    if t.get("source_sha256") != kernel_source_hash() or t.get("shape") != shape:
        return {}
    return t


def recorded_mfma_busy():
    """{kernel instance: matrix-core busy fraction} of the M = 64 step, or None
    if absent or the kernel has changed since the counters were taken."""
    try:
        with open(MFMA_RECORD_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash(MM_SOURCES):
        return None
    return {k: v["mfma_busy"] for k, v in t.get("kernels", {}).items()}


HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--m32-steps", type=int, default=20)
    ap.add_argument("--stream", dest="graph", action="store_false",
                    help="direct launches on one stream instead of replaying each step as "
                         "a captured HIP graph (the default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=6,
                    help="layers of the step the CPU oracle times")
    ap.add_argument("--layers", type=int, default=None, help="(testing) fewer layers")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8 W8A16 step and the 5-/6-bit shapes")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the fp16 dense and tensor-parallel shard measurements")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first copy 64 MiB with rq_probe_copy (the reference kernel "
                         "for scaling the memory-traffic counters)")
    ap.add_argument("--roofline-only", action="store_true",
                    help="run only the per-shape leg whose dominant kernel gives the "
                         "roofline (for tracing exactly those launches)")
    ap.add_argument("--no-small", action="store_true",
                    help="skip the 768-wide single-matrix and 0.1B-shaped step legs")
    return ap.parse_args()


def host_cpu():
    """Model name and usable core count of the host CPU."""
    name = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"model": name, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the hot path runs on a single MI355X and "
              "there is no multi-GPU mode (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import gemm_rwkv_decode_amd as rq
    from gemm_rwkv_decode_amd import step as ST
    from gemm_rwkv_decode_amd import synth as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        a = torch.ones(64 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(4):
            rq.lib().rq_probe_copy(a.data_ptr(), b.data_ptr(), 64 << 20,
                                   torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        del a, b
    cfg = S.CONFIGS["rwkv7-13.3b"]
    fmt = S.INT4_G64
    mats_all = cfg.matrices(with_head=True)
    if args.layers is not None:
        mats_all = [m for m in mats_all if m[0] < args.layers or m[1] == ST.HEAD]
    nlayers = len({m[0] for m in mats_all if m[1] != ST.HEAD})
    mfma_ms = [] if args.roofline_only else [16, 32, 64]

    # ---- inputs, resident in HBM --------------------------------------------
    t0 = time.time()
    W_all = [S.gen_matrix(cfg.key, l, mi, N, K, fmt, device=dev) for (l, mi, N, K) in mats_all]
    X_all = {M: [S.gen_x(cfg, l, mi, M, K, device=dev) for (l, mi, N, K) in mats_all]
             for M in [1] + mfma_ms}
    Y_all = {M: [torch.empty((M, N), dtype=torch.float32, device=dev)
                 for (_, _, N, _) in mats_all] for M in [1] + mfma_ms}
    torch.cuda.synchronize()
    log(f"generated {len(mats_all)} matrices in {time.time() - t0:.1f}s")
    # the headline step: the layer matrices (the head is timed beside it)
    lay = [i for i, m in enumerate(mats_all) if m[1] != ST.HEAD]
    mats = [mats_all[i] for i in lay]
    W = [W_all[i] for i in lay]
    X = {M: [X_all[M][i] for i in lay] for M in X_all}
    Y = {M: [Y_all[M][i] for i in lay] for M in Y_all}

    def bytes_of(ms, M):
        return sum(fmt.weight_bytes(N, K) + 2 * M * K + 4 * M * N for (_, _, N, K) in ms)

    def step_bytes(M):
        return bytes_of(mats, M)

    flops_per_m = sum(2 * N * K for (_, _, N, K) in mats)

    def timed(kind, M, steps, warmup, graph, step=None):
        """Seconds per step.  Graph mode prepares the calls on a side stream,
        captures one step there and replays it.  step: (mats, W, X, Y) of
        another workload (default: this one at M)."""
        smats, sW, sX, sY = step if step is not None else (mats, W, X[M], Y[M])
        if graph:
            s = torch.cuda.Stream()
            calls = ST.step_calls(smats, sW, sX, sY, kind, stream=s)
            with torch.cuda.stream(s):
                for _ in range(warmup):
                    for c in calls:
                        c()
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    for c in calls:
                        c()
            torch.cuda.synchronize()
            run = g.replay
        else:
            calls = ST.step_calls(smats, sW, sX, sY, kind)

            def run():
                for c in calls:
                    c()
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps):
            run()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / steps, len(calls)

    # ---- M = 1: the headline (dependency-ordered decode step) ---------------
    scheds = {}
    with_head = None
    if not args.roofline_only:
        for kind in ST.KINDS:
            log(f"timing M=1 schedule {kind}")
            sec, ncalls = timed(kind, 1, args.steps, args.warmup, args.graph)
            scheds[kind] = {"launch_calls": ncalls, "ms_per_step": round(sec * 1e3, 4),
                            "GBps": round(step_bytes(1) / sec / 1e9, 2)}
        log("timing M=1 step with the head")
        sec, ncalls = timed("layer", 1, args.steps, args.warmup, args.graph,
                            step=(mats_all, W_all, X_all[1], Y_all[1]))
        hb = bytes_of(mats_all, 1)
        with_head = {"matrices": len(mats_all), "launch_calls": ncalls, "bytes_per_step": hb,
                     "ms_per_step": round(sec * 1e3, 4), "GBps": round(hb / sec / 1e9, 2),
                     "pct_of_hbm_peak": round(100 * hb / sec / 1e9 / HBM_PEAK_GBS, 2)}
        sec1 = scheds["layer"]["ms_per_step"] * 1e-3
        gbs = step_bytes(1) / sec1 / 1e9

    # ---- per-shape launch time: events around back-to-back launches of one
    # shape over all layers (distinct, cold matrices), same stream -----------
    log("per-shape events")
    per_kernel = {}
    groups = {}
    nbytes = {}

    def add(key, call, b):
        groups.setdefault(key, []).append(call)
        nbytes[key] = b

    by_layer = {}
    for i, (l, mi, N, K) in enumerate(mats_all):
        by_layer.setdefault(l, {})[mi] = i
    mats_pl, W_pl, X_pl, Y_pl = mats_all, W_all, X_all[1], Y_all[1]

    def mbytes(i):
        _, _, N, K = mats_pl[i]
        return fmt.weight_bytes(N, K) + 2 * K + 4 * N

    for l in sorted(by_layer):
        ix = by_layer[l]
        if ST.RECEPTANCE in ix:
            rkv = [ix[m] for m in (ST.RECEPTANCE, ST.KEY, ST.VALUE)]
            add("rkv batched 3x(4096x4096)",
                ST.step_calls([mats_pl[i] for i in rkv], [W_pl[i] for i in rkv],
                              [X_pl[i] for i in rkv], [Y_pl[i] for i in rkv], "layer")[0],
                sum(mbytes(i) for i in rkv))
        for m in (ST.OUTPUT, ST.FFN_KEY, ST.FFN_VALUE, ST.HEAD):
            if m in ix:
                i = ix[m]
                _, _, N, K = mats_pl[i]
                add(f"{N}x{K}", ST.step_calls([mats_pl[i]], [W_pl[i]], [X_pl[i]], [Y_pl[i]],
                                               "matrix")[0], mbytes(i))
    stream = torch.cuda.current_stream()
    for key, calls in groups.items():
        for c in calls[:4]:
            c()
        ts = []
        for _ in range(3 if len(calls) > 1 else 20):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for c in calls:
                c()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3 / len(calls))
        avg = min(ts)
        per_kernel[key] = {"us_per_launch": round(avg * 1e6, 3), "launches_per_step": len(calls),
                           "bytes": nbytes[key], "GBps": round(nbytes[key] / avg / 1e9, 1)}
    # the dominant kernel of the headline step (the head is not in it)
    dom_name, dom_v = max(((k, v) for k, v in per_kernel.items() if k != "65536x4096"),
                          key=lambda kv: kv[1]["us_per_launch"] * kv[1]["launches_per_step"])
    roofline = {"bound": "hbm", "kernel": f"int4 g64 GEMV {dom_name}, M=1",
                "achieved": dom_v["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom_v["GBps"] / HBM_PEAK_GBS, 4),
                "us_per_launch": dom_v["us_per_launch"], "bytes_per_launch": dom_v["bytes"],
                "timing": "HIP events around back-to-back launches of the shape over the "
                          "61 layers (distinct, cold matrices) on the launch stream",
                "traffic": recorded(dom_name).get("bytes_per_launch"),
                "traffic_unit": "HBM bytes per launch: FETCH_SIZE and WRITE_SIZE per "
                                "dispatch, each scaled by what it reads for a 64 MiB copy",
                "trace_avg_us": recorded(dom_name).get("trace_avg_us"),
                "trace_frac": (round(dom_v["bytes"] / recorded(dom_name)["trace_avg_us"]
                                     / 1e6 / HBM_PEAK_GBS * 1e3, 4)
                               if recorded(dom_name).get("trace_avg_us") else None),
                "trace_record": os.path.relpath(RECORD_FILE, ROOT)}
    if args.roofline_only:
        print(json.dumps({"metric": METRIC, "roofline_only": True, "roofline": roofline,
                          "per_shape_m1": per_kernel}), flush=True)
        return

    # ---- what this GPU sustains for the same step at M = 1: each launch's
    # bytes read by the plain streaming-read probe (cold, best launch shape),
    # and a graph of as many dependent empty launches ------------------------
    log("measured M=1 ceiling")
    from gemm_rwkv_decode_amd import probe as PR
    ceil_shapes = {}
    read_step_us = 0.0
    for key, v in per_kernel.items():
        if key == "65536x4096":
            continue
        t = PR.read_us(v["bytes"])
        ceil_shapes[key] = {"bytes": v["bytes"], "read_probe_us": round(t, 3),
                            "kernel_us": v["us_per_launch"],
                            "kernel_over_read": round(v["us_per_launch"] / t, 3)}
        read_step_us += t * v["launches_per_step"]
    chain = PR.chain_us(scheds["layer"]["launch_calls"])
    ceiling = {
        "read_probe_step_ms": round(read_step_us / 1e3, 4),
        "read_probe_step_GBps": round(step_bytes(1) / (read_step_us * 1e-6) / 1e9, 1),
        "headline_frac_of_read_probe_step": round(read_step_us * 1e-6 / sec1, 4),
        "empty_launch_chain_ms": round(chain / 1e3, 4),
        "per_shape": ceil_shapes,
        "what": "read_probe_step: the step's launches, each replaced by one plain streaming "
                "read of its bytes (rq_probe_read, cold buffers), back to back; "
                "empty_launch_chain: one graph replay of the step's launch count of "
                "dependent empty kernels (rq_probe_empty)"}

    # ---- the dense fp16 matrix-core rate of this GPU (rq_probe_mfma) --------
    sink = torch.zeros(2048, dtype=torch.float32, device=dev)
    pk = {}
    for shape, name in ((0, "v_mfma_f32_16x16x32_f16"), (1, "v_mfma_f32_32x32x16_f16")):
        fn = lambda: rq.lib().rq_probe_mfma(2048, 2000, shape, sink.data_ptr(),  # noqa: E731
                                            torch.cuda.current_stream().cuda_stream)
        fn()
        torch.cuda.synchronize()
        best = 1e9
        for _ in range(3):
            a = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            e.record()
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(e) * 1e-3)
        pk[name] = round(2048 * 4 * 2000 * 8 * 16384 / best / 1e12, 1)
    mfma_peak = max(pk.values())
    del sink

    # ---- M = 16, 32, 64 (matrix cores) ---------------------------------------
    mfma = {}
    for M in mfma_ms:
        log(f"timing M={M}")
        sec, ncalls = timed("layer", M, args.m32_steps, 2, args.graph)
        tf = M * flops_per_m / sec / 1e12
        sb = step_bytes(M)
        mfma[str(M)] = {"entry": "rq_gemm_smallm", "launch_calls": ncalls,
                        "ms_per_step": round(sec * 1e3, 4), "tflops": round(tf, 2),
                        "pct_of_fp16_mfma_peak": round(100 * tf / FP16_MFMA_PEAK_TFLOPS, 2),
                        "pct_of_measured_fp16_mfma_peak": round(100 * tf / mfma_peak, 2),
                        "GBps": round(sb / sec / 1e9, 2),
                        "pct_of_hbm_peak": round(100 * sb / sec / 1e9 / HBM_PEAK_GBS, 2),
                        "hbm_bound_ms": round(sb / HBM_PEAK_GBS / 1e6, 4),
                        "frac_of_hbm_roofline": round(sb / HBM_PEAK_GBS / 1e9 / sec, 4)}

    # ---- the 768-wide workloads: one 768x768 matrix, and the 0.1B-shaped
    # step (12 layers x 6 matrices) ---------------------------------------------
    small = None
    if not args.no_small:
        small = {}
        c0 = S.CONFIGS["gemv768"]
        w0 = S.gen_matrix(c0.key, 0, 0, 768, 768, fmt, device=dev)
        x0 = S.gen_x(c0, 0, 0, 1, 768, device=dev)
        y0 = torch.empty((1, 768), dtype=torch.float32, device=dev)
        b0 = fmt.weight_bytes(768, 768) + 2 * 768 + 4 * 768
        n_warm = 200
        log("768x768: one matrix, back-to-back calls")
        sec, _ = timed("matrix", 1, args.steps, 2, True,
                       step=([(i, 0, 768, 768) for i in range(n_warm)], [w0] * n_warm,
                             [x0] * n_warm, [y0] * n_warm))
        reps0 = 2000
        log(f"768x768: {reps0} distinct matrices")
        w0s = [S.gen_matrix(c0.key + "-replica", r, 0, 768, 768, fmt, device=dev)
               for r in range(reps0)]
        secc, _ = timed("matrix", 1, max(2, args.steps // 10), 1, True,
                        step=([(i, 0, 768, 768) for i in range(reps0)], w0s, [x0] * reps0,
                              [y0] * reps0))
        del w0s
        small["gemv768"] = {
            "workload": "single int4 g64 GEMV 768x768, M=1",
            "bytes_per_call": b0,
            "us_per_call_same_matrix": round(sec / n_warm * 1e6, 3),
            "cold": {"matrices": reps0, "bytes": reps0 * b0,
                     "us_per_call": round(secc / reps0 * 1e6, 3),
                     "GBps": round(reps0 * b0 / secc / 1e9, 1)},
            "timing": "graph replay of back-to-back rq_gemv calls"}
        c1 = S.CONFIGS["rwkv7-0.1b"]
        m1 = c1.matrices()
        nrep = 12
        log(f"0.1B-shaped step: {nrep} replicas")
        W1 = [[S.gen_matrix(f"{c1.key}-replica{r}", l, mi, N, K, fmt, device=dev)
               for (l, mi, N, K) in m1] for r in range(nrep)]
        X1 = [S.gen_x(c1, l, mi, 1, K, device=dev) for (l, mi, N, K) in m1]
        Y1 = [torch.empty((1, N), dtype=torch.float32, device=dev) for (_, _, N, _) in m1]
        b1 = bytes_of(m1, 1)
        sec_w, nc = timed("layer", 1, args.steps, args.warmup, args.graph,
                          step=(m1, W1[0], X1, Y1))
        mc = [(l + c1.layers * r, mi, N, K) for r in range(nrep) for (l, mi, N, K) in m1]
        sec_c, _ = timed("layer", 1, max(2, args.steps // 4), 2, args.graph,
                         step=(mc, [w for r in range(nrep) for w in W1[r]], X1 * nrep,
                               Y1 * nrep))
        sec_c /= nrep
        del W1
        small["rwkv7-0.1b"] = {
            "workload": "RWKV-7 0.1B-shaped decode step, int4 g64, M=1: 12 layers x "
                        "(4 x 768x768, 3072x768, 768x3072)",
            "launch_calls": nc, "bytes_per_step": b1,
            "cache_resident": {"ms_per_step": round(sec_w * 1e3, 4),
                               "GBps": round(b1 / sec_w / 1e9, 1),
                               "note": "the same 45 MB replica every step (fits the "
                                       "256 MB last-level cache)"},
            "cold": {"replicas": nrep, "ms_per_step": round(sec_c * 1e3, 4),
                     "GBps": round(b1 / sec_c / 1e9, 1),
                     "note": f"{nrep} distinct replicas in turn "
                             f"({nrep * b1 / 1e6:.0f} MB between reuses)"}}
        torch.cuda.empty_cache()

    # ---- FP8 E4M3 per-tensor weights (W8A16), M = 1 --------------------------
    # The page's FP8 model shape: width 4096, 32 layers.  Eight distinct weight
    # sets are cycled over the 32 layers: 1.07 GB between reuses of a set,
    # four times the 256 MB MALL, so every byte still comes from HBM.
    fp8 = None
    if not args.no_fp8:
        log("FP8 step")
        f8 = S.FP8_E4M3
        f8_layers, f8_sets = 32, 8
        lay = [(mi, N, K) for (l, mi, N, K) in cfg.matrices(with_head=False) if l == 0]
        W8s = {(s8, mi): S.gen_matrix("rwkv7-7.2b-fp8", s8, mi, N, K, f8, device=dev)
               for s8 in range(f8_sets) for (mi, N, K) in lay}
        mats8 = [(l, mi, N, K) for l in range(f8_layers) for (mi, N, K) in lay]
        W8 = [W8s[(l % f8_sets, mi)] for (l, mi, N, K) in mats8]
        X8 = [S.gen_x(cfg, l, mi, 1, K, device=dev) for (l, mi, N, K) in mats8]
        Y8 = [torch.empty((1, N), dtype=torch.float32, device=dev) for (_, _, N, _) in mats8]
        calls8 = ST.step_calls(mats8, W8, X8, Y8, "layer")
        for _ in range(args.warmup):
            for c in calls8:
                c()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(args.steps):
            for c in calls8:
                c()
        torch.cuda.synchronize()
        sec8 = (time.perf_counter() - t) / args.steps
        b8 = sum(f8.weight_bytes(N, K) + 2 * K + 4 * N for (_, _, N, K) in mats8)
        # the page's concurrency test decodes 64 sequences at once: M = 64 on
        # the matrix cores (grouped r/k/v)
        X64 = [S.gen_x(cfg, l, mi, 64, K, device=dev) for (l, mi, N, K) in mats8]
        Y64 = [torch.empty((64, N), dtype=torch.float32, device=dev) for (_, _, N, _) in mats8]
        calls64 = ST.step_calls(mats8, W8, X64, Y64, "layer")
        for c in calls64:
            c()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(args.m32_steps):
            for c in calls64:
                c()
        torch.cuda.synchronize()
        sec64 = (time.perf_counter() - t) / args.m32_steps
        f64 = 64 * sum(2 * N * K for (_, _, N, K) in mats8)
        b64 = sum(f8.weight_bytes(N, K) + 2 * 64 * K + 4 * 64 * N for (_, _, N, K) in mats8)
        del X64, Y64, calls64
        shapes8 = {}
        for (mi, N, K) in lay[3:]:  # output projection, FFN key, FFN value
            cs = [ST.step_calls([m], [W8[i]], [X8[i]], [Y8[i]], "matrix")[0]
                  for i, m in enumerate(mats8) if m[1] == mi]
            for c in cs[:4]:
                c()
            best = 1e9
            for _ in range(3):
                a = torch.cuda.Event(enable_timing=True)
                e = torch.cuda.Event(enable_timing=True)
                a.record(torch.cuda.current_stream())
                for c in cs:
                    c()
                e.record(torch.cuda.current_stream())
                torch.cuda.synchronize()
                best = min(best, a.elapsed_time(e) * 1e-3 / len(cs))
            mb = f8.weight_bytes(N, K) + 2 * K + 4 * N
            shapes8[f"{N}x{K}"] = {"us_per_launch": round(best * 1e6, 3),
                                   "GBps": round(mb / best / 1e9, 1)}
        fp8 = {"workload": "RWKV-7 7.2B-shaped FP8 E4M3 per-tensor W8A16 decode weight "
                           "stream: 32 layers x (4 x 4096x4096, 16384x4096, 4096x16384), "
                           "8 distinct weight sets cycled (1.07 GB between reuses)",
               "entry": "rq_gemv / rq_gemv_batched (vector units)", "M": 1,
               "launch_mode": "stream",
               "launch_calls": len(calls8), "bytes_per_step": b8,
               "ms_per_step": round(sec8 * 1e3, 4), "GBps": round(b8 / sec8 / 1e9, 2),
               "pct_of_hbm_peak": round(100 * b8 / sec8 / 1e9 / HBM_PEAK_GBS, 2),
               "per_shape": shapes8,
               "m64": {"entry": "rq_gemm_smallm / rq_gemv_batched (matrix cores)",
                       "ms_per_step": round(sec64 * 1e3, 4),
                       "tflops": round(f64 / sec64 / 1e12, 2),
                       "GBps": round(b64 / sec64 / 1e9, 2)}}
        del W8s, W8, X8, Y8, calls8
        torch.cuda.empty_cache()

    # ---- 5- and 6-bit asymmetric codes, M = 1: launch time per shape --------
    # Twelve distinct matrices per shape (over 500 MB between reuses).
    hib = None
    if not args.no_fp8:
        log("5-/6-bit shapes")
        hib = {}
        for f in (S.ASYM5_G32, S.ASYM6_G32):
            for (N, K) in ((16384, 4096), (4096, 16384)):
                Wh = [S.gen_matrix("rwkv7-13.3b-hib", r, 4, N, K, f, device=dev) for r in range(12)]
                xh = S.gen_x(cfg, 0, 4, 1, K, device=dev)
                yh = torch.empty((1, N), dtype=torch.float32, device=dev)
                cs = [ST.step_calls([(0, 4, N, K)], [w], [xh], [yh], "matrix")[0] for w in Wh]
                for c in cs:
                    c()
                best = 1e9
                for _ in range(3):
                    a = torch.cuda.Event(enable_timing=True)
                    e = torch.cuda.Event(enable_timing=True)
                    a.record(torch.cuda.current_stream())
                    for c in cs * 2:
                        c()
                    e.record(torch.cuda.current_stream())
                    torch.cuda.synchronize()
                    best = min(best, a.elapsed_time(e) * 1e-3 / (2 * len(cs)))
                mb = f.weight_bytes(N, K) + 2 * K + 4 * N
                hib[f"{f.tag} {N}x{K}"] = {"us_per_launch": round(best * 1e6, 3),
                                           "bytes": mb, "GBps": round(mb / best / 1e9, 1)}
                del Wh, cs
        torch.cuda.empty_cache()

    # ---- context: the same products in fp16 dense (torch F.linear), and one
    # GPU's share of an 8-way tensor-parallel split -------------------------
    def launch_time(calls, reps=3):
        """Best average seconds per call over back-to-back runs of `calls`."""
        for c in calls[:4]:
            c()
        best = 1e9
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            a.record(torch.cuda.current_stream())
            for c in calls:
                c()
            e.record(torch.cuda.current_stream())
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(e) * 1e-3 / len(calls))
        return best

    dense = None
    if not args.no_context:
        log("fp16 dense comparison")
        dense = {}
        for (N, K) in ((4096, 4096), (16384, 4096), (4096, 16384)):
            reps = max(2, (1 << 30) // (2 * N * K))  # >= 1 GB of fp16 weights between reuses
            Wd = [torch.randn((N, K), device=dev).half() for _ in range(reps)]
            Wq = [S.gen_matrix("rwkv7-13.3b-dense", r, 4, N, K, fmt, device=dev)
                  for r in range(reps)]
            for M in (1, 32):
                xd = S.gen_x(cfg, 0, 4, M, K, device=dev)
                yd = torch.empty((M, N), dtype=torch.float16, device=dev)
                yq = torch.empty((M, N), dtype=torch.float32, device=dev)
                tf = launch_time([(lambda w=w: torch.matmul(xd, w.t(), out=yd)) for w in Wd])
                entry = "rq_gemv" if M == 1 else "rq_gemm_smallm"
                tq = launch_time([rq.prepare(entry, w.qweight, w.scales, None, xd, yq, M, N, K,
                                             4, 64, 0) for w in Wq])
                dense[f"{N}x{K} M={M}"] = {
                    "fp16_us": round(tf * 1e6, 3), "int4g64_us": round(tq * 1e6, 3),
                    "int4g64_entry": entry, "speedup": round(tf / tq, 3),
                    "fp16_GBps": round((2 * N * K + 2 * M * K + 2 * M * N) / tf / 1e9, 1)}
            del Wd, Wq
            torch.cuda.empty_cache()

    tp8 = None
    if not args.no_context:
        log("tensor-parallel shard shapes")
        tp8 = {}
        # column shards (receptance/key/value/output rows, FFN key rows) and row
        # shards (output and FFN value along K) of an 8-way split, M = 1
        for (N, K, what) in ((512, 4096, "column shard of a 4096x4096 projection"),
                             (2048, 4096, "column shard of the FFN key"),
                             (4096, 512, "row shard of the output projection"),
                             (4096, 2048, "row shard of the FFN value")):
            reps = max(2, (600 << 20) // fmt.weight_bytes(N, K))
            Wt = [S.gen_matrix("rwkv7-13.3b-tp8", r, 0, N, K, fmt, device=dev) for r in range(reps)]
            xt = S.gen_x(cfg, 0, 0, 1, K, device=dev)
            yt = torch.empty((1, N), dtype=torch.float32, device=dev)
            t = launch_time([rq.prepare("rq_gemv", w.qweight, w.scales, None, xt, yt, 1, N, K,
                                        4, 64, 0) for w in Wt])
            mb = fmt.weight_bytes(N, K) + 2 * K + 4 * N
            tp8[f"{N}x{K}"] = {"what": what, "us_per_launch": round(t * 1e6, 3),
                               "GBps": round(mb / t / 1e9, 1)}
            del Wt
        torch.cuda.empty_cache()

    # ---- context: the other workload shapes of the pages, same layer schedule
    others = None
    if not args.no_context:
        others = {}
        for wkey in ("rwkv7-1.5b", "rwkv7-2.9b"):
            c2 = S.CONFIGS[wkey]
            m2 = c2.matrices()
            for f2 in c2.formats:
                log(f"workload {wkey} {f2.tag}")
                W2 = [S.gen_matrix(c2.key, l, mi, N, K, f2, device=dev) for (l, mi, N, K) in m2]
                wb = sum(f2.weight_bytes(N, K) for (_, _, N, K) in m2)
                fl = sum(2 * N * K for (_, _, N, K) in m2)
                for M2 in c2.ms:
                    X2 = [S.gen_x(c2, l, mi, M2, K, device=dev) for (l, mi, N, K) in m2]
                    Y2 = [torch.empty((M2, N), dtype=torch.float32, device=dev)
                          for (_, _, N, _) in m2]
                    sec, ncalls = timed("layer", M2, args.m32_steps, 2, args.graph,
                                        step=(m2, W2, X2, Y2))
                    nb = wb + sum(2 * M2 * K + 4 * M2 * N for (_, _, N, K) in m2)
                    others[f"{wkey} {f2.tag} M={M2}"] = {
                        "layers": c2.layers, "width": c2.width, "launch_calls": ncalls,
                        "ms_per_step": round(sec * 1e3, 4), "GBps": round(nb / sec / 1e9, 1),
                        "tflops": round(M2 * fl / sec / 1e12, 2)}
                    del X2, Y2
                del W2
                torch.cuda.empty_cache()

    # ---- CPU oracle on a bounded sample of the same step --------------------
    cpu = cpu_threads = None
    if not args.no_cpu_baseline:
        import oracle
        sample = [i for i, m in enumerate(mats) if m[0] < args.cpu_layers]
        log(f"cpu oracle on {len(sample)} matrices")
        host = [(W[i].qweight.cpu().numpy(), W[i].scales.cpu().numpy(),
                 X[1][i].cpu().numpy(), mats[i]) for i in sample]
        t = time.perf_counter()
        for q, s, x, (_, _, N, K) in host:
            oracle.gemv_ref(q, s, None, x, N, K, 4, 64, 0, threads=1)
        dt = time.perf_counter() - t
        sb = sum(fmt.weight_bytes(N, K) + 2 * K + 4 * N for (_, _, _, (_, _, N, K)) in host)
        cpu = {"value": round(sb / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle", "host_cpu": host_cpu(),
               "sample": f"first {args.cpu_layers} layers ({len(sample)} matrices, "
                         f"{sb / 1e6:.1f} MB) of the same M=1 step, single thread, "
                         f"{dt:.1f} s"}
        # the same sample over disjoint row ranges on P threads (the oracle
        # unchanged; P capped at this GPU's share of host cores)
        P = max(1, min(16, os.cpu_count() or 1))
        t = time.perf_counter()
        for q, s, x, (_, _, N, K) in host:
            oracle.gemv_ref(q, s, None, x, N, K, 4, 64, 0, threads=P)
        dtp = time.perf_counter() - t
        cpu_threads = {"value": round(sb / dtp / 1e9, 4), "unit": "GB/s", "cores": P,
                       "kind": "oracle", "seconds": round(dtp, 2)}

    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec1 * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 weights x f16 activations, f32 accumulate",
        "data": "synthetic (seeded, generated on the GPU)",
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "launch_mode": "graph" if args.graph else "stream",
        "schedule": "per layer: one grouped launch for receptance/key/value, then output, "
                    f"FFN key, FFN value ({scheds['layer']['launch_calls']} launches per "
                    "step)",
        "schedules_m1": scheds,
        "config": {"workload": "RWKV-7 13.3B-shaped decode weight stream, int4 sym g64: "
                               "61 layers x (4 x 4096x4096, 16384x4096, 4096x16384)",
                   "layers": nlayers, "matrices": len(mats), "M": 1,
                   "bytes_per_step": step_bytes(1)},
        "with_head_m1": dict(with_head, workload="the same step followed by the 65536x4096 "
                                                 "vocabulary head"),
        "m32": mfma["32"],
        "mfma_m": mfma,
        "fp16_mfma_peak_measured_tflops": {"best": mfma_peak, "by_instruction": pk,
                                           "probe": "rq_probe_mfma, 2048 workgroups"},
        "mfma_utilization_m64": {
            "value": round(mfma["64"]["tflops"] / mfma_peak, 4),
            "what": "achieved TFLOP/s of the M=64 step / measured dense fp16 peak",
            "counter_busy": recorded_mfma_busy(),
            "counter_busy_what": "SQ_VALU_MFMA_BUSY_CYCLES per SIMD-cycle of each M=64 "
                                 "kernel instance (rocprofv3 record "
                                 + os.path.relpath(MFMA_RECORD_FILE, ROOT) + ")"},
        "small_workloads_m1": small,
        "fp8_w8a16_m1": fp8,
        "asym_5_6_bit_m1": hib,
        "per_shape_m1": per_kernel,
        "measured_ceiling_m1": ceiling,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_oracle_threads": cpu_threads,
        "vs_fp16_dense": dense,
        "tp8_shard_shapes_m1": tp8,
        "other_workloads": others,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
