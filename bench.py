"""Benchmark: int4 group-64 decode GEMV over the full weight stream of a
13.3B-shaped RWKV-7 model (61 layers x 6 quantized matrices at width 4096,
FFN 16384), on one MI355X.

One step = one pass of the decode hot path: every one of the 366 matrices is
multiplied by its own activation row (M = 1) through rq_gemv, in layer order,
on one stream.  Inputs (6.5 GB of packed codes and scales, the activations)
are generated on the GPU from their seeds and are resident in HBM before the
timed region.  The same step at M = 32 (rq_gemm_smallm, matrix cores) gives
the TFLOP/s figure.

Prints one JSON line (rank 0):
  value       algorithmic bytes per step / step time, GB/s (M = 1)
  roofline    the dominant kernel (FFN 16384x4096 or 4096x16384) against 8 TB/s
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
    ap.add_argument("--graph", action="store_true",
                    help="replay the step as a captured graph instead of direct launches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=2,
                    help="layers of the step the CPU oracle times")
    ap.add_argument("--layers", type=int, default=None, help="(testing) fewer layers")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build runs the hot path on a single "
              "MI355X and has no multi-GPU mode (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import gemm_rwkv_decode_amd as rq
    from gemm_rwkv_decode_amd import synth as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = S.CONFIGS[4]
    fmt = S.INT4_G64
    mats = cfg.matrices()
    if args.layers is not None:
        mats = [m for m in mats if m[0] < args.layers]
    nlayers = len({m[0] for m in mats})

    # ---- inputs, resident in HBM --------------------------------------------
    t0 = time.time()
    W = []
    for (l, mi, N, K) in mats:
        W.append(S.gen_matrix(cfg.cid, l, mi, N, K, fmt, device=dev))
    X1 = [S.gen_x(cfg, l, mi, 1, K, device=dev) for (l, mi, N, K) in mats]
    X32 = [S.gen_x(cfg, l, mi, 32, K, device=dev) for (l, mi, N, K) in mats]
    Y1 = [torch.empty((1, N), dtype=torch.float32, device=dev) for (_, _, N, _) in mats]
    Y32 = [torch.empty((32, N), dtype=torch.float32, device=dev) for (_, _, N, _) in mats]
    torch.cuda.synchronize()
    log(f"generated {len(mats)} matrices in {time.time() - t0:.1f}s")

    weight_bytes = sum(fmt.weight_bytes(N, K) for (_, _, N, K) in mats)

    def step_bytes(M):
        return weight_bytes + sum(2 * M * K + 4 * M * N for (_, _, N, K) in mats)

    flops_per_m = sum(2 * N * K for (_, _, N, K) in mats)

    def step(M):
        X, Y = (X1, Y1) if M == 1 else (X32, Y32)
        f = rq.rq_gemv if M < 16 else rq.rq_gemm_smallm
        for p, x, y, (_, _, N, K) in zip(W, X, Y, mats):
            f(p.qweight, p.scales, None, x, y, M, N, K, 4, 64, 0)

    def timed(M, steps, warmup, graph):
        for _ in range(warmup):
            step(M)
        torch.cuda.synchronize()
        run = lambda: step(M)  # noqa: E731
        if graph:
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                step(M)  # the split-K workspace is allocated outside capture
                torch.cuda.synchronize()
                with torch.cuda.graph(g, stream=s):
                    step(M)
            torch.cuda.synchronize()
            run = g.replay
            for _ in range(warmup):
                run()
            torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps):
            run()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / steps

    # ---- M = 1: the headline ------------------------------------------------
    log("timing M=1")
    sec1 = timed(1, args.steps, args.warmup, args.graph)
    gbs = step_bytes(1) / sec1 / 1e9

    # ---- per-kernel durations with events (same launches, same stream) -----
    log("per-kernel events")
    shapes = {}
    for _ in range(3):
        evs = []
        stream = torch.cuda.current_stream()
        for p, x, y, (_, _, N, K) in zip(W, X1, Y1, mats):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            rq.rq_gemv(p.qweight, p.scales, None, x, y, 1, N, K, 4, 64, 0)
            b.record(stream)
            evs.append(((N, K), a, b))
        torch.cuda.synchronize()
        for key, a, b in evs:
            shapes.setdefault(key, []).append(a.elapsed_time(b) * 1e-3)
    per_kernel = {}
    for (N, K), ts in shapes.items():
        avg = sum(ts) / len(ts)
        nbytes = fmt.weight_bytes(N, K) + 2 * K + 4 * N
        per_kernel[f"{N}x{K}"] = {"avg_us": avg * 1e6, "launches_per_step": len(ts) // 3,
                                  "bytes": nbytes, "GBps": nbytes / avg / 1e9}
    dom = max(per_kernel.items(), key=lambda kv: kv[1]["avg_us"] * kv[1]["launches_per_step"])
    dom_name, dom_v = dom

    # ---- M = 32 (matrix cores) ---------------------------------------------
    log("timing M=32")
    sec32 = timed(32, args.m32_steps, 2, args.graph)
    tflops32 = 32 * flops_per_m / sec32 / 1e12

    # ---- CPU oracle on a bounded sample of the same step --------------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        sample = [i for i, m in enumerate(mats) if m[0] < args.cpu_layers]
        log(f"cpu oracle on {len(sample)} matrices")
        host = [(W[i].qweight.cpu().numpy(), W[i].scales.cpu().numpy(),
                 X1[i].cpu().numpy(), mats[i]) for i in sample]
        t = time.perf_counter()
        for q, s, x, (_, _, N, K) in host:
            oracle.gemv_ref(q, s, None, x, N, K, 4, 64, 0, threads=1)
        dt = time.perf_counter() - t
        sb = sum(fmt.weight_bytes(N, K) + 2 * K + 4 * N for (_, _, _, (_, _, N, K)) in host)
        cpu = {"value": round(sb / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"first {args.cpu_layers} layers ({len(sample)} matrices, "
                         f"{sb / 1e6:.1f} MB) of the same M=1 step, single thread, "
                         f"{dt:.1f} s"}

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
        "config": {"workload": "RWKV-7 13.3B-shaped decode weight stream, int4 sym g64",
                   "layers": nlayers, "matrices": len(mats), "M": 1,
                   "shapes": "per layer 4x(4096x4096), 16384x4096, 4096x16384",
                   "bytes_per_step": step_bytes(1)},
        "m32": {"entry": "rq_gemm_smallm", "ms_per_step": round(sec32 * 1e3, 4),
                "tflops": round(tflops32, 2),
                "pct_of_fp16_mfma_peak": round(100 * tflops32 / FP16_MFMA_PEAK_TFLOPS, 2),
                "GBps": round(step_bytes(32) / sec32 / 1e9, 2)},
        "per_kernel_m1": {k: {kk: round(vv, 3) if isinstance(vv, float) else vv
                              for kk, vv in v.items()} for k, v in per_kernel.items()},
        "roofline": {"bound": "hbm", "kernel": f"rq_gemv int4 g64 {dom_name} M=1",
                     "achieved": round(dom_v["GBps"], 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dom_v["GBps"] / HBM_PEAK_GBS, 4),
                     "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
