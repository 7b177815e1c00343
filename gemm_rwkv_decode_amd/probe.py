"""Roofline probes on the current GPU (include/rq_probe.h).

python -m gemm_rwkv_decode_amd.probe  prints one JSON object:
  empty_us      back-to-back launch interval of an empty kernel
  read          for each size, the best streaming-read rate over a sweep of
                launch shapes, with launches rotating over buffers whose total
                exceeds the 256 MB last-level cache (cold reads)
Sizes default to one 4096x4096 and one 16384x4096 int4-g64 matrix (codes and
scales) and 1 GiB.

--sync adds "sync": the cost of cross-workgroup signalling (one arrival per
workgroup after a __threadfence() against after device-scope coherent writes,
per launch of 256..2048 workgroups) and the latency of one grid-wide barrier
among co-resident workgroups, both ways, with the exchanged data checked.
--mfma adds "mfma": the dense fp16 matrix-core rate (v_mfma_f32_16x16x32_f16).
--valu adds "valu": the issue cost, in cycles at 2.4 GHz per wave instruction,
of each vector instruction kind the product kernels use.
--overlap adds "overlap": the duration of matrix-core work alone, vector work
alone, both interleaved in every wave, and both in separate waves of a
workgroup, per SIMD and MFMA slot.
"""
import argparse
import json
import time

import torch

from . import lib


def _time_launches(fn, n):
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / n


def probe(sizes=(8912896, 35651584, 1 << 30), cold_bytes=1 << 30,
          shapes=((256, 256), (512, 256), (1024, 256), (2048, 256), (4096, 256),
                  (512, 512), (1024, 512), (256, 1024), (512, 1024))):
    L = lib()
    stream = torch.cuda.current_stream().cuda_stream
    sink = torch.empty(8192, dtype=torch.int32, device="cuda")
    out = {"device": torch.cuda.get_device_name(), "read": []}
    out["empty_us"] = _time_launches(lambda i: L.rq_probe_empty(stream), 2000) * 1e6
    for size in sizes:
        nbuf = max(1, -(-cold_bytes // size)) if size < cold_bytes else 2
        bufs = [torch.empty(size, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
        for b in bufs:
            b.fill_(1)
        best = None
        rows = []
        for blocks, threads in shapes:
            def fn(i, blocks=blocks, threads=threads):
                L.rq_probe_read(bufs[i % nbuf].data_ptr(), size, sink.data_ptr(), blocks,
                                threads, stream)
            fn(0)
            n = max(8, 2 * nbuf)
            t = _time_launches(fn, n)
            gbs = size / t / 1e9
            rows.append({"blocks": blocks, "threads": threads, "us": t * 1e6, "GBps": gbs})
            if best is None or gbs > best["GBps"]:
                best = rows[-1]
        out["read"].append({"bytes": size, "buffers": nbuf, "best": best, "sweep": rows})
        del bufs
        torch.cuda.empty_cache()
    return out


def read_us(size, cold_bytes=1 << 30,
            shapes=((512, 256), (1024, 256), (2048, 256), (1024, 512), (512, 1024))):
    """Best time (us) of one streaming read of `size` bytes over a few launch
    shapes, launches rotating over buffers whose total exceeds the last-level
    cache (cold reads)."""
    L = lib()
    stream = torch.cuda.current_stream().cuda_stream
    sink = torch.empty(8192, dtype=torch.int32, device="cuda")
    nbuf = max(2, -(-cold_bytes // size))
    bufs = [torch.empty(size, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
    for b in bufs:
        b.fill_(1)
    best = None
    for blocks, threads in shapes:
        def fn(i, blocks=blocks, threads=threads):
            L.rq_probe_read(bufs[i % nbuf].data_ptr(), size, sink.data_ptr(), blocks,
                            threads, stream)
        fn(0)
        t = min(_time_launches(fn, 2 * nbuf) for _ in range(2))
        best = t if best is None else min(best, t)
    del bufs
    torch.cuda.empty_cache()
    return best * 1e6


def chain_us(launches, replays=20):
    """Time (us) of one graph replay of `launches` dependent empty launches:
    the floor a step of that many launches pays before moving any byte."""
    L = lib()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for _ in range(3):
            L.rq_probe_empty(s.cuda_stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for _ in range(launches):
                L.rq_probe_empty(s.cuda_stream)
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(replays):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t) / replays * 1e6


def sync_probe(grids=(256, 512, 1024, 2048), barrier_grids=(256, 512, 1024), rounds=1000,
               spin=1 << 20):
    L = lib()
    stream = torch.cuda.current_stream().cuda_stream
    out = {"signal": [], "barrier": []}
    empty = _time_launches(lambda i: L.rq_probe_empty(stream), 500)
    out["empty_us"] = empty * 1e6
    for G in grids:
        flags = torch.zeros(64 * (G + 1), dtype=torch.int32, device="cuda")
        row = {"blocks": G}
        for mode, name in ((0, "threadfence_us"), (1, "coherent_writes_us")):
            def fn(i, mode=mode):
                st = L.rq_probe_signal(flags.data_ptr(), mode, G, stream)
                assert st == 0, st
            fn(0)
            row[name] = min(_time_launches(fn, 50) for _ in range(3)) * 1e6
        row["fence_cost_per_workgroup_ns"] = (row["threadfence_us"] -
                                              row["coherent_writes_us"]) * 1e3 / G
        out["signal"].append(row)
    for G in barrier_grids:
        flags = torch.zeros(2048 + 65 * G, dtype=torch.int32, device="cuda")
        bad = torch.zeros(G, dtype=torch.int32, device="cuda")
        row = {"blocks": G, "rounds": rounds, "barriers": 2 * rounds}
        for mode, name in ((2, "coherent"), (3, "release_acquire"),
                           (4, "coherent_32_counters"), (5, "coherent_per_workgroup_words")):
            best = None
            for _ in range(3):
                flags.zero_()
                bad.zero_()
                torch.cuda.synchronize()
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                st = L.rq_probe_barrier(flags.data_ptr(), mode, G, rounds, spin,
                                        bad.data_ptr(), stream)
                b.record()
                torch.cuda.synchronize()
                if st != 0:
                    row[name] = {"status": st}
                    break
                t = a.elapsed_time(b) * 1e-3
                nb = bad.cpu()
                r = {"us_per_barrier": t / (2 * rounds) * 1e6,
                     "stale_reads": int((nb & 0xFFFF).sum()),
                     "gave_up": int((nb >> 16).sum())}
                if best is None or r["us_per_barrier"] < best["us_per_barrier"]:
                    best = r
            if best is not None:
                row[name] = best
        out["barrier"].append(row)
    return out


def mfma_probe(blocks=2048, iters=2000):
    L = lib()
    stream = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(blocks, dtype=torch.float32, device="cuda")
    out = {"blocks": blocks, "waves": blocks * 4, "shapes": []}
    for shape, name in ((0, "v_mfma_f32_16x16x32_f16"), (1, "v_mfma_f32_32x32x16_f16")):
        fn = lambda i: L.rq_probe_mfma(blocks, iters, shape, sink.data_ptr(), stream)  # noqa: E731
        fn(0)
        t = min(_time_launches(fn, 5) for _ in range(3))
        flops = blocks * 4 * iters * 8 * 16384
        out["shapes"].append({"instruction": name, "flops": flops, "us": t * 1e6,
                              "tflops": flops / t / 1e12})
    out["tflops"] = max(r["tflops"] for r in out["shapes"])
    return out


VALU_KINDS = ("v_and_b32", "v_lshrrev_b32", "v_perm_b32", "v_bitop3_b32", "v_pk_fma_f16",
              "v_pk_add_f16", "v_dot2c_f32_f16", "v_fma_mix_f32", "v_fma_f32", "v_cvt_f32_f16",
              "v_add_u32", "v_add_f32", "v_mul_f32", "v_mov_b32_dpp", "v_add_f32_dpp",
              "v_lshl_or_b32", "v_and_or_b32")
CLOCK_HZ = 2.4e9


def valu_probe(blocks=512, iters=1000):
    """Cycles (at 2.4 GHz) per wave instruction of each kind, 512-thread
    workgroups, two per CU (four waves per SIMD)."""
    L = lib()
    stream = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    waves_per_simd = blocks // 256 * 2
    out = {"blocks": blocks, "threads": 512, "waves_per_simd": waves_per_simd,
           "clock_hz": CLOCK_HZ, "cycles": {}}
    for op, name in enumerate(VALU_KINDS):
        fn = lambda i, op=op: L.rq_probe_valu(op, blocks, iters, sink.data_ptr(), stream)  # noqa: E731
        if fn(0) != 0:
            raise RuntimeError(f"rq_probe_valu({op}) failed")
        t = min(_time_launches(fn, 3) for _ in range(3))
        out["cycles"][name] = round(t * CLOCK_HZ / (iters * 64 * waves_per_simd), 2)
    return out


def overlap_probe(iters=2000):
    """Cycles (at 2.4 GHz) per SIMD and MFMA slot for matrix-core work alone
    (mode 0), vector work alone (1), both in every wave (2) and both in
    separate waves (3), for three kinds of vector work and 4 or 8 vector
    operations per MFMA, at two and four waves per SIMD."""
    L = lib()
    stream = torch.cuda.current_stream().cuda_stream
    rows = []
    for blocks in (256, 512):
        sink = torch.zeros(blocks, dtype=torch.float32, device="cuda")
        wps = blocks // 256 * 2
        for kind, kname in enumerate(("pk_fma_f16", "bit_ops", "fma_f32")):
            for per in (4, 8):
                row = {"waves_per_simd": wps, "vector_kind": kname, "vector_per_mfma": per}
                for mode, mname in enumerate(("mfma_only", "vector_only", "same_wave",
                                              "separate_waves")):
                    fn = lambda i, mode=mode: L.rq_probe_overlap(  # noqa: E731
                        mode, kind, per, blocks, iters, sink.data_ptr(), stream)
                    if fn(0) != 0:
                        raise RuntimeError("rq_probe_overlap failed")
                    t = min(_time_launches(fn, 2) for _ in range(3))
                    row[mname] = round(t * CLOCK_HZ / (iters * 8 * wps), 1)
                rows.append(row)
    return {"threads": 512, "clock_hz": CLOCK_HZ, "rows": rows}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--sizes", type=str, default=None,
                    help="comma-separated byte counts")
    ap.add_argument("--sync", action="store_true")
    ap.add_argument("--mfma", action="store_true")
    ap.add_argument("--no-read", action="store_true")
    ap.add_argument("--valu", action="store_true")
    ap.add_argument("--overlap", action="store_true")
    a = ap.parse_args()
    kw = {}
    if a.sizes:
        kw["sizes"] = tuple(int(s) for s in a.sizes.split(","))
    t = time.time()
    r = {} if a.no_read else probe(**kw)
    if a.mfma:
        r["mfma"] = mfma_probe()
    if a.sync:
        r["sync"] = sync_probe()
    if a.valu:
        r["valu"] = valu_probe()
    if a.overlap:
        r["overlap"] = overlap_probe()
    r["seconds"] = time.time() - t
    print(json.dumps(r), flush=True)


if __name__ == "__main__":
    main()
