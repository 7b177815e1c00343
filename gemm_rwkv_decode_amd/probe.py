"""Roofline probes on the current GPU (include/rq_probe.h).

python -m gemm_rwkv_decode_amd.probe  prints one JSON object:
  empty_us      back-to-back launch interval of an empty kernel
  read          for each size, the best streaming-read rate over a sweep of
                launch shapes, with launches rotating over buffers whose total
                exceeds the 256 MB last-level cache (cold reads)
Sizes default to one 4096x4096 and one 16384x4096 int4-g64 matrix (codes and
scales) and 1 GiB.
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--sizes", type=str, default=None,
                    help="comma-separated byte counts")
    a = ap.parse_args()
    kw = {}
    if a.sizes:
        kw["sizes"] = tuple(int(s) for s in a.sizes.split(","))
    t = time.time()
    r = probe(**kw)
    r["seconds"] = time.time() - t
    print(json.dumps(r), flush=True)


if __name__ == "__main__":
    main()
