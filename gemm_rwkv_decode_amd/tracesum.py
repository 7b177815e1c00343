"""Summaries of rocprofv3 output for the measurement records.

python -m gemm_rwkv_decode_amd.tracesum trace DIR   per-kernel durations from the
    kernel-trace CSV under DIR (rocprofv3 --kernel-trace --output-format csv),
    grouped by kernel instance and grid: dispatches, average, median, minimum
    in microseconds.
python -m gemm_rwkv_decode_amd.tracesum pmc DIR COUNTER...   per-dispatch medians
    of the listed counters from the counter-collection CSV under DIR, grouped
    the same way.
python -m gemm_rwkv_decode_amd.tracesum mfma DIR   matrix-core busy fraction and
    issued fp16 work per matrix-core kernel instance (counter CSV under DIR).
python -m gemm_rwkv_decode_amd.tracesum mfma-record DIR   the same for the
    M = 64 instances as a JSON record with the hash of the kernel's sources.
python -m gemm_rwkv_decode_amd.tracesum record TRACE_DIR FETCH_DIR WRITE_DIR KERNEL
    GRID SHAPE ALG_BYTES   the roofline record of one kernel instance (name
    containing KERNEL, grid GRID): its average and median duration in the trace,
    and its FETCH_SIZE / WRITE_SIZE per dispatch scaled by what the same
    counters read for the 64 MiB copy kernel in the same runs (JSON).

Only reads files; it measures nothing itself.
"""
import csv
import glob
import os
import statistics
import sys
from collections import defaultdict


def _find(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits


def trace(d):
    rows = defaultdict(list)
    for f in _find(d, "kernel_trace.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
                grid = r.get("Grid_Size") or r.get("Grid_Size_X")
                wg = r.get("Workgroup_Size") or r.get("Workgroup_Size_X")
                rows[(r["Kernel_Name"], grid, wg)].append(dur)
    out = []
    for (k, g, w), v in rows.items():
        out.append((sum(v), k, g, w, len(v), statistics.fmean(v), statistics.median(v), min(v)))
    out.sort(reverse=True)
    print(f"{'kernel':<70} {'grid':>10} {'wg':>5} {'n':>6} {'avg_us':>9} {'med_us':>9} "
          f"{'min_us':>9}")
    for _, k, g, w, n, a, m, lo in out:
        k = k if len(k) <= 70 else k[:67] + "..."
        print(f"{k:<70} {g:>10} {w:>5} {n:>6} {a:>9.3f} {m:>9.3f} {lo:>9.3f}")


def pmc(d, counters):
    rows = defaultdict(lambda: defaultdict(list))
    for f in _find(d, "counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r.get("Counter_Name")
                if name not in counters:
                    continue
                key = (r["Kernel_Name"], r.get("Grid_Size"), r.get("Dispatch_Id"))
                rows[key[:2]][name].append((key[2], float(r["Counter_Value"])))
    print(f"{'kernel':<70} {'grid':>10} {'n':>6} " + " ".join(f"{c:>22}" for c in counters))
    for (k, g), per in sorted(rows.items()):
        n = max(len({d for d, _ in v}) for v in per.values())
        meds = []
        for c in counters:
            by_disp = defaultdict(float)
            for disp, val in per.get(c, []):
                by_disp[disp] += val  # sum over the counter's instances in one dispatch
            meds.append(statistics.median(by_disp.values()) if by_disp else float("nan"))
        k = k if len(k) <= 70 else k[:67] + "..."
        print(f"{k:<70} {g:>10} {n:>6} " + " ".join(f"{m:>22.1f}" for m in meds))


def _durations(d, kernel, grid):
    out = []
    for f in _find(d, "kernel_trace.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                g = r.get("Grid_Size") or r.get("Grid_Size_X")
                if kernel in r["Kernel_Name"] and str(g) == str(grid):
                    out.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    return out


def _counter(d, counter, kernel, grid=None):
    per = defaultdict(float)
    for f in _find(d, "counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") != counter or kernel not in r["Kernel_Name"]:
                    continue
                if grid is not None and str(r.get("Grid_Size")) != str(grid):
                    continue
                per[r.get("Dispatch_Id")] += float(r["Counter_Value"])
    return list(per.values())


def record(trace_dir, fetch_dir, write_dir, kernel, grid, shape, alg_bytes):
    import hashlib
    import json
    dur = _durations(trace_dir, kernel, grid)
    fetch = statistics.median(_counter(fetch_dir, "FETCH_SIZE", kernel, grid))
    write = statistics.median(_counter(write_dir, "WRITE_SIZE", kernel, grid))
    copy_bytes = 64 << 20
    cf = statistics.median(_counter(fetch_dir, "FETCH_SIZE", "k_probe_copy"))
    cw = statistics.median(_counter(write_dir, "WRITE_SIZE", "k_probe_copy"))
    fs, ws = copy_bytes / 1024 / cf, copy_bytes / 1024 / cw
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    h = hashlib.sha256()
    for f in ("gemm_rwkv_decode_amd/csrc/rq_gemv.hip", "gemm_rwkv_decode_amd/csrc/rq_common.h"):
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    tb = int(round((fetch * fs + write * ws) * 1024))
    print(json.dumps({
        "kernel": kernel, "shape": shape, "grid": int(grid),
        "trace_dispatches": len(dur), "trace_avg_us": round(statistics.fmean(dur), 3),
        "trace_median_us": round(statistics.median(dur), 3),
        "fetch_size_kib_median": fetch, "write_size_kib_median": write,
        "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
        "scale_reference": f"the 64 MiB copy kernel of the same runs reads FETCH_SIZE = "
                           f"{cf:.0f} KiB and writes WRITE_SIZE = {cw:.0f} KiB per dispatch",
        "bytes_per_launch": tb, "algorithmic_bytes_per_launch": int(alg_bytes),
        "source_sha256": h.hexdigest()}, indent=1))


# the matrix-core kernel's sources, hashed into its counter record
MM_SOURCES = ("gemm_rwkv_decode_amd/csrc/rq_gemm_impl.h",
              "gemm_rwkv_decode_amd/csrc/rq_gemm_plan.h",
              "gemm_rwkv_decode_amd/csrc/rq_common.h")


def mfma(d, as_json=False):
    """Matrix-core busy fraction per matrix-core kernel instance and grid:
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs), and the
    issued fp16 work (SQ_INSTS_VALU_MFMA_MOPS_F16 x 512 flops).  as_json: a
    record of the M = 64 (four M-tile) instances with the hash of the
    matrix-core kernel's sources."""
    need = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F16", "GRBM_GUI_ACTIVE")
    per = defaultdict(lambda: defaultdict(lambda: defaultdict(float)))
    for f in _find(d, "counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                c = r.get("Counter_Name")
                if c not in need or "k_mm" not in r["Kernel_Name"]:
                    continue
                per[(r["Kernel_Name"], r.get("Grid_Size"))][r.get("Dispatch_Id")][c] += \
                    float(r["Counter_Value"])
    if as_json:
        import hashlib
        import json
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        h = hashlib.sha256()
        for f in MM_SOURCES:
            with open(os.path.join(root, f), "rb") as fh:
                h.update(fh.read())
        rec = {}
        for (k, g), disp in sorted(per.items()):
            if "Mm<0, 4," not in k:
                continue
            util = [v["SQ_VALU_MFMA_BUSY_CYCLES"] / (v["GRBM_GUI_ACTIVE"] / 8 * 1024)
                    for v in disp.values() if v["GRBM_GUI_ACTIVE"] > 0]
            name = k.replace("void rq::", "rq::").split("(")[0]
            rec[f"{name} grid {g}"] = {"dispatches": len(disp),
                                        "mfma_busy": round(statistics.median(util), 4)}
        print(json.dumps({"what": "matrix-core busy fraction of the int4-g64 M=64 step's "
                                  "kernel instances (medians per dispatch)",
                          "kernels": rec, "source_sha256": h.hexdigest()}, indent=1))
        return
    print(f"{'kernel':<70} {'grid':>10} {'n':>6} {'mfma_util':>10} {'issued_GFLOP':>13}")
    for (k, g), disp in sorted(per.items()):
        util = [v["SQ_VALU_MFMA_BUSY_CYCLES"] / (v["GRBM_GUI_ACTIVE"] / 8 * 1024)
                for v in disp.values() if v["GRBM_GUI_ACTIVE"] > 0]
        gf = [v["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512 / 1e9 for v in disp.values()]
        k = k.replace("void rq::", "rq::")
        k = k if len(k) <= 70 else k[:67] + "..."
        print(f"{k:<70} {g:>10} {len(disp):>6} {100 * statistics.median(util):>9.1f}% "
              f"{statistics.median(gf):>13.2f}")


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "trace":
        trace(sys.argv[2])
    elif len(sys.argv) >= 4 and sys.argv[1] == "pmc":
        pmc(sys.argv[2], sys.argv[3:])
    elif len(sys.argv) == 3 and sys.argv[1] == "mfma":
        mfma(sys.argv[2])
    elif len(sys.argv) == 3 and sys.argv[1] == "mfma-record":
        mfma(sys.argv[2], as_json=True)
    elif len(sys.argv) == 9 and sys.argv[1] == "record":
        record(*sys.argv[2:9])
    else:
        raise SystemExit(__doc__)
