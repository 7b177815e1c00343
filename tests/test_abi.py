"""librq's C interface on the CPU: the library loads, exports every function
include/rq.h declares, and rejects bad arguments on the host before any HIP
call (so these run without a GPU: fake, never-dereferenced addresses are
used).  The status values are the ones the header defines."""
import ctypes
import os
import re

import pytest
import torch

import gemm_rwkv_decode_amd as rq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rq.h")

A = 0x7F0000000000  # a 16-byte-aligned address that is never dereferenced


def declared_functions():
    import glob
    src = "".join(open(h).read() for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))))
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rq_[a-z_0-9]+)\s*\(", src)))


def header_enum(name):
    src = open(HEADER).read()
    m = re.search(r"\b" + name + r"\s*=\s*(\d+)", src)
    return int(m.group(1))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(rq.LIB_PATH):
        pytest.fail("librq.so is not built (run __graft_entry__.build())")
    return rq.lib()


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert set(names) >= {"rq_dequant", "rq_gemv", "rq_gemm_smallm", "rq_status_string",
                          "rq_version"}
    for n in names:
        assert hasattr(L, n), f"librq.so does not export {n}"


def test_status_values_match_header():
    for n in ["RQ_OK", "RQ_ERR_NULL", "RQ_ERR_SHAPE", "RQ_ERR_UNSUPPORTED", "RQ_ERR_ALIGN",
              "RQ_ERR_LAUNCH", "RQ_ERR_ALIAS", "RQ_ERR_DEVICE", "RQ_ERR_SCRATCH", "RQ_LAYOUT_SYM",
              "RQ_LAYOUT_ASYM_SB", "RQ_LAYOUT_FP8_TENSOR", "RQ_OUT_F32", "RQ_OUT_CODES_I8"]:
        assert getattr(rq, n) == header_enum(n), n
    assert rq.RQ_MAX_M == int(re.search(r"#define RQ_MAX_M (\d+)", open(HEADER).read()).group(1))


def test_version_and_strings(L):
    assert rq.rq_version() == (1 << 16) | 1
    seen = set()
    for s in range(9):
        t = rq.rq_status_string(s)
        assert t and t not in seen
        seen.add(t)
    assert rq.rq_status_string(99) == "unknown status"


def gemv_args(**kw):
    a = dict(qw=A, sc=A + (1 << 30), z=None, x=A + (2 << 30), y=A + (3 << 30), M=1, N=64,
             K=256, bits=4, group=64, layout=0)
    a.update(kw)
    return [a["qw"], a["sc"], a["z"], a["x"], a["y"], a["M"], a["N"], a["K"], a["bits"],
            a["group"], a["layout"], None]


def dq_args(**kw):
    a = dict(qw=A, sc=A + (1 << 30), z=None, out=A + (3 << 30), N=64, K=256, bits=4,
             group=64, layout=0, kind=0)
    a.update(kw)
    return [a["qw"], a["sc"], a["z"], a["out"], a["N"], a["K"], a["bits"], a["group"],
            a["layout"], a["kind"], None]


CASES = [
    ("null qweight", dict(qw=None), rq.RQ_ERR_NULL),
    ("null scales", dict(sc=None), rq.RQ_ERR_NULL),
    ("asym without zeros", dict(layout=1, group=32, K=512), rq.RQ_ERR_NULL),
    ("sym with zeros", dict(z=A + (4 << 30)), rq.RQ_ERR_UNSUPPORTED),
    ("3-bit codes", dict(bits=3), rq.RQ_ERR_UNSUPPORTED),
    ("int4 group 48", dict(group=48), rq.RQ_ERR_UNSUPPORTED),
    ("int4 group 16", dict(group=16), rq.RQ_ERR_UNSUPPORTED),
    ("int8 group 128", dict(bits=8, group=128), rq.RQ_ERR_UNSUPPORTED),
    ("unknown layout", dict(layout=3), rq.RQ_ERR_UNSUPPORTED),
    ("fp8 with a group", dict(layout=2, bits=8, group=64), rq.RQ_ERR_UNSUPPORTED),
    ("fp8 4-bit", dict(layout=2, bits=4, group=0), rq.RQ_ERR_UNSUPPORTED),
    ("fp8 with zeros", dict(layout=2, bits=8, group=0, z=A + (4 << 30)), rq.RQ_ERR_UNSUPPORTED),
    ("fp8 row not whole 16 bytes", dict(layout=2, bits=8, group=0, K=264), rq.RQ_ERR_SHAPE),
    ("sym group 0", dict(group=0), rq.RQ_ERR_UNSUPPORTED),
    ("int8 codes of exactly 2 GiB", dict(bits=8, group=16, N=131072, K=16384), rq.RQ_ERR_SHAPE),
    ("int4 codes of exactly 2 GiB", dict(N=262144, K=16384), rq.RQ_ERR_SHAPE),
    ("asym group 64", dict(layout=1, group=64, z=A + (4 << 30)), rq.RQ_ERR_UNSUPPORTED),
    ("asym 8-bit", dict(layout=1, group=32, bits=8, z=A + (4 << 30)), rq.RQ_ERR_UNSUPPORTED),
    ("K not a multiple of group", dict(K=96), rq.RQ_ERR_SHAPE),
    ("K below group", dict(K=32), rq.RQ_ERR_SHAPE),
    ("N zero", dict(N=0), rq.RQ_ERR_SHAPE),
    ("N negative", dict(N=-5), rq.RQ_ERR_SHAPE),
    ("asym K not whole superblocks", dict(layout=1, group=32, K=288, z=A + (4 << 30)),
     rq.RQ_ERR_SHAPE),
    ("misaligned qweight", dict(qw=A + 8), rq.RQ_ERR_ALIGN),
    ("misaligned scales", dict(sc=A + (1 << 30) + 2), rq.RQ_ERR_ALIGN),
    ("misaligned zeros", dict(layout=1, group=32, K=512, z=A + (4 << 30) + 4),
     rq.RQ_ERR_ALIGN),
]

GEMV_ONLY = [
    ("null x", dict(x=None), rq.RQ_ERR_NULL),
    ("null y", dict(y=None), rq.RQ_ERR_NULL),
    ("M zero", dict(M=0), rq.RQ_ERR_SHAPE),
    ("M above 64", dict(M=65), rq.RQ_ERR_SHAPE),
    ("x of exactly 2 GiB", dict(M=64, K=1 << 24), rq.RQ_ERR_SHAPE),
    ("y of exactly 2 GiB", dict(M=64, N=1 << 23), rq.RQ_ERR_SHAPE),
    ("misaligned x", dict(x=A + (2 << 30) + 2), rq.RQ_ERR_ALIGN),
    ("misaligned y", dict(y=A + (3 << 30) + 4), rq.RQ_ERR_ALIGN),
    ("y overlaps x", dict(y=A + (2 << 30) + 16), rq.RQ_ERR_ALIAS),
    ("y overlaps codes", dict(y=A + 64), rq.RQ_ERR_ALIAS),
    ("y overlaps scales", dict(y=A + (1 << 30)), rq.RQ_ERR_ALIAS),
]


def ws_args(ws=None, ws_bytes=0, **kw):
    """rq_gemm_smallm_ws arguments: those of gemv_args plus the workspace."""
    a = gemv_args(**kw)
    return a[:-1] + [ws, ws_bytes, None]


@pytest.mark.parametrize("fn", ["rq_gemv", "rq_gemm_smallm", "rq_gemm_smallm_noalloc",
                                "rq_gemm_smallm_ws"])
@pytest.mark.parametrize("what,kw,status", CASES + GEMV_ONLY, ids=[c[0] for c in CASES + GEMV_ONLY])
def test_product_rejects(L, fn, what, kw, status):
    args = ws_args(**kw) if fn == "rq_gemm_smallm_ws" else gemv_args(**kw)
    assert getattr(L, fn)(*args) == status, what


# rq_gemm_smallm_ws at a shape whose automatic choice splits K (int4 g64,
# 4096 x 16384, M = 32), with fake, disjoint addresses
SPLIT = dict(M=32, N=4096, K=16384)
WS = A + (5 << 30)

WS_CASES = [
    ("misaligned workspace", dict(ws=WS + 4, ws_bytes=1 << 26), rq.RQ_ERR_ALIGN),
    ("workspace overlaps y", dict(ws=A + (3 << 30) + 256, ws_bytes=1 << 26), rq.RQ_ERR_ALIAS),
    ("workspace overlaps x", dict(ws=A + (2 << 30), ws_bytes=1 << 26), rq.RQ_ERR_ALIAS),
    ("workspace overlaps codes", dict(ws=A, ws_bytes=1 << 26), rq.RQ_ERR_ALIAS),
    ("workspace one byte short", dict(ws=WS, ws_bytes=None), rq.RQ_ERR_SCRATCH),
    ("workspace of zero bytes", dict(ws=WS, ws_bytes=0), rq.RQ_ERR_SCRATCH),
]


@pytest.mark.parametrize("what,kw,status", WS_CASES, ids=[c[0] for c in WS_CASES])
def test_workspace_rejects(L, what, kw, status):
    """Workspace checks run on the host before any HIP call (a too-small
    workspace enqueues nothing)."""
    need = rq.rq_gemm_smallm_workspace_size(SPLIT["M"], SPLIT["N"], SPLIT["K"], 4, 64, 0)
    assert need > 0
    if kw.get("ws_bytes", 0) is None:
        kw = dict(kw, ws_bytes=need - 1)
    assert L.rq_gemm_smallm_ws(*ws_args(**kw, **SPLIT)) == status, what


def test_workspace_checked_only_where_used(L):
    """Only the bytes the call uses are checked against the operands: a
    workspace whose unused tail runs into y passes the host checks (and then
    reports the missing device here)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    need = rq.rq_gemm_smallm_workspace_size(SPLIT["M"], SPLIT["N"], SPLIT["K"], 4, 64, 0)
    y = A + (3 << 30)
    ws = y - need
    assert L.rq_gemm_smallm_ws(*ws_args(ws=ws, ws_bytes=need + 4096, **SPLIT)) == \
        rq.RQ_ERR_DEVICE
    assert L.rq_gemm_smallm_ws(*ws_args(ws=ws + 16, ws_bytes=need, **SPLIT)) == \
        rq.RQ_ERR_ALIAS


def test_workspace_size_on_the_host(L):
    """The size query matches the split the plan query reports: splits * M * N
    partial sums plus 64 KiB of arrival counters, 0 where K is kept whole, and
    never above RQ_GEMM_WORKSPACE_MAX_BYTES."""
    for (M, N, K) in ((32, 4096, 16384), (64, 4096, 16384), (32, 4096, 4096),
                      (16, 16384, 4096), (64, 1000, 4096), (3, 2048, 8192)):
        plan, splits = rq.gemm_config(M, N, K, 4, 64, 0)
        b = rq.rq_gemm_smallm_workspace_size(M, N, K, 4, 64, 0)
        assert b == (0 if splits == 1 else 65536 + 4 * splits * M * N), (M, N, K)
        assert b <= rq.RQ_GEMM_WORKSPACE_MAX_BYTES
    assert rq.rq_gemm_smallm_workspace_size(32, 4096, 16384, 4, 64, 0) > 0
    sz = ctypes.c_size_t(7)
    assert L.rq_gemm_smallm_workspace_size(0, 64, 256, 4, 64, 0, ctypes.byref(sz)) == \
        rq.RQ_ERR_SHAPE
    assert L.rq_gemm_smallm_workspace_size(1, 64, 256, 3, 64, 0, ctypes.byref(sz)) == \
        rq.RQ_ERR_UNSUPPORTED
    assert L.rq_gemm_smallm_workspace_size(1, 64, 256, 4, 64, 0, None) == rq.RQ_ERR_NULL


DQ_ONLY = [
    ("null out", dict(out=None), rq.RQ_ERR_NULL),
    ("unknown output kind", dict(kind=2), rq.RQ_ERR_UNSUPPORTED),
    ("fp8 codes output", dict(layout=2, bits=8, group=0, kind=1), rq.RQ_ERR_UNSUPPORTED),
    ("misaligned out", dict(out=A + (3 << 30) + 8), rq.RQ_ERR_ALIGN),
    ("out overlaps codes", dict(out=A + 16), rq.RQ_ERR_ALIAS),
]


@pytest.mark.parametrize("what,kw,status", CASES + DQ_ONLY, ids=[c[0] for c in CASES + DQ_ONLY])
def test_dequant_rejects(L, what, kw, status):
    assert L.rq_dequant(*dq_args(**kw)) == status, what


def test_valid_call_without_gpu_reports_device(L):
    """A valid call on a machine without a gfx950 device returns RQ_ERR_DEVICE
    (nothing is launched; the fake addresses are never touched)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert L.rq_gemv(*gemv_args()) == rq.RQ_ERR_DEVICE
    assert L.rq_gemm_smallm(*gemv_args(M=32)) == rq.RQ_ERR_DEVICE
    assert L.rq_gemm_smallm_noalloc(*gemv_args(M=32)) == rq.RQ_ERR_DEVICE
    assert L.rq_gemm_smallm_ws(*ws_args(M=32)) == rq.RQ_ERR_DEVICE
    assert L.rq_gemm_smallm_ws(*ws_args(ws=WS, ws_bytes=1 << 26, **SPLIT)) == rq.RQ_ERR_DEVICE
    assert L.rq_dequant(*dq_args()) == rq.RQ_ERR_DEVICE


def test_binding_rejects_host_tensors():
    import torch
    t = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError):
        rq.rq_dequant(t, t, None, t, 1, 32, 4, 32, 0)


class Prob(ctypes.Structure):
    _fields_ = [("qweight", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("N", ctypes.c_int), ("K", ctypes.c_int)]


def _probs(*kws):
    arr = (rq.RqProblem * len(kws))()
    for i, kw in enumerate(kws):
        a = dict(qw=A + (i << 32), sc=A + (i << 32) + (1 << 30), z=None,
                 x=A + (i << 32) + (2 << 30), y=A + (i << 32) + (3 << 30), N=64, K=256)
        a.update(kw)
        arr[i] = rq.RqProblem(a["qw"], a["sc"], a["z"], a["x"], a["y"], a["N"], a["K"])
    return arr


@pytest.mark.parametrize("what,probs,count,M,status", [
    ("null array", None, 1, 1, rq.RQ_ERR_NULL),
    ("zero count", [{}], 0, 1, rq.RQ_ERR_SHAPE),
    ("count above RQ_MAX_BATCH", [{}], 65, 1, rq.RQ_ERR_SHAPE),
    ("M above 64", [{}, {}], 2, 65, rq.RQ_ERR_SHAPE),
    ("second problem bad K", [{}, {"K": 96}], 2, 1, rq.RQ_ERR_SHAPE),
    ("second problem null x", [{}, {"x": None}], 2, 1, rq.RQ_ERR_NULL),
    ("outputs overlap", [{}, {"y": A + (3 << 30) + 64}], 2, 1, rq.RQ_ERR_ALIAS),
    ("output overlaps another's x", [{}, {"y": A + (2 << 30) + 32}], 2, 1, rq.RQ_ERR_ALIAS),
    ("misaligned y", [{}, {"y": A + (1 << 32) + (3 << 30) + 4}], 2, 1, rq.RQ_ERR_ALIGN),
])
def test_batched_rejects(L, what, probs, count, M, status):
    arr = None if probs is None else _probs(*probs)
    assert L.rq_gemv_batched(arr, count, M, 4, 64, 0, None) == status, what


def test_codes_of_2gib_rejected(L):
    # 65536 x 65536 int4 codes are exactly 2 GiB: beyond the 32-bit offsets
    assert L.rq_gemv(*gemv_args(N=65536, K=65536)) == rq.RQ_ERR_SHAPE


def test_missing_library_raises(monkeypatch):
    """No CPU fallback: without librq.so every entry point raises before any
    work is done."""
    import gemm_rwkv_decode_amd as pkg
    monkeypatch.setattr(pkg, "_lib", None)
    monkeypatch.setattr(pkg, "LIB_PATH", "/nonexistent/librq.so")
    t = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(pkg.RqLibraryMissing):
        pkg.rq_gemv(t, t, None, t, t, 1, 1, 32, 4, 32, 0)
    with pytest.raises(pkg.RqLibraryMissing):
        pkg.rq_gemm_smallm(t, t, None, t, t, 1, 1, 32, 4, 32, 0)
    with pytest.raises(pkg.RqLibraryMissing):
        pkg.rq_dequant(t, t, None, t, 1, 32, 4, 32, 0)
    # the grouped call checks its problem table (device tensors only) first
    with pytest.raises((pkg.RqLibraryMissing, ValueError)):
        pkg.rq_gemv_batched([(t, t, None, t, t, 1, 32)], 1, 4, 32, 0)


def test_host_tensors_are_refused(L):
    """The binding hands the library device memory only; host tensors are
    refused rather than computed on the CPU."""
    t = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU tensors only"):
        rq.rq_gemv(t, t, None, t, t, 1, 1, 32, 4, 32, 0)
    with pytest.raises(ValueError, match="GPU tensors only"):
        rq.rq_dequant(t, t, None, t, 1, 32, 4, 32, 0)


def test_gemm_config_on_the_host(L):
    """The plan query of rq_probe.h runs on the host: rq_gemm_smallm splits K
    for few long rows, rq_gemv's choice keeps K whole, and a K the matrix-core
    kernel cannot take (an odd number of groups) reports no plan."""
    plan, splits = rq.gemm_config(32, 4096, 16384, 4, 64, 0)
    assert 1 <= plan <= 18 and splits == 4
    plan2, splits2 = rq.gemm_config(32, 4096, 16384, 4, 64, 0, allow_split=False)
    assert 1 <= plan2 <= 18 and splits2 == 1
    assert rq.gemm_config(32, 4096, 64 * 7, 4, 64, 0) is None
    for M in (1, 16, 17, 32, 48, 49, 64):
        for (N, K) in ((4096, 4096), (16384, 4096), (4096, 16384), (65536, 4096)):
            p, s = rq.gemm_config(M, N, K, 4, 64, 0)
            assert 1 <= p <= 18 and s >= 1 and s * M * N * 4 <= 64 << 20
    with pytest.raises(rq.RqError):
        rq.gemm_config(0, 64, 256, 4, 64, 0)


# vector-unit launch shapes the chooser takes for the RWKV-7 widths at M = 1
# (lanes per row, 16-byte chunks per lane, rows per lane), as measured on MI355X
GEMV_SHAPES_M1 = [
    # (N, K, bits, group, layout) -> (lpr, cpl, npass)
    ((4096, 4096, 4, 64, 0), (16, 1, 2)),    # 512 workgroups of two rows per lane
    ((16384, 4096, 4, 64, 0), (16, 1, 4)),   # 1024 workgroups of four
    ((4096, 16384, 4, 64, 0), (32, 1, 4)),   # 512 workgroups keep four
    ((2048, 8192, 4, 64, 0), (32, 1, 2)),    # 256 -> 512 workgroups: two rows per lane
    ((2048, 8192, 8, 16, 0), (32, 1, 2)),
    ((2560, 10240, 4, 32, 1), (32, 1, 2)),
    ((768, 768, 4, 64, 0), (8, 1, 1)),
    ((3072, 768, 4, 64, 0), (8, 1, 1)),
    # heavier codes: at most 8 waves per workgroup
    ((4096, 16384, 5, 32, 1), (64, 1, 4)),
    ((4096, 16384, 6, 32, 1), (64, 1, 4)),
    ((2560, 10240, 5, 32, 1), (64, 1, 4)),
    ((16384, 4096, 8, 0, 2), (16, 2, 2)),
    ((4096, 4096, 8, 0, 2), (16, 2, 2)),
    ((4096, 16384, 8, 0, 2), (64, 1, 4)),
]


def test_gemv_config_on_the_host(L):
    """The kernel query of rq_probe.h: rq_gemv's choice of kernel and of the
    vector-unit launch shape, on the host."""
    for (N, K, bits, group, layout), shape in GEMV_SHAPES_M1:
        assert rq.gemv_config(1, N, K, bits, group, layout) == ("vector",) + shape, (N, K, bits)
    # matrix cores from M = 3 where the small-batch kernel takes K; the decode
    # kernel for int4 rows too long for the vector kernel's shapes at M = 1
    for M in (3, 4, 8, 16, 32, 64):
        assert rq.gemv_config(M, 4096, 4096, 4, 64, 0)[0] == "smallm_mfma"
        assert rq.gemv_config(M, 2560, 10240, 4, 32, 1)[0] == "smallm_mfma"
    assert rq.gemv_config(1, 4096, 65536, 4, 64, 0)[0] == "decode_mfma"
    # measured exceptions at M = 3..4: the 2.9B-shaped FFN key (asymmetric)
    # runs on the decode kernel, the 1.5B-shaped FFN value (int4) on the
    # vector units
    for M in (3, 4):
        assert rq.gemv_config(M, 10240, 2560, 4, 32, 1)[0] == "decode_mfma"
        assert rq.gemv_config(M, 2048, 8192, 4, 64, 0)[0] == "vector"
        assert rq.gemv_config(M, 2048, 2048, 8, 16, 0)[0] == "smallm_mfma"
        assert rq.gemv_config(M, 2048, 8192, 8, 16, 0)[0] == "smallm_mfma"
        assert rq.gemv_config(M, 2048, 2048, 4, 64, 0)[0] == "smallm_mfma"
    for M in (2, 5):
        assert rq.gemv_config(M, 2048, 8192, 4, 64, 0)[0] != "decode_mfma"
    assert rq.gemv_config(5, 2048, 8192, 4, 64, 0)[0] == "smallm_mfma"
    assert rq.gemv_config(1, 4096, 65536, 8, 16, 0)[0] == "smallm_mfma"
    # FP8 at M = 2 with a row the vector kernel cannot split
    assert rq.gemv_config(2, 4096, 16384, 8, 0, 2)[0] != "vector"
    with pytest.raises(rq.RqError):
        rq.gemv_config(0, 4096, 4096, 4, 64, 0)
    with pytest.raises(rq.RqError):
        rq.gemv_config(1, 4096, 4096 + 16, 4, 64, 0)  # not a whole number of groups
    with pytest.raises(rq.RqError):
        rq.gemv_config(1, 4096, 4096, 3, 64, 0)


def test_gemv_config_shapes_are_valid(L):
    """Every vector-unit shape the chooser returns splits the row into whole
    slices of at most the workgroup's waves, and at M = 1 a row of 16-chunk
    multiples with at least 512 row pairs takes 16 lanes per row."""
    widths = [(768, 768), (3072, 768), (768, 3072), (2048, 2048), (8192, 2048), (2048, 8192),
              (2560, 2560), (10240, 2560), (2560, 10240), (4096, 4096), (16384, 4096),
              (4096, 16384), (65536, 4096), (1000, 4096), (4096, 1024), (17, 256)]
    fmts = [(4, 64, 0, 32), (8, 16, 0, 16), (4, 32, 1, 32), (8, 0, 2, 16), (4, 128, 0, 32)]
    for M in (1, 2, 4, 8):
        for bits, group, layout, kpc in fmts:
            for N, K in widths:
                if layout == 1 and K % 256:
                    continue
                kern, lpr, cpl, npass = rq.gemv_config(M, N, K, bits, group, layout)
                if kern != "vector" or lpr == 0:
                    continue
                chunks = K // kpc
                mt = 1 if M == 1 else (2 if M == 2 else (4 if M <= 4 else 8))
                max_threads = 256 if mt * cpl >= 4 else (512 if mt * cpl >= 2 else 1024)
                assert lpr in (8, 16, 32, 64) and cpl in (1, 2, 4) and npass in (1, 2, 4, 8)
                assert chunks % (lpr * cpl) == 0, (M, N, K, bits, lpr, cpl)
                assert chunks // (lpr * cpl) <= max_threads // 64, (M, N, K, bits, lpr, cpl)
                if mt >= 4:
                    assert npass <= 4
                tuned = [sh for sh, _ in GEMV_SHAPES_M1 if sh[2] in (5, 6) or sh[4] == 2]
                if (M == 1 and chunks % 16 == 0 and chunks // 16 <= 16 and
                        (N + 15) // 16 >= 512 and (N, K, bits, group, layout) not in tuned):
                    assert (lpr, cpl) == (16, 1), (N, K, bits)


def test_gemv_config_follows_overrides(L, monkeypatch):
    """RQ_GEMV_KERNEL and RQ_GEMV_NPASS are applied by the query as by rq_gemv."""
    try:
        monkeypatch.setenv("RQ_GEMV_KERNEL", "1")
        rq.tuning_reload()
        assert rq.gemv_config(32, 4096, 4096, 4, 64, 0)[0] == "vector"
        monkeypatch.setenv("RQ_GEMV_KERNEL", "3")
        rq.tuning_reload()
        assert rq.gemv_config(1, 4096, 4096, 4, 64, 0)[0] == "smallm_mfma"
        monkeypatch.delenv("RQ_GEMV_KERNEL")
        monkeypatch.setenv("RQ_GEMV_NPASS", "8")
        rq.tuning_reload()
        assert rq.gemv_config(1, 4096, 4096, 4, 64, 0) == ("vector", 16, 1, 8)
    finally:
        monkeypatch.delenv("RQ_GEMV_KERNEL", raising=False)
        monkeypatch.delenv("RQ_GEMV_NPASS", raising=False)
        rq.tuning_reload()
    assert rq.gemv_config(1, 4096, 4096, 4, 64, 0) == ("vector", 16, 1, 2)


def test_probe_arguments_checked_on_the_host(L):
    """The measurement kernels of rq_probe.h reject bad arguments before any
    HIP call."""
    sink = ctypes.c_void_p(A)
    assert L.rq_probe_valu(17, 1, 1, sink, None) == header_enum("RQ_ERR_SHAPE")
    assert L.rq_probe_valu(-1, 1, 1, sink, None) == header_enum("RQ_ERR_SHAPE")
    assert L.rq_probe_valu(0, 0, 1, sink, None) == header_enum("RQ_ERR_SHAPE")
    assert L.rq_probe_valu(0, 1, 1, None, None) == header_enum("RQ_ERR_NULL")
    assert L.rq_probe_overlap(4, 0, 4, 1, 1, sink, None) == header_enum("RQ_ERR_SHAPE")
    assert L.rq_probe_overlap(0, 3, 4, 1, 1, sink, None) == header_enum("RQ_ERR_SHAPE")
    assert L.rq_probe_overlap(0, 0, 5, 1, 1, sink, None) == header_enum("RQ_ERR_SHAPE")
    assert L.rq_probe_overlap(0, 0, 4, 1, 0, sink, None) == header_enum("RQ_ERR_SHAPE")
    assert L.rq_probe_overlap(0, 0, 4, 1, 1, None, None) == header_enum("RQ_ERR_NULL")
    assert L.rq_probe_mfma(1, 1, 2, sink, None) == header_enum("RQ_ERR_SHAPE")
    assert L.rq_probe_barrier(sink, 1, 1, 1, 1, sink, None) == header_enum("RQ_ERR_SHAPE")
    assert L.rq_probe_copy(sink, ctypes.c_void_p(A + 16), 32, None) == header_enum("RQ_ERR_ALIAS")
