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
    src = open(HEADER).read()
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
              "RQ_ERR_LAUNCH", "RQ_ERR_ALIAS", "RQ_ERR_DEVICE", "RQ_LAYOUT_SYM",
              "RQ_LAYOUT_ASYM_SB", "RQ_LAYOUT_FP8_TENSOR", "RQ_OUT_F32", "RQ_OUT_CODES_I8"]:
        assert getattr(rq, n) == header_enum(n), n
    assert rq.RQ_MAX_M == int(re.search(r"#define RQ_MAX_M (\d+)", open(HEADER).read()).group(1))


def test_version_and_strings(L):
    assert rq.rq_version() == (1 << 16)
    seen = set()
    for s in range(8):
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


@pytest.mark.parametrize("fn", ["rq_gemv", "rq_gemm_smallm"])
@pytest.mark.parametrize("what,kw,status", CASES + GEMV_ONLY, ids=[c[0] for c in CASES + GEMV_ONLY])
def test_product_rejects(L, fn, what, kw, status):
    assert getattr(L, fn)(*gemv_args(**kw)) == status, what


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
