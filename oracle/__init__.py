"""CPU oracle for group-wise low-bit dequantization and matvec.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
(``gemm_rwkv_decode_amd``) never imports it, and it imports nothing from there.

This module is argument marshalling over ``librq_oracle.so`` (built from
``rq_oracle.cpp`` by ``oracle/build.py`` with g++).  All arithmetic lives in the
C++ file, whose header states the formats, the readings of the pages and the
passages they follow.  Arrays are numpy arrays in host memory:

* ``qweight``: uint8 ``[N][K/2]`` (4-bit), int8/uint8 ``[N][K]`` (8-bit), or
  for 5- and 6-bit codes the flat ``N*K*bits/8`` bytes of the two planes (the
  ``[N][K/2]`` low nibbles, then the ``[N][K*(bits-4)/8]`` high bits);
* ``scales``: float16 ``[N][K/group]`` (symmetric), uint8 ``[N][K/256][8]``
  superblock records (asymmetric) or one float32 (FP8, the matrix scale);
  ``zeros``: ``None`` or uint8 records;
* ``x``: float16 ``[M][K]``.
"""
import ctypes
import os
import threading

import numpy as np

LAYOUT_SYM = 0
LAYOUT_ASYM_SB = 1
LAYOUT_FP8_TENSOR = 2
RTOL = 1e-3  # per-output tolerance: |y - y_ref| <= RTOL * sum_k |x w|

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librq_oracle.so")
_lib = None
_lock = threading.Lock()

_u8p = ctypes.POINTER(ctypes.c_uint8)
_i8p = ctypes.POINTER(ctypes.c_int8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_vp = ctypes.c_void_p
_i = ctypes.c_int


def _bind(L):
    """Declare the C signatures on a loaded oracle library."""
    L.rqo_half_to_double.argtypes = [ctypes.c_uint16]
    L.rqo_half_to_double.restype = ctypes.c_double
    L.rqo_fp8_to_double.argtypes = [ctypes.c_uint8]
    L.rqo_fp8_to_double.restype = ctypes.c_double
    L.rqo_code_at.argtypes = [_u8p, _i, _i, _i, _i, _i, _i]
    L.rqo_code_at.restype = _i
    L.rqo_unpack_codes.argtypes = [_u8p, _i, _i, _i, _i, _i8p]
    L.rqo_unpack_codes.restype = _i
    L.rqo_pack_codes.argtypes = [_i8p, _i, _i, _i, _i, _u8p]
    L.rqo_pack_codes.restype = _i
    L.rqo_pack_record.argtypes = [ctypes.c_uint16, _u8p, _u8p]
    L.rqo_pack_record.restype = _i
    L.rqo_unpack_record.argtypes = [_u8p, _u16p, _u8p]
    L.rqo_unpack_record.restype = _i
    L.rqo_dequant.argtypes = [_u8p, _vp, _vp, _i, _i, _i, _i, _i, _f32p]
    L.rqo_dequant.restype = _i
    L.rqo_gemv_ref.argtypes = [_u8p, _vp, _vp, _u16p, _i, _i, _i, _i, _i,
                               _i, _i, _i, _f64p, _f64p]
    L.rqo_gemv_ref.restype = _i
    L.rqo_check.argtypes = [_f32p, _f64p, _f64p, ctypes.c_long,
                            ctypes.c_double, ctypes.POINTER(ctypes.c_long),
                            _f64p]
    L.rqo_check.restype = ctypes.c_long
    L.rqo_version.argtypes = []
    L.rqo_version.restype = _i
    return L


def lib():
    """Load (building on first use if absent) the oracle shared library."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                from . import build as _b
                _b.build()
            _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def load_other(path):
    """Load another build of the oracle source (used by the mutation tests,
    which compile deliberately broken copies and check the pins reject them)."""
    return _bind(ctypes.CDLL(path))


def swap_library(L):
    """Make the module functions call ``L``; returns the previous library."""
    global _lib
    lib()
    with _lock:
        prev, _lib = _lib, L
    return prev


def _ptr(a, t):
    return a.ctypes.data_as(t)


def _bytes(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint8) if a.dtype != np.uint8 else a


def _scales_arg(scales):
    if scales is None:
        return None, None
    a = np.ascontiguousarray(scales)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    return a, ctypes.c_void_p(a.ctypes.data)


def half_to_double(bits: int) -> float:
    return lib().rqo_half_to_double(bits)


def fp8_to_double(byte: int) -> float:
    return lib().rqo_fp8_to_double(byte)


def code_at(qweight, N, K, bits, layout, n, k) -> int:
    q = _bytes(qweight)
    return lib().rqo_code_at(_ptr(q, _u8p), N, K, bits, layout, n, k)


def unpack_codes(qweight, N, K, bits, layout):
    q = _bytes(qweight)
    out = np.empty((N, K), dtype=np.int8)
    rc = lib().rqo_unpack_codes(_ptr(q, _u8p), N, K, bits, layout, _ptr(out, _i8p))
    if rc:
        raise ValueError("rqo_unpack_codes: bad argument")
    return out


def pack_codes(codes, bits, layout):
    c = np.ascontiguousarray(codes, dtype=np.int8)
    N, K = c.shape
    if bits in (5, 6):
        out = np.empty(N * K * bits // 8, dtype=np.uint8)
    else:
        out = np.empty((N, K if bits == 8 else K // 2), dtype=np.uint8)
    rc = lib().rqo_pack_codes(_ptr(c, _i8p), N, K, bits, layout, _ptr(out, _u8p))
    if rc:
        raise ValueError("rqo_pack_codes: bad argument or code out of range")
    return out


def pack_record(base_bits: int, sub):
    s = np.ascontiguousarray(sub, dtype=np.uint8)
    assert s.shape == (8,)
    out = np.empty(8, dtype=np.uint8)
    rc = lib().rqo_pack_record(base_bits, _ptr(s, _u8p), _ptr(out, _u8p))
    if rc:
        raise ValueError("rqo_pack_record: sub-code out of range")
    return out


def unpack_record(rec):
    r = np.ascontiguousarray(rec, dtype=np.uint8)
    assert r.shape == (8,)
    base = ctypes.c_uint16(0)
    sub = np.empty(8, dtype=np.uint8)
    rc = lib().rqo_unpack_record(_ptr(r, _u8p), ctypes.byref(base), _ptr(sub, _u8p))
    if rc:
        raise ValueError("rqo_unpack_record: bad argument")
    return int(base.value), sub


def dequant(qweight, scales, zeros, N, K, bits, group, layout):
    q = _bytes(qweight)
    s_keep, s_arg = _scales_arg(scales)
    z_keep, z_arg = _scales_arg(zeros)
    out = np.empty((N, K), dtype=np.float32)
    rc = lib().rqo_dequant(_ptr(q, _u8p), s_arg, z_arg, N, K, bits, group, layout,
                           _ptr(out, _f32p))
    if rc:
        raise ValueError("rqo_dequant: bad argument")
    return out


def gemv_ref(qweight, scales, zeros, x, N, K, bits, group, layout, threads=1):
    """Return (y_ref, bound), both float64 ``[M][N]``.

    ``threads`` > 1 runs the single-threaded routine on disjoint row ranges from
    that many host threads (the routine itself is unchanged)."""
    q = _bytes(qweight)
    s_keep, s_arg = _scales_arg(scales)
    z_keep, z_arg = _scales_arg(zeros)
    xx = np.ascontiguousarray(x, dtype=np.float16)
    if xx.ndim == 1:
        xx = xx[None, :]
    M = xx.shape[0]
    assert xx.shape[1] == K
    xb = xx.view(np.uint16)
    y = np.zeros((M, N), dtype=np.float64)
    b = np.zeros((M, N), dtype=np.float64)
    L = lib()
    errors = []

    def run(n0, n1):
        rc = L.rqo_gemv_ref(_ptr(q, _u8p), s_arg, z_arg, _ptr(xb, _u16p), M, N, K,
                            bits, group, layout, n0, n1, _ptr(y, _f64p),
                            _ptr(b, _f64p))
        if rc:
            errors.append((n0, n1))

    threads = max(1, min(int(threads), N))
    if threads == 1:
        run(0, N)
    else:
        edges = [N * i // threads for i in range(threads + 1)]
        ts = [threading.Thread(target=run, args=(edges[i], edges[i + 1]))
              for i in range(threads)]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
    if errors:
        raise ValueError("rqo_gemv_ref: bad argument")
    return y, b


def check(y, y_ref, bound, rtol=RTOL):
    """Return (n_bad, first_bad_flat_index, worst_ratio)."""
    yy = np.ascontiguousarray(y, dtype=np.float32).ravel()
    yr = np.ascontiguousarray(y_ref, dtype=np.float64).ravel()
    bb = np.ascontiguousarray(bound, dtype=np.float64).ravel()
    assert yy.size == yr.size == bb.size
    first = ctypes.c_long(-1)
    worst = ctypes.c_double(0.0)
    nbad = lib().rqo_check(_ptr(yy, _f32p), _ptr(yr, _f64p), _ptr(bb, _f64p),
                           yy.size, rtol, ctypes.byref(first), ctypes.byref(worst))
    return int(nbad), int(first.value), float(worst.value)


def version() -> int:
    return lib().rqo_version()
