"""Python binding of librq (include/rq.h): group-wise low-bit weight
dequantization and dequantize-and-multiply on MI355X (gfx950).

Argument marshalling only.  Every computation runs in the HIP kernels of
``librq.so``; there is no CPU fallback.  If the library is missing, every call
raises ``RqLibraryMissing`` (build it with ``python gemm_rwkv_decode_amd/build.py``
or ``__graft_entry__.build()``).

Tensors are torch tensors on the GPU, contiguous:

* ``qweight``: uint8 ``[N][K/2]`` (4-bit) or int8 ``[N][K]`` (8-bit);
* ``scales``: float16 ``[N][K/group]`` (symmetric) or uint8 ``[N][K/256][8]``
  superblock records (asymmetric); ``zeros``: ``None`` (symmetric) or uint8
  records (asymmetric);
* ``x``: float16 ``[M][K]``; ``y``: float32 ``[M][N]``.

Work is enqueued on torch's current stream (or the ``stream`` given).
"""
import ctypes
import os
import threading

__all__ = [
    "RQ_OK", "RQ_LAYOUT_SYM", "RQ_LAYOUT_ASYM_SB", "RQ_LAYOUT_FP8_TENSOR", "RQ_OUT_F32",
    "RQ_OUT_CODES_I8",
    "RQ_MAX_M", "RQ_MAX_BATCH", "RqError", "RqLibraryMissing", "rq_dequant", "rq_gemv",
    "rq_gemv_batched", "rq_gemm_smallm", "rq_status_string", "rq_version", "prepare",
    "lib", "LIB_PATH",
]

RQ_OK = 0
RQ_ERR_NULL, RQ_ERR_SHAPE, RQ_ERR_UNSUPPORTED, RQ_ERR_ALIGN = 1, 2, 3, 4
RQ_ERR_LAUNCH, RQ_ERR_ALIAS, RQ_ERR_DEVICE = 5, 6, 7
RQ_LAYOUT_SYM, RQ_LAYOUT_ASYM_SB, RQ_LAYOUT_FP8_TENSOR = 0, 1, 2
RQ_OUT_F32, RQ_OUT_CODES_I8 = 0, 1
RQ_MAX_M = 64
RQ_MAX_BATCH = 64

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librq.so")
_lib = None
_lock = threading.Lock()


class RqProblem(ctypes.Structure):
    """rq_problem of include/rq.h."""
    _fields_ = [("qweight", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("x", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("N", ctypes.c_int), ("K", ctypes.c_int)]


class RqLibraryMissing(RuntimeError):
    pass


class RqError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: status {status} ({rq_status_string(status)})")


def lib():
    """The loaded librq (ctypes), signatures declared."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RqLibraryMissing(
                    f"{LIB_PATH} not found: build it with gemm_rwkv_decode_amd/build.py")
            L = ctypes.CDLL(LIB_PATH)
            vp, i = ctypes.c_void_p, ctypes.c_int
            L.rq_dequant.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, vp]
            L.rq_dequant.restype = i
            for name in ("rq_gemv", "rq_gemm_smallm"):
                f = getattr(L, name)
                f.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
                f.restype = i
            L.rq_gemv_batched.argtypes = [ctypes.POINTER(RqProblem), i, i, i, i, i, vp]
            L.rq_gemv_batched.restype = i
            L.rq_status_string.argtypes = [i]
            L.rq_status_string.restype = ctypes.c_char_p
            L.rq_version.argtypes = []
            L.rq_version.restype = i
            # measurement kernels (include/rq_probe.h)
            L.rq_probe_read.argtypes = [vp, ctypes.c_size_t, vp, i, i, vp]
            L.rq_probe_read.restype = i
            L.rq_probe_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
            L.rq_probe_copy.restype = i
            L.rq_probe_empty.argtypes = [vp]
            L.rq_probe_empty.restype = i
            L.rq_tuning_reload.argtypes = []
            L.rq_tuning_reload.restype = i
            _lib = L
    return _lib


def rq_status_string(status: int) -> str:
    return lib().rq_status_string(int(status)).decode()


def rq_version() -> int:
    return lib().rq_version()


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("librq takes GPU tensors only")
    if not t.is_contiguous():
        raise ValueError("librq takes contiguous tensors only")
    return t.data_ptr()


def _stream(stream, like):
    if stream is not None:
        return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)
    import torch
    return int(torch.cuda.current_stream(like.device).cuda_stream)


def rq_dequant(qweight, scales, zeros, out, N, K, bits, group, layout,
               out_kind=RQ_OUT_F32, stream=None):
    """Unpack (out_kind RQ_OUT_CODES_I8, out int8 [N][K]) or dequantize
    (RQ_OUT_F32, out float32 [N][K]) the packed weights."""
    st = lib().rq_dequant(_ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(out), int(N),
                          int(K), int(bits), int(group), int(layout), int(out_kind),
                          _stream(stream, qweight))
    if st != RQ_OK:
        raise RqError("rq_dequant", st)
    return out


def rq_gemv(qweight, scales, zeros, x, y, M, N, K, bits, group, layout, stream=None):
    """y[m][n] = sum_k x[m][k] w[n][k]; the kernel is chosen for M (vector units
    at M <= 2, matrix cores from M = 5 on), K is never split, nothing is
    allocated."""
    st = lib().rq_gemv(_ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(x), _ptr(y), int(M),
                       int(N), int(K), int(bits), int(group), int(layout),
                       _stream(stream, qweight))
    if st != RQ_OK:
        raise RqError("rq_gemv", st)
    return y


def rq_gemm_smallm(qweight, scales, zeros, x, y, M, N, K, bits, group, layout,
                   stream=None):
    """Same product on the matrix cores (tuned for 16 <= M <= 64)."""
    st = lib().rq_gemm_smallm(_ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(x), _ptr(y),
                              int(M), int(N), int(K), int(bits), int(group), int(layout),
                              _stream(stream, qweight))
    if st != RQ_OK:
        raise RqError("rq_gemm_smallm", st)
    return y


def _problems(problems):
    arr = (RqProblem * len(problems))()
    for i, (qweight, scales, zeros, x, y, N, K) in enumerate(problems):
        arr[i] = RqProblem(_ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(x), _ptr(y),
                           int(N), int(K))
    return arr


def rq_gemv_batched(problems, M, bits, group, layout, stream=None):
    """Independent products in as few launches as possible.  ``problems`` is a
    sequence of (qweight, scales, zeros, x, y, N, K); M, bits, group and layout
    are shared."""
    arr = _problems(problems)
    st = lib().rq_gemv_batched(arr, len(problems), int(M), int(bits), int(group),
                               int(layout), _stream(stream, problems[0][0]))
    if st != RQ_OK:
        raise RqError("rq_gemv_batched", st)


def prepare(name, *args, stream=None):
    """Resolve the tensor arguments of one call now and return a callable that
    repeats it with no per-call argument conversion in Python (for step loops
    and graph capture).  ``name`` is "rq_gemv", "rq_gemm_smallm",
    "rq_gemv_batched" or "rq_dequant"; ``args`` are those of the Python
    function of that name, without ``stream``.  The tensors must stay alive."""
    L = lib()
    f = getattr(L, name)
    if name == "rq_gemv_batched":
        problems, M, bits, group, layout = args
        arr = _problems(problems)
        cargs = (arr, len(problems), int(M), int(bits), int(group), int(layout),
                 _stream(stream, problems[0][0]))
    elif name == "rq_dequant":
        qweight, scales, zeros, out, N, K, bits, group, layout, out_kind = args
        cargs = (_ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(out), int(N), int(K),
                 int(bits), int(group), int(layout), int(out_kind), _stream(stream, qweight))
    else:
        qweight, scales, zeros, x, y, M, N, K, bits, group, layout = args
        cargs = (_ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(x), _ptr(y), int(M), int(N),
                 int(K), int(bits), int(group), int(layout), _stream(stream, qweight))

    def call():
        st = f(*cargs)
        if st != RQ_OK:
            raise RqError(name, st)
    call.args = cargs  # keeps the problem array alive
    return call


def tuning_reload():
    """Re-read the RQ_* launch-shape override variables (tuning and tests)."""
    lib().rq_tuning_reload()
