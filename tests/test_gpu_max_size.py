"""The largest matrices the interface accepts: code bytes one row short of
2 GiB (int8: 131071 x 16384; int4 and asymmetric 4-bit: 262143 x 16384).
The kernels index every operand with 32-bit byte offsets, so these rows sit
at the top of that range; the odd row counts also leave a ragged last block
in every launch shape.  Sampled rows (first, last, the ones around the 1 GiB
and 2 GiB offsets, and a seeded random draw) are checked against the oracle:
products of rq_gemv (M = 1, 4, 32) and rq_gemm_smallm (M = 32, 64) within
|y - y_ref| <= 1e-3 * sum_k |w x|, and rq_dequant (codes and values)
bit-exact.  Every output starts as NaN and must be finite after the call.
FP8 and 5-/6-bit codes use the int8 and int4 byte layouts' offsets and are
covered at smaller sizes elsewhere."""
import numpy as np
import pytest
import torch

import oracle as O
import gemm_rwkv_decode_amd as rq
from gemm_rwkv_decode_amd import synth as S
from tests import rqtest as T

pytestmark = pytest.mark.gpu

K = 16384
LIMIT = 1 << 31
FORMATS = [S.INT8_G16, S.INT4_G64, S.ASYM4_G32]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def row_bytes(f):
    return K if f.bits == 8 else K // 2


def max_rows(f):
    return (LIMIT - 1) // row_bytes(f)


@pytest.fixture(scope="module", params=FORMATS, ids=lambda f: f.tag)
def big(request):
    f = request.param
    N = max_rows(f)
    assert N * row_bytes(f) < LIMIT <= (N + 1) * row_bytes(f)
    T.say(f"[max-size] {f.tag} {N}x{K}: generating {N * row_bytes(f)} code bytes")
    p = S.gen_matrix("maxsize", 0, 0, N, K, f, device="cuda")
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(S.seed_for("maxsize", 0, 0, "rows", f.tag, 0))
    rb = row_bytes(f)
    edge = {0, 1, N - 2, N - 1, (1 << 30) // rb - 1, (1 << 30) // rb, (1 << 30) // rb + 1}
    rows = sorted(edge | set(torch.randint(0, N, (24,), generator=g).tolist()))
    yield p, rows
    del p
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def x_for(M, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((M, K), generator=g)
    x[:, K // 3] *= 200.0  # one large channel
    return x.half().cuda()


@pytest.mark.parametrize("entry,M", [("gemv", 1), ("gemv", 4), ("gemv", 32),
                                     ("gemm", 32), ("gemm", 64)])
def test_product_max_rows(big, entry, M):
    p, rows = big
    x = x_for(M, seed=7000 + M)
    y = torch.full((M, p.N), float("nan"), device="cuda")
    T.say(f"[max-size] rq_{'gemv' if entry == 'gemv' else 'gemm_smallm'} {p.fmt.tag} "
          f"{p.N}x{K} M={M}")
    T.run(entry, p, x, y)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()), "an output was not written"
    sub = S.rows_of(p, rows)
    yr, b = T.oracle_y(sub, x)
    T.assert_close(y[:, rows], yr, b, f"{p.fmt.tag} {p.N}x{K} M={M} via {entry}")


@pytest.mark.parametrize("kind", [rq.RQ_OUT_CODES_I8, rq.RQ_OUT_F32], ids=["codes", "values"])
def test_dequant_max_rows(big, kind):
    p, rows = big
    dt = torch.int8 if kind == rq.RQ_OUT_CODES_I8 else torch.float32
    T.say(f"[max-size] rq_dequant {p.fmt.tag} {p.N}x{K} kind={kind}")
    out = torch.empty((p.N, K), dtype=dt, device="cuda")
    if kind == rq.RQ_OUT_F32:
        out.fill_(float("nan"))
    else:
        out.fill_(0x5A)
    rq.rq_dequant(p.qweight, p.scales, p.zeros, out, p.N, K, p.fmt.bits, p.fmt.group,
                  p.fmt.layout, kind)
    torch.cuda.synchronize()
    if kind == rq.RQ_OUT_F32:
        assert bool(torch.isfinite(out).all()), "a value was not written"
    got = out[rows].cpu().numpy()
    del out
    sub = S.rows_of(p, rows)
    ref = T.oracle_codes(sub) if kind == rq.RQ_OUT_CODES_I8 else T.oracle_dequant(sub)
    assert got.dtype == ref.dtype and got.shape == ref.shape
    bad = np.flatnonzero(got.view(np.uint8 if dt == torch.int8 else np.uint32).ravel() !=
                         ref.view(np.uint8 if dt == torch.int8 else np.uint32).ravel())
    assert bad.size == 0, (f"{p.fmt.tag} {p.N}x{K}: {bad.size} entries differ, first at "
                           f"{np.unravel_index(bad[0], got.shape)}")
