"""Degenerate inputs whose outputs have a bound of 0, so every kernel must
return exactly +-0 there (the tolerance 1e-3 * sum_k |w x| vanishes): rows of
all-zero codes, rows with zero scales (asymmetric: zero scale and zero shift),
and all-zero activations.  The other rows of the same calls are checked
against the oracle.  Both product entry points at M = 1..64, which covers the
vector-unit, decode and matrix-core kernels.  Also the smallest legal shapes of
every format: one to three rows of the shortest row the interface accepts."""
import pytest
import torch

from gemm_rwkv_decode_amd import synth as S
import gemm_rwkv_decode_amd as rq
from tests import rqtest as T

pytestmark = pytest.mark.gpu

N, K = 300, 4096
ZERO_CODE_ROWS = [0, 17, 150, 299]
ZERO_SCALE_ROWS = [5, 200, 298]
MS = [1, 2, 3, 4, 8, 16, 33, 64]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def degenerate(f):
    """Seeded weights with the zero rows planted (sym: zero codes, zero scales;
    asym: zero d and m, which zero both the scale and the shift)."""
    _, codes = S.gen_matrix("degen", 0, 0, N, K, f, keep_codes=True)
    g = torch.Generator().manual_seed(77)
    if f.layout == S.LAYOUT_SYM:
        codes[ZERO_CODE_ROWS] = 0
        scales = S.log_uniform_half((N, K // f.group), 1e-3, 1e-1, g, "cpu")
        scales[ZERO_SCALE_ROWS] = 0
        p = S.encode(codes, f, scales=scales)
        zero_rows = ZERO_CODE_ROWS + ZERO_SCALE_ROWS
    else:
        B = K // S.SUPERBLOCK
        d = S.log_uniform_half((N, B), 1e-4, 2e-3, g, "cpu")
        m = S.log_uniform_half((N, B), 1e-4, 2e-3, g, "cpu")
        sc = torch.randint(0, 64, (N, B, 8), generator=g, dtype=torch.int16).to(torch.uint8)
        mn = torch.randint(0, 64, (N, B, 8), generator=g, dtype=torch.int16).to(torch.uint8)
        d[ZERO_SCALE_ROWS] = 0
        m[ZERO_SCALE_ROWS] = 0
        p = S.encode(codes, f, d=d, sc=sc, m=m, mn=mn)
        zero_rows = ZERO_SCALE_ROWS
    return T.to_dev(p), sorted(zero_rows)


def x_for(M, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((M, K), generator=g)
    x[:, K // 3] *= 200.0
    return x.half().cuda()


@pytest.mark.parametrize("f", [S.INT4_G64, S.INT8_G16, S.ASYM4_G32], ids=lambda f: f.tag)
@pytest.mark.parametrize("entry", ["gemv", "gemm"])
def test_zero_rows_give_exact_zeros(f, entry):
    p, zero_rows = degenerate(f)
    for M in MS:
        x = x_for(M, 900 + M)
        y = torch.full((M, N), float("nan"), device="cuda")
        T.say(f"degenerate rows {entry} {f.tag} M={M}")
        T.run(entry, p, x, y)
        torch.cuda.synchronize()
        z = y[:, zero_rows]
        assert bool((z == 0).all()), f"{entry} {f.tag} M={M}: nonzero output on a zero row"
        yr, b = T.oracle_y(p, x)
        assert float(abs(b[:, zero_rows]).max()) == 0.0
        T.assert_close(y, yr, b, f"{entry} {f.tag} M={M}")


@pytest.mark.parametrize("f", [S.INT4_G64, S.INT8_G16, S.ASYM4_G32], ids=lambda f: f.tag)
@pytest.mark.parametrize("entry", ["gemv", "gemm"])
def test_zero_activations_give_exact_zeros(f, entry):
    p = T.to_dev(S.gen_matrix("degenx", 0, 0, N, K, f))
    for M in MS:
        x = torch.zeros((M, K), dtype=torch.float16, device="cuda")
        y = torch.full((M, N), float("nan"), device="cuda")
        T.say(f"zero activations {entry} {f.tag} M={M}")
        T.run(entry, p, x, y)
        torch.cuda.synchronize()
        assert bool((y == 0).all()), f"{entry} {f.tag} M={M}: nonzero output for x = 0"


def test_zero_rows_in_a_grouped_launch():
    """The same planted rows inside rq_gemv_batched (one launch, three problems)."""
    f = S.INT4_G64
    p, zero_rows = degenerate(f)
    q = T.to_dev(S.gen_matrix("degenb", 0, 1, N, K, f))
    for M in (1, 8, 32):
        x = x_for(M, 950 + M)
        ys = [torch.full((M, N), float("nan"), device="cuda") for _ in range(3)]
        mats = [p, q, p]
        T.say(f"degenerate rows grouped M={M}")
        rq.rq_gemv_batched([(w.qweight, w.scales, w.zeros, x, yb, w.N, w.K)
                            for w, yb in zip(mats, ys)], M, f.bits, f.group, f.layout)
        torch.cuda.synchronize()
        for i, (w, yb) in enumerate(zip(mats, ys)):
            yr, b = T.oracle_y(w, x)
            T.assert_close(yb, yr, b, f"grouped problem {i} M={M}")
        for i in (0, 2):
            assert bool((ys[i][:, zero_rows] == 0).all())


def smallest_k(f):
    """The shortest row the interface accepts: one group, a whole number of
    16-byte code chunks, and whole 256-code superblocks for the asymmetric
    layout."""
    k = max(f.group, 16 * 8 // f.bits)
    if f.layout == S.LAYOUT_ASYM_SB:
        k = S.SUPERBLOCK
    return k


SMALL_FORMATS = T.ALL_FORMATS + [S.FP8_E4M3, S.FORMATS["asym5g32"], S.FORMATS["asym6g32"]]


@pytest.mark.parametrize("f", SMALL_FORMATS, ids=lambda f: f.tag)
def test_smallest_shapes(f):
    """One to three rows of the shortest legal length (and twice that): dequant
    and codes bit-exact, both product entry points within the tolerance."""
    for N in (1, 2, 3):
        for K in (smallest_k(f), 2 * smallest_k(f)):
            p = T.to_dev(S.gen_matrix("tiny", N, K, N, K, f))
            w = T.dequant(p).cpu().numpy()
            assert (w.view("u4") == T.oracle_dequant(p).view("u4")).all(), f"{f.tag} {N}x{K}"
            if f.layout != S.LAYOUT_FP8_TENSOR:
                c = T.dequant(p, rq.RQ_OUT_CODES_I8).cpu().numpy()
                assert (c == T.oracle_codes(p)).all(), f"{f.tag} {N}x{K} codes"
            for M in (1, 2, 4, 5, 16, 64):
                x = x_for_k(M, K, 40 + M)
                yr, b = T.oracle_y(p, x)
                for entry in ("gemv", "gemm"):
                    T.say(f"smallest {entry} {f.tag} {N}x{K} M={M}")
                    y = torch.full((M, N), float("nan"), device="cuda")
                    T.run(entry, p, x, y)
                    torch.cuda.synchronize()
                    T.assert_close(y, yr, b, f"{entry} {f.tag} {N}x{K} M={M}")


def x_for_k(M, k, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((M, k), generator=g).half().cuda()
