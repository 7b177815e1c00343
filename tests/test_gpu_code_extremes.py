"""The most negative codes on every product kernel.

A symmetric 4-bit code is a 4-bit two's complement integer, so its range is
-8..7 (model card "RWKV-7 G1 1.5B -- int4 GPTQ for rwkv-sglang", section
"Format & loading"); an 8-bit code is an int8, -128..127 (news article
"rwkv-quant: keeping one matrix in bf16 ...", section "Two presets and six
sizes").  The seeded generators draw from [-7, 7] and [-127, 127], so these
tests build matrices whose codes take the full range and hold -8 / -128 at
every position of every 16-byte chunk and group, and send them through each
kernel: the vector-unit kernel, the matrix-core decode kernel and the
small-batch matrix-core kernel (forced through rq_gemv), rq_gemm_smallm (with
K split over workgroups as well) and rq_gemv_batched.  Three checks:

* random scales and activations: within 1e-3 * sum|w x| of the oracle;
* one-hot activations: every output is one dequantized weight, bit-exact;
* unit scales and small integer activations: exact integer results.
Outputs start as NaN.
"""
import pytest
import torch

import gemm_rwkv_decode_amd as rq
from gemm_rwkv_decode_amd import synth as S
from tests import rqtest as T

pytestmark = pytest.mark.gpu

FORMATS = [S.INT4_G64, S.INT8_G16, T.fmt("int4g32", 4, 32, S.LAYOUT_SYM),
           T.fmt("int4g128", 4, 128, S.LAYOUT_SYM), T.fmt("int8g64", 8, 64, S.LAYOUT_SYM)]
KERNELS = {"vector": 1, "decode": 2, "smallbatch": 3}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


@pytest.fixture
def tune(monkeypatch):
    def set_(**kv):
        for k, v in kv.items():
            monkeypatch.setenv(k, str(v))
        rq.tuning_reload()
    yield set_
    monkeypatch.undo()
    rq.tuning_reload()


def extreme_codes(f, N, K, seed):
    """Codes uniform over the full range, with the lowest code at every k of
    every third row (offset by the row) and in all of row 0."""
    lo = -8 if f.bits == 4 else -128
    hi = 7 if f.bits == 4 else 127
    g = torch.Generator().manual_seed(seed)
    codes = torch.randint(lo, hi + 1, (N, K), generator=g, dtype=torch.int16)
    n = torch.arange(N).unsqueeze(1)
    k = torch.arange(K).unsqueeze(0)
    codes = torch.where((k + n) % 3 == 0, torch.full_like(codes, lo), codes)
    codes[0] = lo
    return codes.to(torch.int8)


def extreme_matrix(f, N, K, seed, unit_scales=False):
    codes = extreme_codes(f, N, K, seed)
    if unit_scales:
        sc = torch.ones((N, K // f.group), dtype=torch.float16)
    else:
        g = torch.Generator().manual_seed(seed + 1)
        sc = S.log_uniform_half((N, K // f.group), 1e-3, 1e-1, g, "cpu")
    return T.to_dev(S.encode(codes, f, scales=sc)), codes


def k_for(f):
    """K with eight chunks of the decode kernel (eight groups each)."""
    return 8 * 8 * f.group


def x_massive(M, K, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((M, K), generator=g)
    x[:, K // 5] *= 300.0
    return x.half().cuda()


def nan_y(M, N):
    return torch.full((M, N), float("nan"), device="cuda")


@pytest.mark.parametrize("f", FORMATS, ids=lambda f: f.tag)
@pytest.mark.parametrize("kern", list(KERNELS))
def test_lowest_code_forced_kernels(tune, f, kern):
    tune(RQ_GEMV_KERNEL=KERNELS[kern])
    N, K = 131, k_for(f)
    p, _ = extreme_matrix(f, N, K, seed=11)
    for M in (1, 2, 3, 4) + ((5, 16, 40) if kern != "decode" else ()):
        what = f"{kern} {f.tag} M={M} N={N} K={K}"
        T.say(what)
        x = x_massive(M, K, seed=M)
        y = T.run("gemv", p, x, nan_y(M, N))
        yr, b = T.oracle_y(p, x)
        T.assert_close(y, yr, b, what)


@pytest.mark.parametrize("f", FORMATS, ids=lambda f: f.tag)
def test_lowest_code_smallm_and_split(tune, f):
    """rq_gemm_smallm by its own choice (K whole at these shapes), then with K
    split over 2 and 4 workgroups."""
    N, K = 300, 4 * k_for(f)
    p, _ = extreme_matrix(f, N, K, seed=12)
    for splits in (None, 2, 4):
        if splits:
            tune(RQ_GEMM_SPLITS=splits)
        for M in (1, 16, 33, 64):
            what = f"smallm splits={splits} {f.tag} M={M} N={N} K={K}"
            T.say(what)
            x = x_massive(M, K, seed=100 + M)
            y = T.run("gemm", p, x, nan_y(M, N))
            yr, b = T.oracle_y(p, x)
            T.assert_close(y, yr, b, what)


@pytest.mark.parametrize("f", FORMATS, ids=lambda f: f.tag)
@pytest.mark.parametrize("M", [1, 3, 8, 32])
def test_lowest_code_batched(f, M):
    shapes = [(131, k_for(f)), (64, k_for(f)), (200, 2 * k_for(f))]
    mats = [extreme_matrix(f, N, K, seed=20 + i)[0] for i, (N, K) in enumerate(shapes)]
    xs = [x_massive(M, K, seed=30 + i) for i, (_, K) in enumerate(shapes)]
    ys = [nan_y(M, N) for (N, _) in shapes]
    T.say(f"batched lowest code {f.tag} M={M}")
    rq.rq_gemv_batched([(p.qweight, p.scales, None, x, y, p.N, p.K)
                        for p, x, y in zip(mats, xs, ys)], M, f.bits, f.group, f.layout)
    for i, (p, x, y) in enumerate(zip(mats, xs, ys)):
        yr, b = T.oracle_y(p, x)
        T.assert_close(y, yr, b, f"batched {f.tag} M={M} problem {i}")


def entries():
    """(name, callable(p, x, y)) for every path a product can take."""
    def forced(k):
        def run(tune, p, x, y):
            tune(RQ_GEMV_KERNEL=k)
            T.run("gemv", p, x, y)
        return run

    def smallm(tune, p, x, y):
        tune(RQ_GEMV_KERNEL=0)
        T.run("gemm", p, x, y)

    def batched(tune, p, x, y):
        tune(RQ_GEMV_KERNEL=0)
        f = p.fmt
        rq.rq_gemv_batched([(p.qweight, p.scales, None, x, y, p.N, p.K)], x.shape[0], f.bits,
                           f.group, f.layout)
    return [("vector", forced(1)), ("decode", forced(2)), ("smallbatch", forced(3)),
            ("smallm", smallm), ("batched", batched)]


@pytest.mark.parametrize("f", [S.INT4_G64, S.INT8_G16], ids=lambda f: f.tag)
@pytest.mark.parametrize("name,call", entries(), ids=[e[0] for e in entries()])
def test_lowest_code_one_hot_bit_exact(tune, f, name, call):
    """x = e_j per activation row: y[m][n] is the dequantized w[n][j], reached
    without rounding; the columns j cover every position of a chunk."""
    N, K = 96, k_for(f)
    p, _ = extreme_matrix(f, N, K, seed=13)
    w = T.dequant(p).cpu()
    for M in ((1, 4) if name == "decode" else (1, 4, 16, 64)):
        js = (torch.arange(M) * 5 + 3) % K
        x = torch.zeros((M, K), dtype=torch.float16)
        x[torch.arange(M), js] = 1.0
        T.say(f"one-hot lowest code {name} {f.tag} M={M}")
        y = nan_y(M, N)
        call(tune, p, x.cuda(), y)
        assert torch.equal(y.cpu(), w[:, js].T.contiguous()), f"{name} {f.tag} M={M}"
    # the columns where row 0 (all lowest codes) meets every position of one
    # 16-byte chunk
    cpc = 32 if f.bits == 4 else 16
    for j0 in range(0, cpc, 4 if name == "decode" else 16):
        M = 4 if name == "decode" else 16
        js = torch.arange(j0, j0 + M) % K
        x = torch.zeros((M, K), dtype=torch.float16)
        x[torch.arange(M), js] = 1.0
        y = nan_y(M, N)
        call(tune, p, x.cuda(), y)
        assert torch.equal(y.cpu(), w[:, js].T.contiguous()), f"{name} {f.tag} cols {j0}.."


@pytest.mark.parametrize("f", [S.INT4_G64, S.INT8_G16], ids=lambda f: f.tag)
@pytest.mark.parametrize("name,call", entries(), ids=[e[0] for e in entries()])
def test_lowest_code_integer_exact(tune, f, name, call):
    """Unit scales and integer activations in [-4, 4]: every partial sum is an
    integer below 2^24, so y must equal the int64 matmul of the codes."""
    N, K = 96, k_for(f)
    p, codes = extreme_matrix(f, N, K, seed=14, unit_scales=True)
    W = codes.to(torch.int64)
    for M in ((1, 3) if name == "decode" else (1, 3, 16, 64)):
        g = torch.Generator().manual_seed(M + 7)
        xi = torch.randint(-4, 5, (M, K), generator=g)
        T.say(f"integer lowest code {name} {f.tag} M={M}")
        y = nan_y(M, N)
        call(tune, p, xi.half().cuda(), y)
        expect = (xi.to(torch.int64) @ W.T).to(torch.float64)
        assert torch.equal(y.cpu().to(torch.float64), expect), f"{name} {f.tag} M={M}"
