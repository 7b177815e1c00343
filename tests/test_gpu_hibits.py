"""5- and 6-bit asymmetric superblock codes on the GPU against the oracle:
rq_dequant bit for bit (codes and binary32 weights), products within
|y - y_ref| <= 1e-3 * sum_k |w x| at every M through every entry point, a
grouped launch with mixed shapes, and the width-4096 FFN key shape the
COMPRESSION preset keeps in 5 bits.  Outputs start as NaN."""
import numpy as np
import pytest
import torch

import oracle as O
import gemm_rwkv_decode_amd as rq
from gemm_rwkv_decode_amd import synth as S
from tests import rqtest as T

pytestmark = pytest.mark.gpu
FMTS = [S.ASYM5_G32, S.ASYM6_G32]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def x_for(M, K, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((M, K), generator=g)
    x[:, K // 3] *= 150.0
    return x.half().cuda()


@pytest.mark.parametrize("f", FMTS, ids=lambda f: f.tag)
@pytest.mark.parametrize("N,K", [(37, 512), (129, 2560), (3, 256)])
def test_dequant_bit_exact(f, N, K):
    p, codes = S.gen_matrix("hbdq", 0, 0, N, K, f, keep_codes=True)
    p = T.to_dev(p)
    got_codes = T.dequant(p, rq.RQ_OUT_CODES_I8).cpu().numpy()
    assert np.array_equal(got_codes, codes.numpy())
    q, s, z = T.to_np(p)
    assert np.array_equal(got_codes, O.unpack_codes(q, N, K, f.bits, f.layout))
    w = T.dequant(p).cpu().numpy()
    ref = O.dequant(q, s, z, N, K, f.bits, f.group, f.layout)
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("f", FMTS, ids=lambda f: f.tag)
def test_every_code_value_at_every_position(f):
    """Row r holds code (k + r) mod 2^bits at k: every value at every chunk
    position across the rows."""
    N, K = 64, 256
    codes = ((torch.arange(K)[None, :] + torch.arange(N)[:, None]) % (1 << f.bits)).to(torch.int8)
    g = torch.Generator().manual_seed(3)
    B = K // 256
    d = S.log_uniform_half((N, B), 1e-4, 2e-3, g, "cpu")
    m = S.log_uniform_half((N, B), 1e-4, 2e-3, g, "cpu")
    sc = torch.randint(0, 64, (N, B, 8), generator=g, dtype=torch.int16).to(torch.uint8)
    mn = torch.randint(0, 64, (N, B, 8), generator=g, dtype=torch.int16).to(torch.uint8)
    p = T.to_dev(S.encode(codes, f, d=d, sc=sc, m=m, mn=mn))
    assert np.array_equal(T.dequant(p, rq.RQ_OUT_CODES_I8).cpu().numpy(), codes.numpy())
    x = x_for(3, K, seed=4)
    y = torch.full((3, N), float("nan"), device="cuda")
    T.run("gemv", p, x, y)
    yr, b = T.oracle_y(p, x)
    T.assert_close(y, yr, b, f"{f.tag} every value")


@pytest.mark.parametrize("f", FMTS, ids=lambda f: f.tag)
@pytest.mark.parametrize("N,K", [(37, 512), (300, 2048), (129, 4096), (33, 256 * 3)])
@pytest.mark.parametrize("entry", ["gemv", "gemm"])
def test_products(f, N, K, entry):
    p = T.to_dev(S.gen_matrix("hbmv", 1, 0, N, K, f))
    for M in (1, 2, 3, 4, 5, 8, 16, 33, 64):
        what = f"{entry} {f.tag} M={M} N={N} K={K}"
        T.say(what)
        x = x_for(M, K, seed=M * 11 + N)
        y = torch.full((M, N), float("nan"), device="cuda")
        T.run(entry, p, x, y)
        yr, b = T.oracle_y(p, x)
        T.assert_close(y, yr, b, what)


@pytest.mark.parametrize("f", FMTS, ids=lambda f: f.tag)
def test_batched_mixed_shapes(f):
    shapes = [(256, 4096), (100, 1024), (64, 4096), (17, 512)] * 3
    mats = [T.to_dev(S.gen_matrix("hbb", i, 0, N, K, f)) for i, (N, K) in enumerate(shapes)]
    for M in (1, 4, 17):
        xs = [x_for(M, K, seed=70 + i) for i, (_, K) in enumerate(shapes)]
        ys = [torch.full((M, N), float("nan"), device="cuda") for (N, _) in shapes]
        rq.rq_gemv_batched([(p.qweight, p.scales, p.zeros, x, y, p.N, p.K)
                            for p, x, y in zip(mats, xs, ys)], M, f.bits, f.group, f.layout)
        for i, (p, x, y) in enumerate(zip(mats, xs, ys)):
            yr, b = T.oracle_y(p, x)
            T.assert_close(y, yr, b, f"batched {f.tag} M={M} problem {i} {p.N}x{p.K}")


@pytest.mark.parametrize("f", FMTS, ids=lambda f: f.tag)
def test_ffn_key_width_4096(f):
    """16384x4096 at M = 1: a seeded sample of rows (and the first and last)."""
    N, K = 16384, 4096
    p = T.to_dev(S.gen_matrix("hbffn", 0, 4, N, K, f))
    x = x_for(1, K, seed=9)
    y = torch.full((1, N), float("nan"), device="cuda")
    T.run("gemv", p, x, y)
    g = torch.Generator().manual_seed(N + f.bits)
    rows = sorted(set(torch.randperm(N, generator=g)[:64].tolist()) | {0, N - 1})
    yr, b = T.oracle_y(S.rows_of(p, rows), x)
    T.assert_close(y[:, rows], yr, b, f"{f.tag} 16384x4096 M=1")


@pytest.fixture
def tune(monkeypatch):
    def set_(**kv):
        for k, v in kv.items():
            monkeypatch.setenv(k, str(v))
        rq.tuning_reload()
    yield set_
    monkeypatch.undo()
    rq.tuning_reload()


@pytest.mark.parametrize("plan", [str(i) for i in range(1, 19)])
@pytest.mark.parametrize("f", FMTS, ids=lambda f: f.tag)
def test_matrix_core_plans(tune, plan, f):
    """Every workgroup arrangement of the matrix-core kernel (high-bit plane
    copied with the codes each round), ragged N, 1..4 M-tiles."""
    tune(RQ_GEMM_PLAN=plan)
    p = T.to_dev(S.gen_matrix("hbmm", 2, 0, 130, 4096, f))
    for M in (16, 20, 33, 64):
        what = f"plan={plan} {f.tag} M={M}"
        T.say(what)
        x = x_for(M, 4096, seed=M + 3)
        y = torch.full((M, p.N), float("nan"), device="cuda")
        T.run("gemm", p, x, y)
        yr, b = T.oracle_y(p, x)
        T.assert_close(y, yr, b, what)


@pytest.mark.parametrize("splits", ["2", "4", "8"])
@pytest.mark.parametrize("f", FMTS, ids=lambda f: f.tag)
def test_matrix_core_split_k(tune, splits, f):
    tune(RQ_GEMM_SPLITS=splits)
    p = T.to_dev(S.gen_matrix("hbsk", 3, 0, 256, 8192, f))
    for M in (16, 64):
        what = f"splits={splits} {f.tag} M={M}"
        T.say(what)
        x = x_for(M, 8192, seed=M + 5)
        y = torch.full((M, p.N), float("nan"), device="cuda")
        T.run("gemm", p, x, y)
        yr, b = T.oracle_y(p, x)
        T.assert_close(y, yr, b, what)


@pytest.mark.parametrize("f", FMTS, ids=lambda f: f.tag)
def test_ffn_shapes_m32_matrix_cores(f):
    """The width-4096 FFN shapes at M = 32 on the matrix cores, every row."""
    for (N, K) in ((16384, 4096), (4096, 16384)):
        p = T.to_dev(S.gen_matrix("hbffn32", 0, 4, N, K, f))
        x = x_for(32, K, seed=N + K)
        y = torch.full((32, N), float("nan"), device="cuda")
        T.say(f"{f.tag} {N}x{K} M=32")
        T.run("gemm", p, x, y)
        yr, b = T.oracle_y(p, x)
        T.assert_close(y, yr, b, f"{f.tag} {N}x{K} M=32")
