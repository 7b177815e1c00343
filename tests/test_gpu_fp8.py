"""FP8 E4M3 per-tensor weights (package page "RWKV-7 FP8 Quantized Inference",
sections "Core Approach: Full FP8, No Residuals" and "Quantization Principle")
on the GPU against the oracle: rq_dequant bit for bit over every code byte
and on matrices quantized by the page's recipe; products within
|y - y_ref| <= 1e-3 * sum_k |w x| at every M, through every entry point, at
small and at full RWKV-7 width-4096 shapes.  Outputs start as NaN.
"""
import numpy as np
import pytest
import torch

import oracle as O
import gemm_rwkv_decode_amd as rq
from gemm_rwkv_decode_amd import synth as S
from tests import rqtest as T

pytestmark = pytest.mark.gpu
F = S.FP8_E4M3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def every_code_matrix(scale):
    """16 rows x 256 codes: row r holds all 256 bytes rotated by 16 r."""
    base = np.arange(256, dtype=np.uint8)
    q = np.stack([np.roll(base, 16 * r) for r in range(16)])
    return S.Packed(torch.from_numpy(q).cuda(), torch.tensor([scale], dtype=torch.float32).cuda(),
                    None, 16, 256, F)


def assert_dequant_equal(got, ref, what):
    g = got.view(np.uint32)
    r = ref.view(np.uint32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), what
    bad = (g != r) & ~nan
    assert not bad.any(), f"{what}: {bad.sum()} weights differ, first at {np.argwhere(bad)[0]}"


@pytest.mark.parametrize("scale", [1.0, 0.0123, 2.0 ** -20, 3.3e4])
def test_dequant_every_code(scale):
    p = every_code_matrix(scale)
    got = T.dequant(p).cpu().numpy()
    q, s, _ = T.to_np(p)
    ref = O.dequant(q, s, None, p.N, p.K, 8, 0, O.LAYOUT_FP8_TENSOR)
    assert_dequant_equal(got, ref, f"scale {scale}")


@pytest.mark.parametrize("N,K", [(37, 512), (300, 2048), (5, 16)])
def test_dequant_page_recipe(N, K):
    p = T.to_dev(S.gen_matrix("f8dq", 0, 0, N, K, F))
    got = T.dequant(p).cpu().numpy()
    q, s, _ = T.to_np(p)
    assert_dequant_equal(got, O.dequant(q, s, None, N, K, 8, 0, O.LAYOUT_FP8_TENSOR),
                         f"{N}x{K}")


def test_codes_output_rejected():
    p = every_code_matrix(1.0)
    with pytest.raises(rq.RqError) as e:
        T.dequant(p, rq.RQ_OUT_CODES_I8)
    assert e.value.status == rq.RQ_ERR_UNSUPPORTED


def x_for(M, K, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((M, K), generator=g)
    x[:, K // 5] *= 100.0
    return x.half().cuda()


@pytest.mark.parametrize("N,K", [(37, 512), (300, 2048), (129, 4096), (70, 16), (33, 48 * 16)])
@pytest.mark.parametrize("entry", ["gemv", "gemm"])
def test_products(N, K, entry):
    p = T.to_dev(S.gen_matrix("f8mv", 1, 0, N, K, F))
    for M in (1, 2, 3, 4, 5, 8, 16, 33, 64):
        what = f"{entry} fp8 M={M} N={N} K={K}"
        T.say(what)
        x = x_for(M, K, seed=M * 7 + N)
        y = torch.full((M, N), float("nan"), device="cuda")
        T.run(entry, p, x, y)
        yr, b = T.oracle_y(p, x)
        T.assert_close(y, yr, b, what)


def test_zero_scale_and_negative_zero_codes():
    """A zero scale gives zero outputs (bound 0: +-0 required); codes 0x00 and
    0x80 (+0, -0) contribute nothing."""
    q = torch.tensor([[0x00, 0x80] * 16] * 20, dtype=torch.uint8).cuda()
    p = S.Packed(q, torch.tensor([0.5], device="cuda"), None, 20, 32, F)
    x = x_for(3, 32, seed=1)
    y = T.run("gemv", p, x)
    assert torch.count_nonzero(y) == 0
    p2 = every_code_matrix(0.0)
    x2 = x_for(2, 256, seed=2)
    codes = p2.qweight.clone()
    codes[(codes & 0x7F) == 0x7F] = 0x38  # no NaN codes
    p2 = S.Packed(codes, p2.scales, None, 16, 256, F)
    y2 = T.run("gemv", p2, x2)
    assert torch.count_nonzero(y2) == 0


def test_batched_mixed_shapes():
    shapes = [(256, 4096), (100, 1024), (64, 4096), (17, 512)] * 3
    mats = [T.to_dev(S.gen_matrix("f8b", i, 0, N, K, F)) for i, (N, K) in enumerate(shapes)]
    for M in (1, 4, 17):
        xs = [x_for(M, K, seed=50 + i) for i, (_, K) in enumerate(shapes)]
        ys = [torch.full((M, N), float("nan"), device="cuda") for (N, _) in shapes]
        rq.rq_gemv_batched([(p.qweight, p.scales, None, x, y, p.N, p.K)
                            for p, x, y in zip(mats, xs, ys)], M, 8, 0, rq.RQ_LAYOUT_FP8_TENSOR)
        for i, (p, x, y) in enumerate(zip(mats, xs, ys)):
            yr, b = T.oracle_y(p, x)
            T.assert_close(y, yr, b, f"batched fp8 M={M} problem {i} {p.N}x{p.K}")


@pytest.mark.parametrize("N,K", [(4096, 4096), (16384, 4096), (4096, 16384)])
def test_full_width_shapes(N, K):
    """The width-4096 decode shapes the page tiles (section "Operator
    Optimization Details"), at M = 1: every output of the 4096-row matrices, a
    seeded sample of rows (and the first and last) of the 16384-row one."""
    p = T.to_dev(S.gen_matrix("f8full", 0, 0, N, K, F))
    x = x_for(1, K, seed=N + K)
    y = torch.full((1, N), float("nan"), device="cuda")
    T.run("gemv", p, x, y)
    rows = None
    if N > 4096:
        g = torch.Generator().manual_seed(N)
        rows = sorted(set(torch.randperm(N, generator=g)[:64].tolist()) | {0, N - 1})
    sub = p if rows is None else S.rows_of(p, rows)
    yr, b = T.oracle_y(sub, x)
    got = y if rows is None else y[:, rows]
    T.assert_close(got, yr, b, f"fp8 {N}x{K} M=1")


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
def test_matrix_core_plans(tune, plan):
    """FP8 on every workgroup arrangement of the matrix-core kernel (the
    products accumulate straight into the tile; the matrix scale multiplies
    the stored sums), ragged N."""
    tune(RQ_GEMM_PLAN=plan)
    p = T.to_dev(S.gen_matrix("f8plan", 2, 0, 130, 2048, F))
    for M in (16, 48):
        x = x_for(M, 2048, seed=M + int(plan))
        y = torch.full((M, 130), float("nan"), device="cuda")
        T.run("gemm", p, x, y)
        yr, b = T.oracle_y(p, x)
        T.assert_close(y, yr, b, f"fp8 plan={plan} M={M}")


@pytest.mark.parametrize("splits", ["2", "4"])
def test_matrix_core_split_k(tune, splits):
    """K split over workgroups: each partial is scaled, the reduce adds them."""
    tune(RQ_GEMM_SPLITS=splits)
    p = T.to_dev(S.gen_matrix("f8split", 0, 0, 256, 8192, F))
    x = x_for(64, 8192, seed=5)
    y = torch.full((64, 256), float("nan"), device="cuda")
    T.run("gemm", p, x, y)
    yr, b = T.oracle_y(p, x)
    T.assert_close(y, yr, b, f"fp8 splits={splits}")
