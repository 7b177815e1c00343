"""K split over workgroups on the matrix-core kernel: partial tiles in the
per-stream workspace, added in K-range order by the wave that finishes each
16-row tile last (same launch; arrival counters reset by that wave).  Against the oracle: forced and automatic splits, calls back to back
that reuse the workspace (with changing splits, M and shapes, and a grouped
launch in between), bit-identical repeats, and the width-4096 FFN-value
shape at full size.  Products within |y - y_ref| <= 1e-3 * sum_k |w x|;
outputs start as NaN."""
import pytest
import torch

from gemm_rwkv_decode_amd import synth as S
import gemm_rwkv_decode_amd as rq
from tests import rqtest as T

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
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


def mat(f, N, K, tag):
    return T.to_dev(S.gen_matrix(f"sk{tag}", 0, 0, N, K, f))


def x_for(M, K, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((M, K), generator=g)
    x[:, K // 3] *= 200.0
    return x.half().cuda()


def gemm_nan(p, x):
    y = torch.full((x.shape[0], p.N), float("nan"), device="cuda")
    return T.run("gemm", p, x, y)


@pytest.mark.parametrize("f", [S.INT4_G64, S.INT8_G16, S.ASYM4_G32, S.FP8_E4M3],
                         ids=lambda f: f.tag)
def test_calls_back_to_back(tune, f):
    """A sequence of split launches with different splits, M, plans and row
    counts on one stream, sharing the workspace."""
    seq = [(2, 16, 300, "5"), (4, 33, 130, "3"), (16, 64, 300, "2"), (3, 17, 77, "1"),
           (8, 48, 1000, "7"), (4, 64, 300, "5")]
    for i, (sp, M, N, plan) in enumerate(seq):
        tune(RQ_GEMM_SPLITS=sp, RQ_GEMM_PLAN=plan)
        p = mat(f, N, 8192, i)
        x = x_for(M, 8192, seed=60 + i)
        T.say(f"split-k {f.tag} splits={sp} M={M} N={N} plan={plan}")
        y = gemm_nan(p, x)
        yr, b = T.oracle_y(p, x)
        T.assert_close(y, yr, b, f"{f.tag} call {i} splits={sp} M={M} N={N}")


def test_repeats_bit_identical(tune):
    tune(RQ_GEMM_SPLITS=8)
    p = mat(S.INT4_G64, 1000, 16384, 20)
    x = x_for(32, 16384, seed=9)
    ys = [gemm_nan(p, x) for _ in range(5)]
    for y in ys[1:]:
        assert torch.equal(y, ys[0])
    yr, b = T.oracle_y(p, x)
    T.assert_close(ys[0], yr, b, "16384 K, M=32, 8 splits")


@pytest.mark.parametrize("M", [16, 32, 64])
def test_ffn_value_shape_automatic_split(M):
    """4096 x 16384 (K split automatically) at full size, every row checked."""
    p = mat(S.INT4_G64, 4096, 16384, 30)
    x = x_for(M, 16384, seed=300 + M)
    T.say(f"split-k automatic 4096x16384 M={M}")
    y = gemm_nan(p, x)
    yr, b = T.oracle_y(p, x)
    T.assert_close(y, yr, b, f"4096x16384 M={M}")


def test_split_then_batched_then_split(tune):
    """A grouped launch (never split) between split calls on the same stream."""
    tune(RQ_GEMM_SPLITS=4)
    f = S.INT4_G64
    p = mat(f, 300, 4096, 40)
    x = x_for(32, 4096, seed=41)
    yr, b = T.oracle_y(p, x)
    T.assert_close(gemm_nan(p, x), yr, b, "split before")
    mats = [mat(f, 200, 4096, 42 + i) for i in range(3)]
    ys = [torch.full((32, 200), float("nan"), device="cuda") for _ in mats]
    rq.rq_gemv_batched([(q.qweight, q.scales, q.zeros, x, yb, q.N, q.K)
                        for q, yb in zip(mats, ys)], 32, f.bits, f.group, f.layout)
    for i, (q, yb) in enumerate(zip(mats, ys)):
        yq, bq = T.oracle_y(q, x)
        T.assert_close(yb, yq, bq, f"batched {i}")
    T.assert_close(gemm_nan(p, x), yr, b, "split after")
