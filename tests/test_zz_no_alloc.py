"""rq_gemm_smallm_noalloc: the allocation-free form of rq_gemm_smallm.

It runs the same kernels, arrangement and K split as rq_gemm_smallm_ws (which
the binding's rq_gemm_smallm calls with its per-stream workspace), with the
split-K partial sums in the library's fixed device array instead of a
caller's workspace.  Checked through the C interface:

* two calls in a row, each splitting K (the second smaller), bit-identical to
  rq_gemm_smallm_ws on the same inputs and within 1e-3 * sum|w x| of the oracle;
* a shape that keeps K whole;
* a call whose partial sums would exceed the array (a forced split count)
  returns RQ_ERR_SCRATCH and leaves y untouched;
* captured into a graph as the first call on a fresh stream (where
  the binding has no workspace yet), every replay matches the eager
  call, with other work on the GPU between replays.
"""
import ctypes

import pytest
import torch

import gemm_rwkv_decode_amd as rq
from gemm_rwkv_decode_amd import synth as S
from tests import rqtest as T

pytestmark = pytest.mark.gpu


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


def mat(f, N, K, tag):
    return T.to_dev(S.gen_matrix(f"noalloc{tag}", 0, 0, N, K, f))


def xs(M, K, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((M, K), generator=g)
    x[:, K // 7] *= 150.0
    return x.half().cuda()


def c_call(p, x, y, stream=None):
    """rq_gemm_smallm_noalloc through the C interface; returns the status."""
    f = p.fmt
    s = stream if stream is not None else torch.cuda.current_stream()
    return rq.lib().rq_gemm_smallm_noalloc(
        p.qweight.data_ptr(), p.scales.data_ptr(),
        None if p.zeros is None else p.zeros.data_ptr(), x.data_ptr(), y.data_ptr(),
        x.shape[0], p.N, p.K, f.bits, f.group, f.layout, ctypes.c_void_p(s.cuda_stream))


def nan_y(M, N):
    return torch.full((M, N), float("nan"), device="cuda")


CASES = [  # (format, N, K, M): the first two of each pair split K
    (S.INT4_G64, 4096, 16384, 32), (S.INT4_G64, 1000, 4096, 64),
    (S.INT8_G16, 2048, 8192, 64), (S.INT8_G16, 300, 2048, 49),
    (S.ASYM4_G32, 2560, 10240, 64), (S.ASYM4_G32, 640, 2560, 50),
]


@pytest.mark.parametrize("i", [0, 2, 4], ids=["int4g64", "int8g16", "asym4g32"])
def test_two_calls_in_a_row_match_the_workspace_entry(i):
    for (f, N, K, M) in CASES[i:i + 2]:
        cfg = rq.gemm_config(M, N, K, f.bits, f.group, f.layout)
        assert cfg is not None and cfg[1] > 1, f"{f.tag} {N}x{K} M={M} does not split K"
    p1, p2 = (mat(f, N, K, i + j) for j, (f, N, K, M) in enumerate(CASES[i:i + 2]))
    (f, N1, K1, M1), (_, N2, K2, M2) = CASES[i:i + 2]
    x1, x2 = xs(M1, K1, 1 + i), xs(M2, K2, 2 + i)
    y1, y2 = nan_y(M1, N1), nan_y(M2, N2)
    T.say(f"noalloc {f.tag}: {N1}x{K1} M={M1}, then {N2}x{K2} M={M2}")
    assert c_call(p1, x1, y1) == rq.RQ_OK
    assert c_call(p2, x2, y2) == rq.RQ_OK
    r1 = T.run("gemm", p1, x1)
    r2 = T.run("gemm", p2, x2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), r1.view(torch.int32)), "first call"
    assert torch.equal(y2.view(torch.int32), r2.view(torch.int32)), "second call"
    yr, b = T.oracle_y(p1, x1)
    T.assert_close(y1, yr, b, f"noalloc {f.tag} {N1}x{K1} M={M1}")
    yr, b = T.oracle_y(p2, x2)
    T.assert_close(y2, yr, b, f"noalloc {f.tag} {N2}x{K2} M={M2}")


def test_k_kept_whole():
    f, N, K, M = S.INT4_G64, 12288, 4096, 32
    assert rq.gemm_config(M, N, K, f.bits, f.group, f.layout)[1] == 1
    p = mat(f, N, K, 9)
    x = xs(M, K, 9)
    y = nan_y(M, N)
    T.say("noalloc K whole")
    assert c_call(p, x, y) == rq.RQ_OK
    r = T.run("gemm", p, x)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), r.view(torch.int32))


def test_too_large_for_the_scratch_is_rejected(tune):
    f, N, K, M = S.INT4_G64, 8192, 16384, 64
    tune(RQ_GEMM_SPLITS=8)
    cfg = rq.gemm_config(M, N, K, f.bits, f.group, f.layout)
    assert cfg[1] * M * N * 4 > rq.RQ_NOALLOC_SCRATCH_BYTES
    p = mat(f, N, K, 10)
    x = xs(M, K, 10)
    y = nan_y(M, N)
    T.say("noalloc oversize")
    assert c_call(p, x, y) == rq.RQ_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool(torch.isnan(y).all()), "a rejected call wrote y"
    with pytest.raises(rq.RqError):
        rq.rq_gemm_smallm_noalloc(p.qweight, p.scales, None, x, y, M, N, K, 4, 64, 0)


def test_graph_capture_on_a_fresh_stream():
    f, N, K, M = S.INT4_G64, 4096, 16384, 32
    p = mat(f, N, K, 11)
    x = xs(M, K, 11)
    y_eager = nan_y(M, N)
    assert c_call(p, x, y_eager) == rq.RQ_OK
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    y = nan_y(M, N)
    g = torch.cuda.CUDAGraph()
    T.say("noalloc graph capture")
    with torch.cuda.graph(g, stream=s):
        assert c_call(p, x, y, stream=s) == rq.RQ_OK
    other = mat(f, 1000, 4096, 12)
    xo = xs(64, 4096, 12)
    for rep in range(4):
        y.fill_(float("nan"))
        g.replay()
        yo = nan_y(64, 1000)
        assert c_call(other, xo, yo) == rq.RQ_OK  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y_eager.view(torch.int32)), f"replay {rep}"
    yr, b = T.oracle_y(p, x)
    T.assert_close(y, yr, b, "noalloc graph replay")
