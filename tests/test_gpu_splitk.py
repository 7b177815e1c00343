"""K split over workgroups on the matrix-core kernel: partial tiles in the
caller's workspace (the binding's per-stream one unless a test passes its
own), added in K-range order by the wave that finishes each
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


def c_smallm(p, x, y, ws=None, ws_bytes=0, plain=False):
    """rq_gemm_smallm (plain) or rq_gemm_smallm_ws through the C interface."""
    import ctypes
    f = p.fmt
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [p.qweight.data_ptr(), p.scales.data_ptr(),
            None if p.zeros is None else p.zeros.data_ptr(), x.data_ptr(), y.data_ptr(),
            x.shape[0], p.N, p.K, f.bits, f.group, f.layout]
    if plain:
        return rq.lib().rq_gemm_smallm(*args, s)
    return rq.lib().rq_gemm_smallm_ws(*args, None if ws is None else ws.data_ptr(), ws_bytes, s)


@pytest.mark.parametrize("f,N,K,M", [(S.INT4_G64, 4096, 16384, 32),
                                     (S.ASYM4_G32, 2560, 10240, 64),
                                     (S.INT8_G16, 1000, 4096, 64)],
                         ids=["int4g64", "asym4g32", "int8g16"])
def test_caller_workspace_and_k_kept_whole(f, N, K, M):
    """At shapes the chooser splits: a workspace of exactly the queried size
    (counters zeroed by the caller) gives the binding's result bit for bit,
    twice in a row; rq_gemm_smallm (no workspace) and rq_gemm_smallm_ws with
    NULL keep K whole and agree bit for bit; all within the oracle's bound;
    a workspace one byte short is refused with y untouched."""
    need = rq.rq_gemm_smallm_workspace_size(M, N, K, f.bits, f.group, f.layout)
    assert need > 0, "shape does not split K"
    p = mat(f, N, K, f"ws{f.tag}")
    x = x_for(M, K, 11)
    yr, b = T.oracle_y(p, x)
    T.say(f"caller workspace {f.tag} {N}x{K} M={M} need={need}")
    ya = gemm_nan(p, x)  # binding's workspace
    torch.cuda.synchronize()
    T.assert_close(ya, yr, b, "auto workspace")
    ws = torch.zeros(need // 4, dtype=torch.int32, device="cuda")
    for r in range(2):
        y = torch.full((M, N), float("nan"), device="cuda")
        assert c_smallm(p, x, y, ws, need) == rq.RQ_OK
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), ya.view(torch.int32)), f"call {r}"
    assert torch.count_nonzero(ws[:16384]).item() == 0, "counters not left at zero"
    y1 = torch.full((M, N), float("nan"), device="cuda")
    y2 = torch.full((M, N), float("nan"), device="cuda")
    assert c_smallm(p, x, y1, plain=True) == rq.RQ_OK
    assert c_smallm(p, x, y2) == rq.RQ_OK
    torch.cuda.synchronize()
    T.assert_close(y1, yr, b, "K kept whole")
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    y3 = torch.full((M, N), float("nan"), device="cuda")
    assert c_smallm(p, x, y3, ws, need - 1) == rq.RQ_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.isnan(y3).all()


def test_graph_with_caller_workspace_forced_split(tune):
    """A graph captured with the caller's workspace and a forced 8-way split
    (more than the automatic choice) replays at parity into NaN-filled
    outputs, bit-identical on every replay, with other GPU work between."""
    f, M, N, K = S.INT4_G64, 32, 2048, 16384
    tune(RQ_GEMM_SPLITS=8)
    assert rq.gemm_config(M, N, K, f.bits, f.group, f.layout)[1] == 8
    need = rq.rq_gemm_smallm_workspace_size(M, N, K, f.bits, f.group, f.layout)
    p = mat(f, N, K, "graphws")
    x = x_for(M, K, 5)
    yr, b = T.oracle_y(p, x)
    ws = torch.zeros(need // 4, dtype=torch.int32, device="cuda")
    y = torch.full((M, N), float("nan"), device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    call = rq.prepare("rq_gemm_smallm_ws", p.qweight, p.scales, None, x, y, M, N, K, f.bits,
                      f.group, f.layout, ws, stream=s)
    T.say(f"graph with caller workspace {N}x{K} M={M} splits=8 need={need}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device="cuda")
    first = None
    for r in range(4):
        y.fill_(float("nan"))
        junk.mul_(1.0001)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        T.assert_close(y, yr, b, f"replay {r}")
        if first is None:
            first = y.clone()
        assert torch.equal(y.view(torch.int32), first.view(torch.int32)), f"replay {r}"


def test_two_streams_two_workspaces_at_once():
    """Split-K calls on two streams at the same time, each with its own
    caller workspace (and the binding's per-stream workspaces), do not
    interfere: every output matches the single-stream result bit for bit."""
    f, M, N, K = S.INT4_G64, 32, 4096, 16384
    need = rq.rq_gemm_smallm_workspace_size(M, N, K, f.bits, f.group, f.layout)
    assert need > 0
    mats = [mat(f, N, K, f"2s{i}") for i in range(2)]
    xs = [x_for(M, K, 20 + i) for i in range(2)]
    ref = []
    for p, x in zip(mats, xs):
        ref.append(gemm_nan(p, x))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [torch.zeros(need // 4, dtype=torch.int32, device="cuda") for _ in range(2)]
    for auto in (False, True):
        T.say(f"two streams at once, {'binding' if auto else 'caller'} workspaces")
        ys = [torch.full((M, N), float("nan"), device="cuda") for _ in range(2)]
        torch.cuda.synchronize()
        for r in range(4):  # several rounds in flight on both streams
            for i in range(2):
                with torch.cuda.stream(streams[i]):
                    rq.rq_gemm_smallm(mats[i].qweight, mats[i].scales, None, xs[i], ys[i], M, N,
                                      K, f.bits, f.group, f.layout, stream=streams[i],
                                      workspace=rq.AUTO if auto else wss[i])
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(ys[i].view(torch.int32), ref[i].view(torch.int32)), (auto, i)
