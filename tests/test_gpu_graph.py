"""A decode step captured as a HIP graph and replayed gives the same outputs
as direct launches, bit for bit, on every replay (the kernels are
deterministic), with other GPU work between replays.  Covers the grouped
vector-unit launch (M = 1), the small-batch matrix-core kernel with four
staged activation rows (M = 4), grouped
matrix-core launches (M = 16) and the split-K path with its in-launch
reduction (M = 64, few long rows), rq_gemv on the matrix cores captured as
the first call on a fresh stream, and rq_gemm_smallm captured after one eager
call at the largest split shapes (its workspace then exists, so the captured
call allocates and waits for nothing), or as the first call (K kept whole)."""
import pytest
import torch

from gemm_rwkv_decode_amd import step as ST
from gemm_rwkv_decode_amd import synth as S
from tests.rqtest import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("wkey,M", [("rwkv7-0.1b", 1), ("rwkv7-1.5b", 4), ("rwkv7-1.5b", 16),
                                    ("rwkv7-1.5b", 64)])
def test_graph_replays_match_direct_launches(wkey, M):
    cfg = S.CONFIGS[wkey]
    f = cfg.formats[0]
    mats = [m for m in cfg.matrices() if m[0] < 2]
    W = [S.gen_matrix(cfg.key, l, mi, N, K, f, device="cuda") for (l, mi, N, K) in mats]
    X = [S.gen_x(cfg, l, mi, M, K, device="cuda") for (l, mi, N, K) in mats]
    Y = [torch.full((M, N), float("nan"), device="cuda") for (_, _, N, _) in mats]
    s = torch.cuda.Stream()
    calls = ST.step_calls(mats, W, X, Y, "layer", stream=s)
    say(f"[graph] {wkey} M={M}: {len(calls)} launches")
    with torch.cuda.stream(s):
        for c in calls:  # eager: also creates any workspace before capture
            c()
    torch.cuda.synchronize()
    eager = [y.clone() for y in Y]
    for y in Y:
        y.fill_(float("nan"))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for c in calls:
            c()
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device="cuda")
    for r in range(4):
        for y in Y:
            y.fill_(float("nan"))
        junk.mul_(1.0001)  # other work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (y, e) in enumerate(zip(Y, eager)):
            assert torch.equal(y, e), f"replay {r}, matrix {i} {mats[i]}"


@pytest.mark.parametrize("M", [8, 12])
def test_rq_gemv_captures_as_first_call(M):
    """rq_gemv takes the matrix cores from M = 5 on but never allocates, so it
    can be captured as the first call on a fresh stream, also for long rows
    that rq_gemm_smallm would split through its workspace."""
    import gemm_rwkv_decode_amd as rq
    from tests import rqtest as T
    f = S.INT4_G64
    N, K = 512, 16384
    p = T.to_dev(S.gen_matrix("graph-first", 0, M, N, K, f))
    g0 = torch.Generator().manual_seed(M)
    x = torch.randn((M, K), generator=g0).half().cuda()
    y = torch.full((M, N), float("nan"), device="cuda")
    s = torch.cuda.Stream()
    call = rq.prepare("rq_gemv", p.qweight, p.scales, None, x, y, M, N, K, f.bits, f.group,
                      f.layout, stream=s)
    say(f"[graph] rq_gemv first call captured, M={M}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    yr, b = T.oracle_y(p, x)
    ye = torch.full((M, N), float("nan"), device="cuda")
    rq.rq_gemv(p.qweight, p.scales, None, x, ye, M, N, K, f.bits, f.group, f.layout)
    torch.cuda.synchronize()
    T.assert_close(ye, yr, b, f"eager M={M}")
    junk = torch.randn(1 << 20, device="cuda")
    for r in range(3):
        y.fill_(float("nan"))
        junk.mul_(1.0001)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ye), f"replay {r}"


@pytest.mark.parametrize("M,N,K", [(64, 4096, 16384), (32, 4096, 16384), (64, 1000, 4096)])
def test_rq_gemm_smallm_captured_after_one_eager_call(M, N, K):
    """The binding makes its workspace for a stream at the first call there
    (a torch tensor; the library never allocates); a capture of the same call
    afterwards holds no allocation, free or wait, and every
    replay matches the eager call bit for bit (counters reset each time)."""
    import gemm_rwkv_decode_amd as rq
    from tests import rqtest as T
    f = S.INT4_G64
    cfg = rq.gemm_config(M, N, K, f.bits, f.group, f.layout)
    assert cfg[1] > 1, f"{N}x{K} M={M} does not split K"
    p = T.to_dev(S.gen_matrix("graph-smallm", 0, M, N, K, f))
    g0 = torch.Generator().manual_seed(M + N)
    x = torch.randn((M, K), generator=g0).half().cuda()
    s = torch.cuda.Stream()
    ye = torch.full((M, N), float("nan"), device="cuda")
    say(f"[graph] rq_gemm_smallm {N}x{K} M={M} splits={cfg[1]}: eager, then captured")
    rq.rq_gemm_smallm(p.qweight, p.scales, None, x, ye, M, N, K, f.bits, f.group, f.layout,
                      stream=s)
    torch.cuda.synchronize()
    yr, b = T.oracle_y(p, x)
    T.assert_close(ye, yr, b, f"eager {N}x{K} M={M}")
    y = torch.full((M, N), float("nan"), device="cuda")
    call = rq.prepare("rq_gemm_smallm", p.qweight, p.scales, None, x, y, M, N, K, f.bits,
                      f.group, f.layout, stream=s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device="cuda")
    for r in range(4):
        y.fill_(float("nan"))
        junk.mul_(1.0001)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), ye.view(torch.int32)), f"replay {r}"


def test_rq_gemm_smallm_captured_as_first_call_keeps_k_whole():
    """As the first call on a fresh stream under capture the binding has no
    workspace yet: the call keeps K whole (no allocation under capture) and is still at
    parity on every replay."""
    import gemm_rwkv_decode_amd as rq
    from tests import rqtest as T
    f = S.INT4_G64
    M, N, K = 32, 2048, 16384
    assert rq.gemm_config(M, N, K, f.bits, f.group, f.layout)[1] > 1
    p = T.to_dev(S.gen_matrix("graph-smallm-first", 0, M, N, K, f))
    g0 = torch.Generator().manual_seed(7)
    x = torch.randn((M, K), generator=g0).half().cuda()
    y = torch.full((M, N), float("nan"), device="cuda")
    s = torch.cuda.Stream()
    call = rq.prepare("rq_gemm_smallm", p.qweight, p.scales, None, x, y, M, N, K, f.bits,
                      f.group, f.layout, stream=s)
    say("[graph] rq_gemm_smallm first call captured")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    yr, b = T.oracle_y(p, x)
    first = None
    for r in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        T.assert_close(y, yr, b, f"replay {r}")
        if first is None:
            first = y.clone()
        assert torch.equal(y.view(torch.int32), first.view(torch.int32)), f"replay {r}"
