"""A decode step captured as a HIP graph and replayed gives the same outputs
as direct launches, bit for bit, on every replay (the kernels are
deterministic), with other GPU work between replays.  Covers the grouped
vector-unit launch (M = 1), the matrix-core decode kernel (M = 4), grouped
matrix-core launches (M = 16) and the split-K path with its reduce kernel
(M = 64, few long rows)."""
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
