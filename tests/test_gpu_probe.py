"""The measurement kernels of include/rq_probe.h on the GPU: each runs, the
copy moves its bytes exactly, the grid barrier's exchanged data is never
stale, and the rates come out in a plausible range for an MI355X (so a probe
that silently did no work would fail)."""
import pytest
import torch

import gemm_rwkv_decode_amd as rq
from gemm_rwkv_decode_amd import probe as P
from tests.rqtest import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def test_copy_moves_exact_bytes():
    say("probe copy")
    src = torch.randint(-2**31, 2**31 - 1, (1 << 20,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    assert rq.lib().rq_probe_copy(src.data_ptr(), dst.data_ptr(), src.numel() * 4, _stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_read_and_empty_run():
    say("probe read, empty")
    L = rq.lib()
    src = torch.ones(1 << 22, dtype=torch.int32, device="cuda")
    sink = torch.zeros(2048, dtype=torch.int32, device="cuda")
    assert L.rq_probe_read(src.data_ptr(), src.numel() * 4, sink.data_ptr(), 0, 0, _stream()) == 0
    assert L.rq_probe_empty(_stream()) == 0
    torch.cuda.synchronize()


def test_barrier_data_never_stale():
    say("probe barrier")
    L = rq.lib()
    blocks = 256
    flags = torch.zeros(2048 + 65 * blocks, dtype=torch.int32, device="cuda")
    bad = torch.full((blocks,), -1, dtype=torch.int32, device="cuda")
    st = L.rq_probe_barrier(flags.data_ptr(), 4, blocks, 20, 1 << 20, bad.data_ptr(), _stream())
    if st == rq.RQ_ERR_LAUNCH:
        pytest.skip("cooperative launch of 256 workgroups refused")
    assert st == 0
    torch.cuda.synchronize()
    assert int(bad.abs().sum()) == 0


def test_mfma_valu_and_overlap_rates():
    say("probe mfma, valu, overlap")
    m = P.mfma_probe(blocks=512, iters=200)
    assert all(300 < r["tflops"] < 3000 for r in m["shapes"]), m
    v = P.valu_probe(blocks=512, iters=50)
    assert set(v["cycles"]) == set(P.VALU_KINDS)
    # a wave instruction takes at least one and at most a few dozen cycles
    assert all(1.0 < c < 40.0 for c in v["cycles"].values()), v
    o = P.overlap_probe(iters=100)
    assert len(o["rows"]) == 12
    for r in o["rows"]:
        for k in ("mfma_only", "vector_only", "same_wave", "separate_waves"):
            assert 1.0 < r[k] < 500.0, r
        # doing both kinds of work never takes less than the larger alone
        assert r["same_wave"] > 0.8 * max(r["mfma_only"], r["vector_only"]), r
