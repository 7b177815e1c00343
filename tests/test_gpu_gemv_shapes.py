"""Every instantiated launch shape of the vector-unit GEMV, integer-exact.

The vector-unit kernel adds each row's products over the LPR lanes that share
the row; a lane's row sums (NP rows x M activation rows) are added together,
halving the values at each exchange level (cross-row swaps at distances 16
and 32, row mirrors at 8 and 4, quad permutes at 2 and 1), and the lane that
ends with a row's total stores it.  A wrong pairing at any level, or a total
stored for the wrong row or activation row, changes the result.  With unit
scales and small integer codes and activations every product and partial sum
is an integer below 2^24, so the output must equal the int64 matmul of the
codes exactly, whatever the summation order.  Every (lanes per row, chunks per
lane, rows per lane) the kernel is instantiated with, at M = 1, 2, 4 and 8
(one pass of 1, 2, 4 or 8 activation rows) and a ragged row count; a forced
shape the chooser does not take is reported and skipped.  Outputs start as NaN.
"""
import pytest
import torch

import gemm_rwkv_decode_amd as rq
from gemm_rwkv_decode_amd import synth as S
from tests import rqtest as T

pytestmark = pytest.mark.gpu

# (lanes per row, 16-byte chunks per lane): the instantiated pairs; rows per
# lane 1, 2, 4 and 8 each (8 only below four activation rows per pass)
SHAPES = [(8, 1), (16, 1), (32, 1), (64, 1), (8, 2), (16, 2), (8, 4)]
FORMATS = [S.INT4_G64, S.INT8_G16]


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


def integer_matrix(f, N, K, seed):
    lo, hi = (-8, 7) if f.bits == 4 else (-128, 127)
    g = torch.Generator().manual_seed(seed)
    codes = torch.randint(lo, hi + 1, (N, K), generator=g, dtype=torch.int16).to(torch.int8)
    sc = torch.ones((N, K // f.group), dtype=torch.float16)
    return T.to_dev(S.encode(codes, f, scales=sc)), codes.to(torch.int64)


@pytest.mark.parametrize("f", FORMATS, ids=lambda f: f.tag)
@pytest.mark.parametrize("lpr,cpl", SHAPES, ids=[f"lpr{a}cpl{b}" for a, b in SHAPES])
def test_every_launch_shape_integer_exact(tune, f, lpr, cpl):
    N, K = 1003, 2048
    p, W = integer_matrix(f, N, K, seed=lpr * 10 + cpl)
    ran = 0
    for M in (1, 2, 4, 8):
        for npass in (1, 2, 4, 8):
            tune(RQ_GEMV_LPR=lpr, RQ_GEMV_CPL=cpl, RQ_GEMV_NPASS=npass, RQ_GEMV_KERNEL=1)
            got = rq.gemv_config(M, N, K, f.bits, f.group, f.layout)
            if got != ("vector", lpr, cpl, npass):
                T.say(f"{f.tag} M={M} lpr={lpr} cpl={cpl} np={npass}: not taken ({got})")
                continue
            g = torch.Generator().manual_seed(M * 100 + npass)
            xi = torch.randint(-4, 5, (M, K), generator=g)
            T.say(f"{f.tag} M={M} lpr={lpr} cpl={cpl} np={npass}")
            y = torch.full((M, N), float("nan"), device="cuda")
            rq.rq_gemv(p.qweight, p.scales, None, xi.half().cuda(), y, M, N, K, f.bits,
                       f.group, f.layout)
            expect = (xi.to(torch.int64) @ W.T).to(torch.float64)
            assert torch.equal(y.cpu().to(torch.float64), expect), \
                f"{f.tag} M={M} lpr={lpr} cpl={cpl} np={npass}"
            ran += 1
    assert ran > 0, "no forced shape was taken"
