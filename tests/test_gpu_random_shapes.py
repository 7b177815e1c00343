"""Seeded random shapes through every product entry point, against the oracle.

Each case draws a format (every layout, bit width and group the library
takes), an M between 1 and 64, a row count N up to 2500 (ragged against every
tile) and a K that is any valid multiple for the format up to 8192 (including
odd numbers of groups, which the matrix-core kernel does not take).  The same
product goes through rq_gemv, rq_gemm_smallm and rq_gemm_smallm_noalloc, and
together with a second random problem of the same format through
rq_gemv_batched; every output starts as NaN and must lie within
1e-3·Σ|w x| of the oracle."""
import math

import numpy as np
import pytest
import torch

import gemm_rwkv_decode_amd as rq
from gemm_rwkv_decode_amd import synth as S
from tests import rqtest as T

pytestmark = pytest.mark.gpu

FORMATS = T.ALL_FORMATS + [S.ASYM5_G32, S.ASYM6_G32, S.FP8_E4M3]
MS = (1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 32, 33, 47, 48, 63, 64)
CASES = 120
MACS = 12 << 20  # oracle work per case, at most


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def k_step(f):
    """The smallest K granularity the format takes: whole groups, rows of whole
    16-byte chunks, whole superblocks for the asymmetric layout."""
    if f.layout == S.LAYOUT_ASYM_SB:
        return S.SUPERBLOCK
    row = 128 // f.bits  # codes per 16 bytes
    return row * f.group // math.gcd(row, f.group) if f.group else row


def draw(rng, M=None):
    f = FORMATS[int(rng.integers(len(FORMATS)))]
    M = int(rng.choice(MS)) if M is None else M
    ks = k_step(f)
    kmax = max(1, min(8192 // ks, MACS // (ks * M)))
    K = ks * int(rng.integers(1, kmax + 1))
    nmax = max(1, min(2500, MACS // (K * M)))
    N = int(rng.integers(1, nmax + 1))
    return f, M, N, K


def x_of(M, K, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((M, K), generator=g)
    x[:, int(torch.randint(0, K, (1,), generator=g))] *= 50.0  # one massive channel
    return x.half().cuda()


def nan_y(M, N):
    return torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")


@pytest.mark.parametrize("seed", range(CASES))
def test_random_shape(seed):
    rng = np.random.default_rng(1000 + seed)
    f, M, N, K = draw(rng)
    T.say(f"random case {seed}: {f.tag} M={M} N={N} K={K}")
    p = T.to_dev(S.gen_matrix(f"rand{seed}", 0, 0, N, K, f))
    x = x_of(M, K, 5000 + seed)
    yr, b = T.oracle_y(p, x)
    args = (p.qweight, p.scales, p.zeros, x)
    tail = (M, N, K, f.bits, f.group, f.layout)
    for name, fn in (("rq_gemv", rq.rq_gemv), ("rq_gemm_smallm", rq.rq_gemm_smallm),
                     ("rq_gemm_smallm_noalloc", rq.rq_gemm_smallm_noalloc)):
        y = nan_y(M, N)
        fn(*args, y, *tail)
        T.assert_close(y, yr, b, f"{name} {f.tag} M={M} {N}x{K}")
    # batched with a second problem of the same format and M
    f2, _, N2, K2 = draw(rng, M)
    while f2.tag != f.tag:
        f2, _, N2, K2 = draw(rng, M)
    p2 = T.to_dev(S.gen_matrix(f"rand{seed}", 0, 1, N2, K2, f))
    x2 = x_of(M, K2, 7000 + seed)
    y1, y2 = nan_y(M, N), nan_y(M, N2)
    rq.rq_gemv_batched([(p.qweight, p.scales, p.zeros, x, y1, N, K),
                        (p2.qweight, p2.scales, p2.zeros, x2, y2, N2, K2)],
                       M, f.bits, f.group, f.layout)
    T.assert_close(y1, yr, b, f"batched {f.tag} M={M} {N}x{K}")
    yr2, b2 = T.oracle_y(p2, x2)
    T.assert_close(y2, yr2, b2, f"batched {f.tag} M={M} {N2}x{K2}")


@pytest.mark.parametrize("seed", range(40))
def test_random_dequant(seed):
    """rq_dequant at random shapes: binary32 values and int8 codes bit-exact."""
    rng = np.random.default_rng(3000 + seed)
    f, _, N, K = draw(rng, 1)
    T.say(f"random dequant {seed}: {f.tag} N={N} K={K}")
    p = T.to_dev(S.gen_matrix(f"rdq{seed}", 0, 0, N, K, f))
    w = T.dequant(p).cpu().numpy()
    ref = T.oracle_dequant(p)
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32)), (f.tag, N, K)
    if f.layout != S.LAYOUT_FP8_TENSOR:
        c = T.dequant(p, rq.RQ_OUT_CODES_I8).cpu().numpy()
        assert np.array_equal(c, T.oracle_codes(p)), (f.tag, N, K)


@pytest.mark.parametrize("seed", range(30))
def test_random_forced_kernel_and_plan(seed, monkeypatch):
    """rq_gemv with its kernel forced (vector units, matrix-core decode,
    small-batch matrix cores; each falls back where it cannot take the shape),
    and rq_gemm_smallm with a random plan and split count (ignored where they
    do not fit), at random shapes."""
    rng = np.random.default_rng(4000 + seed)
    f, M, N, K = draw(rng)
    p = T.to_dev(S.gen_matrix(f"rfk{seed}", 0, 0, N, K, f))
    x = x_of(M, K, 9000 + seed)
    yr, b = T.oracle_y(p, x)
    try:
        for kern in (1, 2, 3):
            monkeypatch.setenv("RQ_GEMV_KERNEL", str(kern))
            rq.tuning_reload()
            T.say(f"random forced {seed}: {f.tag} M={M} N={N} K={K} kernel {kern} "
                  f"-> {rq.gemv_config(M, N, K, f.bits, f.group, f.layout)}")
            y = T.run("gemv", p, x)
            T.assert_close(y, yr, b, f"forced kernel {kern} {f.tag} M={M} {N}x{K}")
        monkeypatch.delenv("RQ_GEMV_KERNEL")
        plan, splits = int(rng.integers(1, 28)), int(rng.choice([1, 2, 3, 4, 8]))
        monkeypatch.setenv("RQ_GEMM_PLAN", str(plan))
        monkeypatch.setenv("RQ_GEMM_SPLITS", str(splits))
        rq.tuning_reload()
        T.say(f"random plan {seed}: {f.tag} M={M} N={N} K={K} asked p{plan}s{splits} -> "
              f"{rq.gemm_config(M, N, K, f.bits, f.group, f.layout)}")
        y = T.run("gemm", p, x)
        T.assert_close(y, yr, b, f"plan {plan} splits {splits} {f.tag} M={M} {N}x{K}")
    finally:
        for v in ("RQ_GEMV_KERNEL", "RQ_GEMM_PLAN", "RQ_GEMM_SPLITS"):
            monkeypatch.delenv(v, raising=False)
        rq.tuning_reload()
