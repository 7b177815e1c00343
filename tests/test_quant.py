"""The offline quantizer (gemm_rwkv_decode_amd.quant), on the CPU: every
layout it emits decodes (through the oracle) to weights within the rounding
bound of round-to-nearest, the E[x^2]-weighted search never does worse than
RTN on its own measure and does better where it matters, and FP8 follows the
FP8 page's recipe bit for bit."""
import numpy as np
import pytest
import torch

import oracle as O
from gemm_rwkv_decode_amd import quant as Q
from gemm_rwkv_decode_amd import synth as S

SYM_FMTS = [S.INT4_G64, S.INT8_G16, S.Fmt("int4g32", 4, 32, S.LAYOUT_SYM),
            S.Fmt("int4g128", 4, 128, S.LAYOUT_SYM), S.Fmt("int8g64", 8, 64, S.LAYOUT_SYM)]
ASYM_FMTS = [S.ASYM4_G32, S.ASYM5_G32, S.ASYM6_G32]


def weights(N=24, K=512, seed=0):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K)) * np.exp(rng.standard_normal((N, 1)))
    W[:, 7] *= 6.0  # an outlier column
    return W


def deq(p):
    q = p.qweight.numpy()
    s = p.scales.numpy()
    z = None if p.zeros is None else p.zeros.numpy()
    return O.dequant(q, s, z, p.N, p.K, p.fmt.bits, p.fmt.group, p.fmt.layout).astype(np.float64)


def werr(W, Wh, xsq):
    return float((xsq[None, :] * (W - Wh) ** 2).sum())


@pytest.mark.parametrize("f", SYM_FMTS, ids=lambda f: f.tag)
def test_sym_rtn_within_half_a_step(f):
    W = weights()
    p = Q.quantize(W, f, method="rtn")
    Wh = deq(p)
    s = np.repeat(p.scales.numpy().astype(np.float64), f.group, axis=1)
    qmax = Q.SYM_QMAX[f.bits]
    # half a step, plus what lies beyond the binary16-rounded range
    bound = s / 2 + np.maximum(0.0, np.abs(W) - s * qmax) + 1e-12 * np.abs(W)
    assert np.all(np.abs(W - Wh) <= bound)
    codes = O.unpack_codes(p.qweight.numpy(), p.N, p.K, f.bits, f.layout)
    assert codes.min() >= -qmax and codes.max() <= qmax


@pytest.mark.parametrize("f", ASYM_FMTS, ids=lambda f: f.tag)
def test_asym_rtn_within_half_a_step(f):
    W = weights(K=768)
    p = Q.quantize(W, f, method="rtn")
    Wh = deq(p)
    qmax = (1 << f.bits) - 1
    rec = p.scales.numpy()
    zr = p.zeros.numpy()
    N, K = W.shape
    for n in range(N):
        for k in range(0, K, 5):
            b, j = k // 256, (k % 256) // 32
            db, sc = O.unpack_record(rec[n, b])
            mb, mn = O.unpack_record(zr[n, b])
            s = O.half_to_double(db) * sc[j]
            t = O.half_to_double(mb) * mn[j]
            lo, hi = -t, s * qmax - t
            excess = max(0.0, lo - W[n, k], W[n, k] - hi)
            assert abs(W[n, k] - Wh[n, k]) <= s / 2 + excess + 1e-6 * abs(W[n, k]) + 1e-9, (n, k)


@pytest.mark.parametrize("f", SYM_FMTS + ASYM_FMTS, ids=lambda f: f.tag)
def test_search_never_worse_and_usually_better(f):
    K = 768 if f.layout == S.LAYOUT_ASYM_SB else 512
    W = weights(K=K, seed=3)
    xsq = np.ones(K)
    xsq[[5, 300]] = 1e4  # massive channels
    e_rtn = werr(W, deq(Q.quantize(W, f, xsq, method="rtn")), xsq)
    e_srch = werr(W, deq(Q.quantize(W, f, xsq, method="search")), xsq)
    assert e_srch <= e_rtn * (1 + 1e-9)
    assert e_srch < 0.97 * e_rtn


def test_search_follows_the_activation_weights():
    """Weighting a channel by E[x^2] lowers its error against an unweighted
    search."""
    f = S.INT4_G64
    W = weights(K=512, seed=5)
    ch = np.arange(0, 512, 64) + 3  # one channel per group
    xsq = np.ones(512)
    xsq[ch] = 1e6
    plain = deq(Q.quantize(W, f, None))
    weighted = deq(Q.quantize(W, f, xsq))
    assert (np.abs(W - weighted)[:, ch] ** 2).sum() < (np.abs(W - plain)[:, ch] ** 2).sum()


def test_fp8_is_the_page_recipe():
    W = weights(K=256, seed=9)
    p = Q.quantize(W, S.FP8_E4M3)
    Wt = torch.from_numpy(W.astype(np.float32))
    scale = Wt.abs().max() / 448.0
    ref = (Wt / scale).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    assert torch.equal(p.qweight, ref) and p.scales.item() == scale.item()
    Wh = deq(p)
    # E4M3 keeps 3 fraction bits: relative error <= 2^-4 on normals
    big = np.abs(W) > 2 ** -6 * scale.item()
    assert np.all(np.abs(W - Wh)[big] <= 2 ** -4 * np.abs(W)[big] * (1 + 1e-6))


@pytest.mark.parametrize("f", [S.INT4_G64, S.ASYM5_G32, S.FP8_E4M3], ids=lambda f: f.tag)
def test_zero_matrix(f):
    p = Q.quantize(np.zeros((4, 256)), f)
    assert np.all(deq(p) == 0.0)


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        Q.quantize(np.full((2, 64), np.nan), S.INT4_G64)
    with pytest.raises(ValueError):
        Q.quantize(np.zeros((2, 100)), S.INT4_G64)
    with pytest.raises(ValueError):
        Q.quantize(np.zeros((2, 300)), S.ASYM4_G32)
    with pytest.raises(ValueError):
        Q.quantize(np.zeros((2, 64)), S.INT4_G64, xsq=np.ones(5))
    with pytest.raises(ValueError):
        Q.quantize(np.zeros((2, 64)), S.INT4_G64, method="gptq")


@pytest.mark.gpu
@pytest.mark.parametrize("f", [S.INT4_G64, S.INT8_G16, S.ASYM4_G32, S.ASYM6_G32, S.FP8_E4M3],
                         ids=lambda f: f.tag)
def test_quantized_product_end_to_end(f):
    """Quantize real weights, multiply on the GPU: within the product tolerance
    of the oracle on the same bytes, and within the quantization error of the
    real-valued product (|y - x W^T| <= sum_k |x| |w - w^| + tolerance)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import rqtest as T
    K = 1024
    W = weights(N=200, K=K, seed=12)
    rng = np.random.default_rng(13)
    x = rng.standard_normal((3, K)).astype(np.float16)
    x[:, 100] *= 50
    xsq = (x.astype(np.float64) ** 2).mean(axis=0)
    p = Q.quantize(W, f, xsq)
    pd = T.to_dev(p)
    xd = torch.from_numpy(x).cuda()
    y = T.run("gemv", pd, xd).cpu().numpy().astype(np.float64)
    yr, b = T.oracle_y(pd, xd)
    T.assert_close(torch.from_numpy(y), yr, b, f"quantized {f.tag}")
    Wh = deq(p)
    exact = x.astype(np.float64) @ W.T
    qerr = np.abs(x.astype(np.float64)) @ np.abs(W - Wh).T
    assert np.all(np.abs(y - exact) <= qerr + 1e-3 * b + 1e-9)
