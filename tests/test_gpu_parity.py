"""GPU parity: librq against the CPU oracle on the same seeded bytes.

Bar: rq_dequant and the unpacked codes bit-exact; rq_gemv and rq_gemm_smallm
within |y - y_ref| <= 1e-3 * sum_k |w x| per output; one-hot and integer-exact
inputs (where every partial sum is exact) bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle as O
import gemm_rwkv_decode_amd as rq
from gemm_rwkv_decode_amd import synth as S
from tests import rqtest as T

pytestmark = pytest.mark.gpu

ENTRIES = ["gemv", "gemm"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


@pytest.fixture
def tune(monkeypatch):
    """Set launch-shape overrides for one test; restored (and re-read) after."""
    def set_(**kv):
        for k, v in kv.items():
            monkeypatch.setenv(k, str(v))
        rq.tuning_reload()
    yield set_
    monkeypatch.undo()
    rq.tuning_reload()


def small(fmt, N, K, tag=0):
    p = S.gen_matrix(f"t{90 + tag}", 0, 0, N, K, fmt)
    return T.to_dev(p)


def x_for(M, K, seed, massive=True):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((M, K), generator=g)
    if massive:
        x[:, K // 3] *= 200.0
    return x.half().cuda()


# --------------------------------------------------------------- dequant ---
DQ_SHAPES = [(37, 512), (1, 256), (129, 768)]


@pytest.mark.parametrize("f", T.ALL_FORMATS, ids=lambda f: f.tag)
@pytest.mark.parametrize("N,K", DQ_SHAPES)
def test_dequant_bit_exact(f, N, K):
    if K % 256 and f.layout == S.LAYOUT_ASYM_SB:
        pytest.skip("asymmetric K must be whole superblocks")
    T.say(f"dequant {f.tag} N={N} K={K}")
    p = small(f, N, K)
    w = T.dequant(p).cpu().numpy()
    ref = T.oracle_dequant(p)
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))
    c = T.dequant(p, rq.RQ_OUT_CODES_I8).cpu().numpy()
    assert np.array_equal(c, T.oracle_codes(p))


@pytest.mark.parametrize("N,K,f", [(768, 768, S.INT4_G64), (2048, 2048, S.INT8_G16),
                                   (2560, 2560, S.ASYM4_G32), (4096, 4096, S.INT4_G64),
                                   (16384, 4096, S.INT4_G64), (2560, 10240, S.ASYM4_G32)])
def test_dequant_bit_exact_config_shapes(N, K, f):
    T.say(f"dequant {f.tag} N={N} K={K}")
    p = small(f, N, K, tag=1)
    w = T.dequant(p).cpu().numpy()
    assert np.array_equal(w.view(np.uint32), T.oracle_dequant(p).view(np.uint32))
    c = T.dequant(p, rq.RQ_OUT_CODES_I8).cpu().numpy()
    assert np.array_equal(c, T.oracle_codes(p))


@pytest.mark.parametrize("f", [S.INT4_G64, S.INT8_G16, S.ASYM4_G32], ids=lambda f: f.tag)
def test_dequant_subnormal_and_extreme_values(f):
    """binary16 subnormal / negative / largest scales, the code -8 (4-bit) and
    -128 (8-bit): still bit-exact."""
    N, K = 16, 512
    T.say(f"dequant extremes {f.tag}")
    p, codes = S.gen_matrix("t77", 0, 0, N, K, f, keep_codes=True)
    if f.layout == S.LAYOUT_SYM:
        lo = -8 if f.bits == 4 else -128
        codes[:, ::5] = lo
        sc = p.scales.clone().view(torch.int16)
        bits16 = [0x0001, 0x03FF, 0x8001, 0x7BFF, 0xFBFF, 0x0400, 0x0000, 0x8000]
        special = torch.tensor([b - 0x10000 if b >= 0x8000 else b for b in bits16],
                               dtype=torch.int16)
        sc.view(-1)[: special.numel() * 3] = special.repeat(3)
        p = S.encode(codes, f, scales=sc.view(torch.float16))
    else:
        B = K // 256
        d = torch.full((N, B), 2.0 ** -24, dtype=torch.float16)
        d[::2] = 65504.0
        m = torch.full((N, B), 2.0 ** -20, dtype=torch.float16)
        sc = torch.randint(0, 64, (N, B, 8), dtype=torch.int16).to(torch.uint8)
        mn = torch.randint(0, 64, (N, B, 8), dtype=torch.int16).to(torch.uint8)
        p = S.encode(codes, f, d=d, sc=sc, m=m, mn=mn)
    p = T.to_dev(p)
    w = T.dequant(p).cpu().numpy()
    assert np.array_equal(w.view(np.uint32), T.oracle_dequant(p).view(np.uint32))
    assert np.array_equal(T.dequant(p, rq.RQ_OUT_CODES_I8).cpu().numpy(), T.oracle_codes(p))


# ------------------------------------------------------- products, small ---
SHAPES = [(37, 512), (100, 768), (256, 2048), (8, 256)]
GEMV_MS = [1, 2, 3, 4, 5, 8, 9, 16, 33, 64]
GEMM_MS = [1, 7, 16, 17, 32, 48, 64]


@pytest.mark.parametrize("f", T.ALL_FORMATS, ids=lambda f: f.tag)
@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("entry", ENTRIES)
def test_product_parity_small(f, N, K, entry):
    if K % 256 and f.layout == S.LAYOUT_ASYM_SB:
        pytest.skip("asymmetric K must be whole superblocks")
    p = small(f, N, K, tag=2)
    for M in (GEMV_MS if entry == "gemv" else GEMM_MS):
        T.say(f"{entry} {f.tag} M={M} N={N} K={K}")
        x = x_for(M, K, seed=M * 1000 + N)
        y = T.run(entry, p, x)
        yr, b = T.oracle_y(p, x)
        T.assert_close(y, yr, b, f"{entry} {f.tag} M={M} N={N} K={K}")


@pytest.mark.parametrize("f", T.ALL_FORMATS, ids=lambda f: f.tag)
@pytest.mark.parametrize("N,K", SHAPES)
def test_vector_kernel_parity_small(tune, f, N, K):
    """The vector-unit kernel forced at every M (rq_gemv takes the matrix
    cores for most of these by itself), in passes of up to eight rows."""
    if K % 256 and f.layout == S.LAYOUT_ASYM_SB:
        pytest.skip("asymmetric K must be whole superblocks")
    tune(RQ_GEMV_KERNEL=1)
    p = small(f, N, K, tag=2)
    for M in (2, 3, 5, 8, 9, 16, 33, 64):
        T.say(f"vector {f.tag} M={M} N={N} K={K}")
        x = x_for(M, K, seed=M * 1000 + N + 7)
        y = torch.full((M, N), float("nan"), device="cuda")
        T.run("gemv", p, x, y)
        yr, b = T.oracle_y(p, x)
        T.assert_close(y, yr, b, f"vector {f.tag} M={M} N={N} K={K}")


@pytest.mark.parametrize("N,K,f", [(50, 544, T.fmt("int4g32", 4, 32, S.LAYOUT_SYM)),
                                   (70, 64, S.INT4_G64), (20, 16, S.INT8_G16),
                                   (3, 48 * 16, S.INT8_G16)])
@pytest.mark.parametrize("entry", ENTRIES)
def test_product_parity_odd_k(N, K, f, entry):
    """Row lengths whose chunk count has no power-of-two split (generic kernel;
    the matrix-core entry falls back to it too) and the smallest legal K."""
    p = small(f, N, K, tag=3)
    for M in (1, 3, 16, 40):
        T.say(f"{entry} odd-K {f.tag} M={M} N={N} K={K}")
        x = x_for(M, K, seed=M + K)
        y = T.run(entry, p, x)
        yr, b = T.oracle_y(p, x)
        T.assert_close(y, yr, b, f"{entry} {f.tag} M={M} N={N} K={K}")


def test_generic_kernel_forced(tune):
    """The generic kernel also serves shapes the tuned one handles."""
    tune(RQ_GEMV_LPR=-1, RQ_GEMV_KERNEL=1)
    for f in (S.INT4_G64, S.INT8_G16, S.ASYM4_G32):
        p = small(f, 45, 1024, tag=4)
        for M in (1, 5):
            T.say(f"generic {f.tag} M={M}")
            x = x_for(M, 1024, seed=M)
            y = T.run("gemv", p, x)
            yr, b = T.oracle_y(p, x)
            T.assert_close(y, yr, b, f"generic {f.tag} M={M}")


@pytest.mark.parametrize("lpr,cpl,npass", [(16, 1, 1), (16, 1, 2), (32, 1, 8), (8, 4, 2),
                                           (16, 2, 4), (64, 1, 4), (8, 1, 8)])
def test_gemv_launch_shapes(tune, lpr, cpl, npass):
    """Every instantiated launch shape, with a ragged last row block."""
    tune(RQ_GEMV_LPR=lpr, RQ_GEMV_CPL=cpl, RQ_GEMV_NPASS=npass, RQ_GEMV_KERNEL=1)
    for f in (S.INT4_G64, S.ASYM4_G32, S.INT8_G16):
        p = small(f, 1000, 512, tag=5)
        x = x_for(2, 512, seed=7)
        T.say(f"lpr={lpr} cpl={cpl} npass={npass} {f.tag}")
        y = T.run("gemv", p, x)
        yr, b = T.oracle_y(p, x)
        T.assert_close(y, yr, b, f"lpr={lpr} cpl={cpl} npass={npass} {f.tag}")
        x1 = x_for(1, 512, seed=8)
        y1 = T.run("gemv", p, x1)
        yr1, b1 = T.oracle_y(p, x1)
        T.assert_close(y1, yr1, b1, f"M=1 lpr={lpr} cpl={cpl} npass={npass} {f.tag}")


# ---------------------------------------------- decode kernels, M <= 4 ---
def chunk_k(f):
    """k per chunk of the matrix-core decode kernel (8 groups, or a superblock)."""
    return 256 if f.layout == S.LAYOUT_ASYM_SB else 8 * f.group


@pytest.mark.parametrize("f", T.ALL_FORMATS, ids=lambda f: f.tag)
@pytest.mark.parametrize("kern", ["vector", "matrix", "smallm"])
def test_decode_kernels(tune, f, kern):
    """The three kernels rq_gemv chooses from at M <= 4, forced: one chunk per
    wave, waves with unequal chunk counts, several chunks per wave, a ragged
    last row block and a single row.  Outputs start as NaN."""
    tune(RQ_GEMV_KERNEL={"vector": 1, "matrix": 2, "smallm": 3}[kern])
    ck = chunk_k(f)
    for N, K in [(37, 8 * ck), (300, 13 * ck), (129, 32 * ck), (1, 9 * ck)]:
        p = small(f, N, K, tag=7)
        for M in (1, 2, 3, 4):
            what = f"{kern} {f.tag} M={M} N={N} K={K}"
            T.say(what)
            x = x_for(M, K, seed=M * 31 + N)
            y = torch.full((M, N), float("nan"), device="cuda")
            T.run("gemv", p, x, y)
            yr, b = T.oracle_y(p, x)
            T.assert_close(y, yr, b, what)


@pytest.mark.parametrize("f,K,M", [
    (S.FP8_E4M3, 16384, 2),    # no tuned vector-unit shape: small-batch kernel
    (S.INT8_G16, 32768, 1),    # the same at M = 1
    (S.INT4_G64, 65536, 1),    # decode kernel
    (S.ASYM4_G32, 65536, 1),   # decode kernel
    (S.INT4_G64, 16384, 3),    # small-batch kernel at M = 3
    (S.ASYM5_G32, 4096, 4),    # small-batch kernel from M = 3 for every format
    (S.ASYM5_G32, 16384, 4),   # the same with long rows
], ids=lambda v: getattr(v, "tag", str(v)))
def test_kernel_choice_long_rows(f, K, M):
    """Rows too long for the vector-unit kernel's tuned launch shapes take a
    matrix-core kernel by themselves (rq_gemv and rq_gemv_batched)."""
    p = small(f, 70, K, tag=9)
    x = x_for(M, K, seed=K + M)
    yr, b = T.oracle_y(p, x)
    T.say(f"kernel choice {f.tag} K={K} M={M}")
    y = torch.full((M, 70), float("nan"), device="cuda")
    T.run("gemv", p, x, y)
    T.assert_close(y, yr, b, f"rq_gemv {f.tag} K={K} M={M}")
    yb = torch.full((M, 70), float("nan"), device="cuda")
    rq.rq_gemv_batched([(p.qweight, p.scales, p.zeros, x, yb, 70, K)], M, f.bits, f.group,
                       f.layout)
    T.assert_close(yb, yr, b, f"rq_gemv_batched {f.tag} K={K} M={M}")


@pytest.mark.parametrize("f,N,K,M,kernel", [
    # measured vector-unit launch shapes of heavier codes at M = 1
    (S.ASYM5_G32, 4096, 16384, 1, ("vector", 64, 1, 4)),
    (S.ASYM6_G32, 4096, 16384, 1, ("vector", 64, 1, 4)),
    (S.ASYM5_G32, 2560, 10240, 1, ("vector", 64, 1, 4)),
    (S.FP8_E4M3, 16384, 4096, 1, ("vector", 16, 2, 2)),
    (S.FP8_E4M3, 4096, 4096, 1, ("vector", 16, 2, 2)),
    # measured decode-kernel and vector-unit shapes at M = 3..4
    (S.ASYM4_G32, 10240, 2560, 3, ("decode_mfma", 0, 0, 0)),
    (S.INT4_G64, 2048, 8192, 4, ("vector", 64, 1, 4)),
    (S.INT4_G64, 2048, 8192, 3, ("vector", 64, 1, 4)),
], ids=lambda v: getattr(v, "tag", str(v)))
def test_tuned_shapes(f, N, K, M, kernel):
    """The RWKV-7 shapes with a measured kernel or launch shape of their own
    take it, and match the oracle at full size."""
    assert rq.gemv_config(M, N, K, f.bits, f.group, f.layout) == kernel
    p = small(f, N, K, tag=11)
    x = x_for(M, K, seed=N + K + M)
    yr, b = T.oracle_y(p, x)
    T.say(f"tuned shape {f.tag} {N}x{K} M={M} {kernel}")
    y = T.run("gemv", p, x)
    T.assert_close(y, yr, b, f"rq_gemv {f.tag} {N}x{K} M={M}")


def test_matrix_decode_kernel_falls_back(tune):
    """Forcing the matrix-core decode kernel where K holds fewer than eight
    chunks leaves the vector-unit kernel in charge (still correct)."""
    tune(RQ_GEMV_KERNEL=2)
    for f in (S.INT4_G64, S.INT8_G16, S.ASYM4_G32):
        K = 4 * chunk_k(f)
        p = small(f, 70, K, tag=8)
        x = x_for(2, K, seed=5)
        y = T.run("gemv", p, x)
        yr, b = T.oracle_y(p, x)
        T.assert_close(y, yr, b, f"fallback {f.tag}")


GEMM_PLANS = [str(i) for i in range(1, 28)]  # every workgroup arrangement (27)


def forced_plan_taken(f, M, N, K, plan):
    """Whether rq_gemm_smallm takes the forced plan for this problem; the
    chooser keeps its own choice where the plan cannot take the shape, and
    such a case would only re-test that choice."""
    cfg = rq.gemm_config(M, N, K, f.bits, f.group, f.layout)
    return cfg is not None and cfg[0] == int(plan)


@pytest.mark.parametrize("splits", ["1", "2", "4", "16"])
@pytest.mark.parametrize("plan", GEMM_PLANS)
def test_gemm_split_and_plans(tune, splits, plan):
    """Every workgroup arrangement of the matrix-core kernel, with and without
    K split over workgroups, ragged N.  Each case checks that the forced plan
    was the one launched; combinations the plan cannot take are skipped."""
    tune(RQ_GEMM_SPLITS=splits, RQ_GEMM_PLAN=plan)
    ran = 0
    for f in (S.INT4_G64, S.INT8_G16, S.ASYM4_G32):
        p = small(f, 300, 4096, tag=6)
        for M in (5, 16, 33, 64):  # M = 5 stages 8 x rows per round
            if not forced_plan_taken(f, M, 300, 4096, plan):
                T.say(f"gemm splits={splits} plan={plan} {f.tag} M={M}: plan cannot take it")
                continue
            got = rq.gemm_config(M, 300, 4096, f.bits, f.group, f.layout)
            T.say(f"gemm splits={splits} plan={plan} {f.tag} M={M}: launched {got}")
            x = x_for(M, 4096, seed=M)
            y = T.run("gemm", p, x)
            yr, b = T.oracle_y(p, x)
            T.assert_close(y, yr, b, f"splits={splits} plan={plan} {f.tag} M={M}")
            ran += 1
    if not ran:
        pytest.skip(f"plan {plan} fits none of these formats and M")


@pytest.mark.parametrize("plan", GEMM_PLANS)
@pytest.mark.parametrize("f", T.ALL_FORMATS, ids=lambda f: f.tag)
def test_gemm_plans_all_formats(tune, plan, f):
    tune(RQ_GEMM_PLAN=plan)
    p = small(f, 130, 2048, tag=9)
    ran = 0
    for M in (3, 7, 17, 48):  # 4 and 8 staged x rows, then 16 per M-tile
        if not forced_plan_taken(f, M, 130, 2048, plan):
            T.say(f"gemm plan={plan} {f.tag} M={M}: plan cannot take it")
            continue
        T.say(f"gemm plan={plan} {f.tag} M={M}")
        x = x_for(M, 2048, seed=M + 1)
        y = T.run("gemm", p, x)
        yr, b = T.oracle_y(p, x)
        T.assert_close(y, yr, b, f"plan={plan} {f.tag} M={M}")
        ran += 1
    if not ran:
        pytest.skip(f"plan {plan} cannot take {f.tag} at K=2048, M=3, 7, 17 or 48")


# ------------------------------------------------------ exact cases ---
@pytest.mark.parametrize("f", [S.INT4_G64, S.INT8_G16, S.ASYM4_G32], ids=lambda f: f.tag)
@pytest.mark.parametrize("entry", ENTRIES)
def test_one_hot_is_bit_exact(f, entry):
    """x rows = e_j: every output is one weight, reached without rounding."""
    N, K = 200, 1024
    p = small(f, N, K, tag=7)
    w = T.dequant(p).cpu()
    for M in (1, 16, 64):
        js = torch.arange(M) * 37 % K
        x = torch.zeros((M, K), dtype=torch.float16)
        x[torch.arange(M), js] = 1.0
        T.say(f"one-hot {entry} {f.tag} M={M}")
        y = T.run(entry, p, x.cuda()).cpu()
        assert torch.equal(y, w[:, js].T.contiguous()), f"{entry} {f.tag} M={M}"


@pytest.mark.parametrize("f", [S.INT4_G64, S.INT8_G16, S.ASYM4_G32], ids=lambda f: f.tag)
@pytest.mark.parametrize("entry", ENTRIES)
def test_integer_inputs_are_exact(f, entry):
    """Unit scales and small integer x: every partial sum is an exact integer
    in binary32, so y must equal the integer matmul of the unpacked codes."""
    N, K = 96, 2048
    p, codes = S.gen_matrix("t91", 0, 0, N, K, f, keep_codes=True)
    if f.layout == S.LAYOUT_SYM:
        p = S.encode(codes, f, scales=torch.ones((N, K // f.group), dtype=torch.float16))
        W = codes.to(torch.int64)
    else:
        B = K // 256
        g = torch.Generator().manual_seed(5)
        sc = torch.randint(0, 64, (N, B, 8), generator=g, dtype=torch.int16).to(torch.uint8)
        mn = torch.randint(0, 64, (N, B, 8), generator=g, dtype=torch.int16).to(torch.uint8)
        one = torch.ones((N, B), dtype=torch.float16)
        p = S.encode(codes, f, d=one, sc=sc, m=one, mn=mn)
        sck = sc.reshape(N, B * 8).repeat_interleave(32, dim=1).to(torch.int64)
        mnk = mn.reshape(N, B * 8).repeat_interleave(32, dim=1).to(torch.int64)
        W = sck * codes.to(torch.int64) - mnk
    p = T.to_dev(p)
    for M in (1, 4, 16, 64):
        g = torch.Generator().manual_seed(M)
        xi = torch.randint(-4, 5, (M, K), generator=g)
        T.say(f"integer {entry} {f.tag} M={M}")
        y = T.run(entry, p, xi.half().cuda()).cpu()
        expect = (xi.to(torch.int64) @ W.T).to(torch.float64)
        assert torch.equal(y.to(torch.float64), expect), f"{entry} {f.tag} M={M}"


# ------------------------------------------------------ contract details ---
@pytest.mark.parametrize("entry", ENTRIES)
def test_guard_bands_untouched_and_deterministic(entry):
    f = S.INT4_G64
    N, K, M, PAD = 333, 4096, 24, 64
    p = small(f, N, K, tag=8)
    x = x_for(M, K, seed=3)
    big = torch.full((M * N + 2 * PAD,), float("nan"), dtype=torch.float32, device="cuda")
    big.view(torch.int32)[:PAD] = 0x7FC0DEAD
    big.view(torch.int32)[-PAD:] = 0x7FC0BEEF
    y = big[PAD:PAD + M * N].view(M, N)
    T.say(f"guard {entry}")
    T.run(entry, p, x, y)
    torch.cuda.synchronize()
    gi = big.view(torch.int32).cpu()
    assert torch.all(gi[:PAD] == 0x7FC0DEAD) and torch.all(gi[-PAD:] == 0x7FC0BEEF)
    y1 = y.clone()
    T.run(entry, p, x, y)
    assert torch.equal(y1.view(torch.int32), y.view(torch.int32)), "not deterministic"
    yr, b = T.oracle_y(p, x)
    T.assert_close(y, yr, b, f"guard {entry}")


def test_misaligned_output_is_rejected_and_untouched():
    p = small(S.INT4_G64, 64, 256, tag=9)
    x = x_for(1, 256, seed=1)
    buf = torch.zeros(65, dtype=torch.float32, device="cuda")
    with pytest.raises(rq.RqError) as e:
        rq.rq_gemv(p.qweight, p.scales, None, x, buf[1:], 1, 64, 256, 4, 64, 0)
    assert e.value.status == rq.RQ_ERR_ALIGN
    assert torch.count_nonzero(buf).item() == 0


def test_side_stream():
    p = small(S.INT8_G16, 512, 2048, tag=10)
    x = x_for(16, 2048, seed=2)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y1 = T.run("gemv", p, x)
        y2 = T.run("gemm", p, x)
    s.synchronize()
    yr, b = T.oracle_y(p, x)
    T.assert_close(y1, yr, b, "side stream gemv")
    T.assert_close(y2, yr, b, "side stream gemm")


# ------------------------------------------------------------ batched ---
@pytest.mark.parametrize("f", [S.INT4_G64, S.INT8_G16, S.ASYM4_G32], ids=lambda f: f.tag)
@pytest.mark.parametrize("M", [1, 3, 5, 8, 15, 17, 48])
def test_batched_matches_oracle(f, M):
    """Mixed N and K in one call (K groups share launches), more problems than
    one launch holds, and a K the tuned kernel cannot split."""
    shapes = [(256, 1024), (100, 1024), (300, 2048), (64, 1024)] * 5 + [(40, 768)]
    shapes += [(130, 4096), (64, 4096), (17, 4096)] * 7  # matrix-core kernels at M <= 4
    if f.layout == S.LAYOUT_SYM and f.bits == 4:
        shapes.append((33, 64 * 7))  # 14 chunks: generic kernel
    mats = [small(f, N, K, tag=20 + i) for i, (N, K) in enumerate(shapes)]
    xs = [x_for(M, K, seed=100 + i) for i, (_, K) in enumerate(shapes)]
    ys = [torch.full((M, N), float("nan"), device="cuda") for (N, _) in shapes]
    T.say(f"batched {f.tag} M={M} count={len(shapes)}")
    rq.rq_gemv_batched([(p.qweight, p.scales, p.zeros, x, y, p.N, p.K)
                        for p, x, y in zip(mats, xs, ys)], M, f.bits, f.group, f.layout)
    for i, (p, x, y) in enumerate(zip(mats, xs, ys)):
        yr, b = T.oracle_y(p, x)
        T.assert_close(y, yr, b, f"batched {f.tag} M={M} problem {i} {p.N}x{p.K}")


@pytest.mark.parametrize("M", [1, 3, 32])
def test_batched_at_the_maximum_count(M):
    """RQ_MAX_BATCH problems in one call: two K groups, several launches each."""
    f = S.INT4_G64
    shapes = [(64 + 8 * (i % 5), 1024 if i % 3 else 2048) for i in range(rq.RQ_MAX_BATCH)]
    mats = [small(f, N, K, tag=400 + i) for i, (N, K) in enumerate(shapes)]
    xs = [x_for(M, K, seed=500 + i) for i, (_, K) in enumerate(shapes)]
    ys = [torch.full((M, N), float("nan"), device="cuda") for (N, _) in shapes]
    T.say(f"batched maximum count M={M}")
    rq.rq_gemv_batched([(p.qweight, p.scales, p.zeros, x, y, p.N, p.K)
                        for p, x, y in zip(mats, xs, ys)], M, f.bits, f.group, f.layout)
    for i, (p, x, y) in enumerate(zip(mats, xs, ys)):
        yr, b = T.oracle_y(p, x)
        T.assert_close(y, yr, b, f"batched maximum M={M} problem {i} {p.N}x{p.K}")


def test_batched_rejects_overlapping_outputs():
    p = small(S.INT4_G64, 64, 256, tag=40)
    x = x_for(1, 256, seed=4)
    y = torch.zeros(200, device="cuda")
    with pytest.raises(rq.RqError) as e:
        rq.rq_gemv_batched([(p.qweight, p.scales, None, x, y[:64], 64, 256),
                            (p.qweight, p.scales, None, x, y[32:96], 64, 256)], 1, 4, 64, 0)
    assert e.value.status == rq.RQ_ERR_ALIAS
    assert torch.count_nonzero(y).item() == 0


def test_prepared_calls_match_direct_calls():
    f = S.INT4_G64
    p = small(f, 512, 4096, tag=41)
    x = x_for(1, 4096, seed=5)
    x32 = x_for(32, 4096, seed=6)
    y1 = torch.full((1, 512), float("nan"), device="cuda")
    y2 = torch.full((32, 512), float("nan"), device="cuda")
    c1 = rq.prepare("rq_gemv", p.qweight, p.scales, None, x, y1, 1, 512, 4096, 4, 64, 0)
    c2 = rq.prepare("rq_gemm_smallm", p.qweight, p.scales, None, x32, y2, 32, 512, 4096, 4,
                    64, 0)
    c3 = rq.prepare("rq_gemv_batched", [(p.qweight, p.scales, None, x, y1, 512, 4096)], 1, 4,
                    64, 0)
    for c, y, xx in ((c1, y1, x), (c2, y2, x32), (c3, y1, x)):
        y.fill_(float("nan"))
        c()
        yr, b = T.oracle_y(p, xx)
        T.assert_close(y, yr, b, "prepared")
