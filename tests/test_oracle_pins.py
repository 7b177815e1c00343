"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test ties one part of the oracle to something other than its own code:
hand-derived literal bytes (tests/golden/format_literals.json, with the pages'
passages and the readings they rest on), library conversions (numpy's binary16
decoding, Python's exact rationals), integer-exact special cases checked with
an integer matmul, one-hot inputs, dense float64 matmuls, and round trips.
A plausible slip in the oracle -- swapped nibbles, a lost sign, a wrong group
index, a transposed operand, a dropped shift term, a wrong tolerance test --
breaks at least one of them (see test_oracle_mutants.py, which builds such
slips into copies of the oracle and runs these pins on them).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "format_literals.json")
SYM, ASYM = O.LAYOUT_SYM, O.LAYOUT_ASYM_SB


@pytest.fixture(scope="module")
def lit():
    with open(GOLDEN) as f:
        return json.load(f)


def hx(s):
    return int(s, 16) if isinstance(s, str) else int(s)


def half_bits(v):
    return int(np.array([v], dtype=np.float16).view(np.uint16)[0])


# ---------------------------------------------------------------- binary16 ---
def test_half_to_double_every_finite_value():
    """Every finite binary16 decodes exactly as numpy's float16 -> float64."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([O.half_to_double(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.all(np.isinf(got[np.isinf(ref)]))
    assert np.all(np.isnan(got[np.isnan(ref)]))
    # sign of zero survives
    assert np.signbit(O.half_to_double(0x8000))


def test_half_to_double_landmarks():
    assert O.half_to_double(0x3C00) == 1.0
    assert O.half_to_double(0xC000) == -2.0
    assert O.half_to_double(0x7BFF) == 65504.0
    assert O.half_to_double(0x0001) == 2.0 ** -24
    assert O.half_to_double(0x0400) == 2.0 ** -14
    assert O.half_to_double(0x03FF) == 1023 * 2.0 ** -24


# ------------------------------------------------------------ code unpack ---
def test_sym4_literals(lit):
    for e in lit["sym4_bytes"]:
        q = np.array([[hx(e["byte"])]], dtype=np.uint8)
        assert O.unpack_codes(q, 1, 2, 4, SYM).tolist() == [e["codes"]], e


def test_asym4_literals(lit):
    for e in lit["asym4_bytes"]:
        q = np.array([[hx(e["byte"])]], dtype=np.uint8)
        assert O.unpack_codes(q, 1, 2, 4, ASYM).tolist() == [e["codes"]], e


def test_sym8_literals(lit):
    for e in lit["sym8_bytes"]:
        q = np.array([[hx(e["byte"])]], dtype=np.uint8)
        assert O.unpack_codes(q, 1, 1, 8, SYM).tolist() == [[e["code"]]], e


@pytest.mark.parametrize("bits,layout", [(4, SYM), (4, ASYM), (8, SYM)])
def test_every_byte_round_trips(bits, layout):
    """unpack then pack is the identity on all 256 byte values, and pack then
    unpack is the identity on every code tuple one byte holds."""
    allb = np.arange(256, dtype=np.uint8)
    K = 2 if bits == 4 else 1
    q = allb.reshape(256, 1)
    codes = O.unpack_codes(q, 256, K, bits, layout)
    assert np.array_equal(O.pack_codes(codes, bits, layout), q)
    if bits == 4:
        lo, hi = (-8, 7) if layout == SYM else (0, 15)
        pairs = np.array([(a, b) for a in range(lo, hi + 1) for b in range(lo, hi + 1)],
                         dtype=np.int8)
        assert np.array_equal(O.unpack_codes(O.pack_codes(pairs, 4, layout), 256, 2, 4,
                                             layout), pairs)
        # every code tuple maps to a distinct byte
        assert len(set(O.pack_codes(pairs, 4, layout).ravel().tolist())) == 256


def test_pack_rejects_out_of_range():
    with pytest.raises(ValueError):
        O.pack_codes(np.array([[8, 0]], dtype=np.int8), 4, SYM)
    with pytest.raises(ValueError):
        O.pack_codes(np.array([[-1, 0]], dtype=np.int8), 4, ASYM)


def test_code_positions_in_a_long_row():
    """The code at k sits in byte k/2 of its row, rows are K/2 bytes apart."""
    rng = np.random.default_rng(1)
    N, K = 5, 64
    codes = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    q = O.pack_codes(codes, 4, SYM)
    for n, k in [(0, 0), (0, 1), (3, 17), (4, 63), (2, 32)]:
        byte = int(q[n, k // 2])
        nib = (byte >> 4) if k % 2 else (byte & 15)
        assert O.code_at(q, N, K, 4, SYM, n, k) == codes[n, k]
        assert (nib - 16 if nib >= 8 else nib) == codes[n, k]


# ----------------------------------------------------------------- records ---
def test_record_literals(lit):
    for e in lit["records"]:
        rec = O.pack_record(hx(e["base"]), e["sub"])
        assert [int(b) for b in rec] == [hx(b) for b in e["bytes"]], e
        base, sub = O.unpack_record(np.array([hx(b) for b in e["bytes"]], dtype=np.uint8))
        assert base == hx(e["base"]) and sub.tolist() == e["sub"]


def test_record_round_trip_every_position_and_value():
    for j in range(8):
        for v in range(64):
            sub = [0] * 8
            sub[j] = v
            sub[(j + 3) % 8] = 63 - v
            rec = O.pack_record(0x1234, sub)
            base, got = O.unpack_record(rec)
            assert base == 0x1234 and got.tolist() == sub
    with pytest.raises(ValueError):
        O.pack_record(0, [64, 0, 0, 0, 0, 0, 0, 0])


# ----------------------------------------------------------------- dequant ---
def _one_row(K, head):
    q = np.zeros((1, K), dtype=np.uint8)
    q[0, :len(head)] = [hx(b) for b in head]
    return q


def test_dequant_sym4_literal(lit):
    e = lit["dequant_sym4"]
    K, g = e["K"], e["group"]
    q = _one_row(K // 2, e["head_bytes"])
    s = np.full((1, K // g), hx(e["scale"]), dtype=np.uint16).view(np.float16)
    w = O.dequant(q, s, None, 1, K, 4, g, SYM)
    assert w[0, :6].tolist() == e["head_weights"]
    assert np.all(w[0, 6:] == 0)


def test_dequant_sym4_subnormal_scale(lit):
    e = lit["dequant_sym4_subnormal"]
    K, g = e["K"], e["group"]
    q = _one_row(K // 2, e["head_bytes"])
    s = np.full((1, K // g), hx(e["scale"]), dtype=np.uint16).view(np.float16)
    w = O.dequant(q, s, None, 1, K, 4, g, SYM)
    assert w[0, :2].tolist() == e["head_weights"]


def test_dequant_sym8_literal(lit):
    e = lit["dequant_sym8"]
    K, g = e["K"], e["group"]
    q = _one_row(K, e["head_bytes"])
    s = np.full((1, K // g), hx(e["scale"]), dtype=np.uint16).view(np.float16)
    w = O.dequant(q, s, None, 1, K, 8, g, SYM)
    assert w[0, :4].tolist() == e["head_weights"]


@pytest.mark.parametrize("case", ["dequant_asym", "dequant_asym_rounding"])
def test_dequant_asym_literal(lit, case):
    e = lit[case]
    K = e["K"]
    q = np.zeros((1, K // 2), dtype=np.uint8)
    for pos, b in e["code_bytes"].items():
        q[0, int(pos)] = hx(b)
    srec = O.pack_record(hx(e["d"]), e["sc"]).reshape(1, 1, 8)
    zrec = O.pack_record(hx(e["m"]), e["mn"]).reshape(1, 1, 8)
    w = O.dequant(q, srec, zrec, 1, K, 4, 32, ASYM)
    for k, v in e["weights"].items():
        assert w[0, int(k)] == v, (k, w[0, int(k)], v)


@pytest.mark.parametrize("bits,group", [(4, 64), (4, 32), (4, 128), (8, 16), (8, 64)])
def test_dequant_sym_closed_form(bits, group):
    """w[n][k] = s[n][k//g] * q[n][k] exactly, for codes known before packing."""
    rng = np.random.default_rng(bits * 1000 + group)
    N, K = 7, 4 * group
    lo, hi = (-8, 7) if bits == 4 else (-128, 127)
    codes = rng.integers(lo, hi + 1, size=(N, K)).astype(np.int8)
    scales = np.exp(rng.uniform(np.log(1e-6), np.log(60.0), size=(N, K // group)))
    scales = scales.astype(np.float16)
    q = O.pack_codes(codes, bits, SYM)
    w = O.dequant(q, scales, None, N, K, bits, group, SYM)
    expect = (np.repeat(scales.astype(np.float64), group, axis=1)
              * codes.astype(np.float64)).astype(np.float32)
    assert np.array_equal(w.view(np.uint32), expect.view(np.uint32))


def test_dequant_sym_power_of_two_scales():
    """With scale 2^e the weight is q * 2^e (ldexp), for every e binary16 holds."""
    N, K, g = 40, 64, 64
    rng = np.random.default_rng(5)
    codes = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    exps = np.arange(-24, 16)  # subnormal 2^-24 .. 2^15
    scales = np.ldexp(1.0, exps).astype(np.float16).reshape(N, 1)
    w = O.dequant(O.pack_codes(codes, 4, SYM), scales, None, N, K, 4, g, SYM)
    assert np.array_equal(w, np.ldexp(codes.astype(np.float32), exps.reshape(N, 1)))


def _asym_problem(rng, N, K, dlo=1e-4, dhi=2e-3):
    B = K // 256
    codes = rng.integers(0, 16, size=(N, K)).astype(np.int8)
    d = np.exp(rng.uniform(np.log(dlo), np.log(dhi), size=(N, B))).astype(np.float16)
    m = np.exp(rng.uniform(np.log(dlo), np.log(dhi), size=(N, B))).astype(np.float16)
    sc = rng.integers(0, 64, size=(N, B, 8)).astype(np.uint8)
    mn = rng.integers(0, 64, size=(N, B, 8)).astype(np.uint8)
    srec = np.zeros((N, B, 8), dtype=np.uint8)
    zrec = np.zeros((N, B, 8), dtype=np.uint8)
    for n in range(N):
        for b in range(B):
            srec[n, b] = O.pack_record(half_bits(d[n, b]), sc[n, b])
            zrec[n, b] = O.pack_record(half_bits(m[n, b]), mn[n, b])
    return codes, d, m, sc, mn, srec, zrec


@pytest.mark.parametrize("dlo,dhi,mlo,mhi", [(1e-7, 10.0, 1e-7, 10.0),
                                             (1.0, 10.0, 1e-7, 1e-5)])
def test_dequant_asym_exact_rational(dlo, dhi, mlo, mhi):
    """w = binary32 nearest the exact rational (d*sc_j)*q - (m*mn_j), with
    j = (k mod 256) // 32, for codes and sub-codes known before packing.  The
    second case makes s*q and t far apart, so most results need rounding."""
    rng = np.random.default_rng(11)
    N, K = 3, 512
    codes, d, m, sc, mn, srec, zrec = _asym_problem(rng, N, K, dlo, dhi)
    m = np.exp(rng.uniform(np.log(mlo), np.log(mhi), size=m.shape)).astype(np.float16)
    for n in range(N):
        for b in range(K // 256):
            zrec[n, b] = O.pack_record(half_bits(m[n, b]), mn[n, b])
    w = O.dequant(O.pack_codes(codes, 4, ASYM), srec, zrec, N, K, 4, 32, ASYM)
    for n in range(N):
        for k in range(0, K, 7):
            b, j = k // 256, (k % 256) // 32
            exact = (Fraction(float(d[n, b])) * int(sc[n, b, j]) * int(codes[n, k])
                     - Fraction(float(m[n, b])) * int(mn[n, b, j]))
            # the exact value is a binary64 here; numpy rounds it once to binary32
            assert Fraction(float(exact)) == exact
            assert w[n, k] == np.float32(float(exact)), (n, k)


def test_dequant_asym_zero_subcodes_give_zero():
    rng = np.random.default_rng(2)
    N, K = 4, 256
    codes, d, m, sc, mn, srec, zrec = _asym_problem(rng, N, K)
    z = np.zeros(8, dtype=np.uint8)
    for n in range(N):
        srec[n, 0] = O.pack_record(half_bits(d[n, 0]), z)
        zrec[n, 0] = O.pack_record(half_bits(m[n, 0]), z)
    w = O.dequant(O.pack_codes(codes, 4, ASYM), srec, zrec, N, K, 4, 32, ASYM)
    assert np.all(w == 0)


def test_dequant_rejects_bad_shapes():
    q = np.zeros((1, 32), dtype=np.uint8)
    s = np.zeros((1, 1), dtype=np.float16)
    with pytest.raises(ValueError):
        O.dequant(q, s, None, 1, 64, 4, 48, SYM)   # K % group != 0
    with pytest.raises(ValueError):
        O.dequant(q, s, None, 1, 64, 4, 64, ASYM)  # asym needs zeros and K % 256
    with pytest.raises(ValueError):
        O.dequant(q, s, None, 1, 64, 3, 64, SYM)   # 3-bit codes do not exist


# -------------------------------------------------------------------- gemv ---
@pytest.mark.parametrize("bits,group,M", [(4, 64, 1), (4, 64, 3), (8, 16, 2), (8, 16, 17),
                                          (4, 32, 5)])
def test_gemv_integer_exact_sym(bits, group, M):
    """Scale 1 and integer x: y is an integer the fp64 sum reaches exactly, so it
    must equal the int64 matmul codes @ x^T of the codes known before packing."""
    rng = np.random.default_rng(100 + bits + M)
    N, K = 9, 8 * group
    lo, hi = (-8, 7) if bits == 4 else (-128, 127)
    codes = rng.integers(lo, hi + 1, size=(N, K)).astype(np.int8)
    xi = rng.integers(-6, 7, size=(M, K))
    scales = np.ones((N, K // group), dtype=np.float16)
    y, b = O.gemv_ref(O.pack_codes(codes, bits, SYM), scales, None,
                      xi.astype(np.float16), N, K, bits, group, SYM)
    expect = xi.astype(np.int64) @ codes.astype(np.int64).T
    assert np.array_equal(y, expect.astype(np.float64))
    assert np.array_equal(b, (np.abs(xi) @ np.abs(codes.astype(np.int64)).T).astype(np.float64))


def test_gemv_integer_exact_asym():
    """d = m = 1, integer sub-codes and x: w = sc_j*q - mn_j is an integer and y
    must equal the int64 matmul built from the unpacked pieces."""
    rng = np.random.default_rng(7)
    N, K, M = 5, 768, 3
    codes = rng.integers(0, 16, size=(N, K)).astype(np.int8)
    B = K // 256
    sc = rng.integers(0, 64, size=(N, B, 8)).astype(np.uint8)
    mn = rng.integers(0, 64, size=(N, B, 8)).astype(np.uint8)
    srec = np.stack([np.stack([O.pack_record(0x3C00, sc[n, b]) for b in range(B)])
                     for n in range(N)])
    zrec = np.stack([np.stack([O.pack_record(0x3C00, mn[n, b]) for b in range(B)])
                     for n in range(N)])
    xi = rng.integers(-4, 5, size=(M, K))
    y, _ = O.gemv_ref(O.pack_codes(codes, 4, ASYM), srec, zrec, xi.astype(np.float16),
                      N, K, 4, 32, ASYM)
    sck = np.repeat(sc.reshape(N, B * 8), 32, axis=1).astype(np.int64)
    mnk = np.repeat(mn.reshape(N, B * 8), 32, axis=1).astype(np.int64)
    w_int = sck * codes.astype(np.int64) - mnk
    assert np.array_equal(y, (xi.astype(np.int64) @ w_int.T).astype(np.float64))


def test_gemv_one_hot_returns_a_column():
    """x = e_j gives y[n] = w[n][j] exactly (one nonzero product)."""
    rng = np.random.default_rng(3)
    N, K = 6, 128
    codes = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    scales = np.exp(rng.uniform(-7, -2, size=(N, K // 64))).astype(np.float16)
    q = O.pack_codes(codes, 4, SYM)
    w = O.dequant(q, scales, None, N, K, 4, 64, SYM)
    x = np.zeros((K, K), dtype=np.float16)
    x[np.arange(K), np.arange(K)] = 1.0
    y, _ = O.gemv_ref(q, scales, None, x, N, K, 4, 64, SYM)
    assert np.array_equal(y, w.T.astype(np.float64))


@pytest.mark.parametrize("fmt", ["int4g64", "int8g16", "asym"])
def test_gemv_matches_dense_float64_matmul(fmt):
    """y_ref equals x @ W^T over the dequantized matrix (float64 library matmul)
    up to float64 summation order, and bound equals |x| @ |W|^T."""
    rng = np.random.default_rng(21)
    M, N = 4, 11
    if fmt == "asym":
        K = 512
        codes, d, m, sc, mn, srec, zrec = _asym_problem(rng, N, K)
        q, s, z, bits, group, lay = O.pack_codes(codes, 4, ASYM), srec, zrec, 4, 32, ASYM
    else:
        bits, group = (4, 64) if fmt == "int4g64" else (8, 16)
        K = 256
        lo, hi = (-7, 7) if bits == 4 else (-127, 127)
        codes = rng.integers(lo, hi + 1, size=(N, K)).astype(np.int8)
        s = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=(N, K // group))).astype(np.float16)
        q, z, lay = O.pack_codes(codes, bits, SYM), None, SYM
    x = rng.standard_normal((M, K)).astype(np.float16)
    x[:, 5] = 300.0
    W = O.dequant(q, s, z, N, K, bits, group, lay).astype(np.float64)
    y, b = O.gemv_ref(q, s, z, x, N, K, bits, group, lay)
    xd = x.astype(np.float64)
    bb = np.abs(xd) @ np.abs(W).T
    assert np.allclose(b, bb, rtol=1e-14, atol=0)
    assert np.all(np.abs(y - xd @ W.T) <= 1e-13 * bb)


def test_gemv_threads_equal_single():
    rng = np.random.default_rng(4)
    N, K, M = 37, 256, 2
    codes = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    s = np.exp(rng.uniform(-7, -2, size=(N, K // 64))).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    q = O.pack_codes(codes, 4, SYM)
    y1, b1 = O.gemv_ref(q, s, None, x, N, K, 4, 64, SYM, threads=1)
    y4, b4 = O.gemv_ref(q, s, None, x, N, K, 4, 64, SYM, threads=4)
    assert np.array_equal(y1, y4) and np.array_equal(b1, b4)


def test_gemv_linear_in_scale():
    """Doubling every scale doubles y exactly (a power of two changes only exponents)."""
    rng = np.random.default_rng(8)
    N, K = 8, 256
    codes = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    s = np.exp(rng.uniform(-7, -2, size=(N, K // 64))).astype(np.float16)
    x = rng.standard_normal((1, K)).astype(np.float16)
    q = O.pack_codes(codes, 4, SYM)
    y1, _ = O.gemv_ref(q, s, None, x, N, K, 4, 64, SYM)
    y2, _ = O.gemv_ref(q, (s.astype(np.float32) * 2).astype(np.float16), None, x, N, K,
                       4, 64, SYM)
    assert np.array_equal(y2, 2 * y1)


# ------------------------------------------------------------------- check ---
def test_check_criterion():
    yr = np.array([1.0, 1.0, 0.0, 0.0, 5.0, 5.0], dtype=np.float64)
    bd = np.array([1000.0, 1000.0, 0.0, 0.0, 1.0, 1.0], dtype=np.float64)
    y = np.array([2.0, 2.0009765625, -0.0, 1e-30, np.nan, np.inf], dtype=np.float32)
    nbad, first, worst = O.check(y, yr, bd, rtol=1e-3)
    # |2-1| = 1 <= 1e-3*1000 passes; 1.0009765625 > 1 fails; -0 with bound 0
    # passes; 1e-30 with bound 0 fails; NaN and inf fail.
    assert nbad == 4 and first == 1 and worst == np.inf
    nbad, first, worst = O.check(y[:1], yr[:1], bd[:1])
    assert nbad == 0 and first == -1 and worst == pytest.approx(1e-3)


def test_check_catches_bf16_rounded_activations():
    """Rounding x to bfloat16 (8 significant bits) before the product can cost
    up to 2^-8 of a term, far above the 1e-3 tolerance: the check sees it.
    x = 1 + 2^-8 is exact in binary16; bfloat16 rounds it (ties to even) to 1."""
    K = 64
    x = np.zeros((1, K), dtype=np.float16)
    x[0, 0] = 1.0 + 2.0 ** -8
    codes = np.zeros((1, K), dtype=np.int8)
    codes[0, 0] = 7
    q = O.pack_codes(codes, 4, SYM)
    s = np.ones((1, 1), dtype=np.float16)
    y_ref, bound = O.gemv_ref(q, s, None, x, 1, K, 4, 64, SYM)
    assert y_ref[0, 0] == 7.0 + 7.0 * 2.0 ** -8
    exact = np.array([[7.0 + 7.0 * 2.0 ** -8]], dtype=np.float32)
    rounded = np.array([[7.0 * 1.0]], dtype=np.float32)
    assert O.check(exact, y_ref, bound)[0] == 0
    assert O.check(rounded, y_ref, bound)[0] == 1


# ------------------------------------------------------------------- FP8 ---
FP8 = O.LAYOUT_FP8_TENSOR


def f32_bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def test_fp8_literals(lit):
    for e in lit["fp8_e4m3"]:
        v = O.fp8_to_double(hx(e["byte"]))
        if e["value"] == "nan":
            assert np.isnan(v), e
        else:
            assert v == float(e["value"]) and np.signbit(v) == e["value"].startswith("-"), e


def test_fp8_every_code_matches_torch():
    """All 256 bytes against torch's float8_e4m3fn decoding (an independent
    implementation of the same OCP encoding)."""
    import torch
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = ref.to(torch.float64).numpy()
    got = np.array([O.fp8_to_double(b) for b in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got)) and nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_fp8_dequant_literal(lit):
    for c in lit["dequant_fp8"]:
        q = np.array([[hx(c["code"])] * 16], dtype=np.uint8)
        s = np.array([hx(c["scale_bits"])], dtype=np.uint32).view(np.float32)
        w = O.dequant(q, s, None, 1, 16, 8, 0, FP8)
        assert np.all(f32_bits(w) == hx(c["w_bits"])), c


def test_fp8_dequant_matches_the_page_recipe():
    """Quantize with the page's per-tensor recipe in torch (scale = max|W|/448,
    clamp, cast to float8_e4m3fn) and dequantize as it does (fp8 * scale in
    binary32): the oracle agrees bit for bit."""
    import torch
    g = torch.Generator().manual_seed(8)
    W = torch.randn(37, 96, generator=g) * torch.exp(2 * torch.randn(37, 1, generator=g))
    scale = W.abs().max() / 448.0
    q = (W / scale).clamp(-448, 448).to(torch.float8_e4m3fn)
    ref = (q.to(torch.float32) * scale).numpy()
    got = O.dequant(q.view(torch.uint8).numpy(), np.array([scale.item()], np.float32), None,
                    37, 96, 8, 0, FP8)
    assert np.array_equal(f32_bits(got), f32_bits(ref))


def test_fp8_gemv_matches_dense_float64():
    import torch
    rng = np.random.default_rng(81)
    N, K, M = 29, 160, 3
    codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38  # no NaN codes
    scale = np.array([0.0123], np.float32)
    wv = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    w = (wv * scale[0]).astype(np.float32)  # binary32 product, as the page dequantizes
    x = rng.standard_normal((M, K)).astype(np.float16)
    y, b = O.gemv_ref(codes, scale, None, x, N, K, 8, 0, FP8)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(b, np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T,
                       rtol=1e-12, atol=1e-12)


def test_fp8_rejects_groups_and_integer_views():
    q = np.zeros((2, 32), dtype=np.uint8)
    s = np.ones(1, np.float32)
    with pytest.raises(ValueError):
        O.dequant(q, s, None, 2, 32, 8, 16, FP8)
    with pytest.raises(ValueError):
        O.dequant(q, s, None, 2, 32, 4, 0, FP8)
    with pytest.raises(ValueError):
        O.unpack_codes(q, 2, 32, 8, FP8)


# ------------------------------------------------------- 5- and 6-bit codes ---
def test_hi_bit_literals(lit):
    K = 256
    for c in lit["asym_hi_bits"]:
        bits = c["bits"]
        codes = np.zeros((1, K), dtype=np.int8)
        codes[0, c["k"]] = c["value"]
        q = O.pack_codes(codes, bits, ASYM)
        assert q.size == K * bits // 8
        want = np.zeros_like(q)
        if c["nibble"] is not None:
            want[c["nibble"][0]] = hx(c["nibble"][1])
        want[K // 2 + c["plane"][0]] = hx(c["plane"][1])
        assert np.array_equal(q, want), c
        assert O.code_at(q, 1, K, bits, ASYM, 0, c["k"]) == c["value"], c


@pytest.mark.parametrize("bits", [5, 6])
def test_hi_bits_fill_the_plane_once(bits):
    """Each high bit of each of the 32 codes of a chunk has a bit of its own,
    and together they fill the chunk's 4 (5-bit) or 8 (6-bit) bytes."""
    K = 32 * 8
    seen = set()
    for k in range(32):
        for b in range(bits - 4):
            codes = np.zeros((1, K), dtype=np.int8)
            codes[0, 64 + k] = 1 << (4 + b)  # chunk 2
            q = O.pack_codes(codes, bits, ASYM)
            plane = np.unpackbits(q[K // 2:], bitorder="little")
            on = np.flatnonzero(plane)
            assert on.size == 1
            seen.add(int(on[0]))
    nb = 32 * (bits - 4)
    assert seen == set(range(2 * nb, 3 * nb))


@pytest.mark.parametrize("bits", [5, 6])
def test_hi_bits_round_trip_every_value(bits):
    rng = np.random.default_rng(bits)
    N, K = 5, 512
    codes = rng.integers(0, 1 << bits, size=(N, K)).astype(np.int8)
    codes[0, :32] = np.arange(32) % (1 << bits)
    codes[1, :64] = np.arange(64) % (1 << bits)
    q = O.pack_codes(codes, bits, ASYM)
    assert np.array_equal(O.unpack_codes(q, N, K, bits, ASYM), codes)
    with pytest.raises(ValueError):
        bad = codes.copy()
        bad[2, 7] = 1 << bits
        O.pack_codes(bad, bits, ASYM)


@pytest.mark.parametrize("bits", [5, 6])
def test_dequant_hi_bits_exact_rational(bits):
    """w = RN32((d*sc_j)*q - m*mn_j) with q up to 2^bits - 1, against Python's
    exact rationals."""
    rng = np.random.default_rng(40 + bits)
    N, K = 3, 512
    codes = rng.integers(0, 1 << bits, size=(N, K)).astype(np.int8)
    q = O.pack_codes(codes, bits, ASYM)
    B = K // 256
    d = rng.uniform(1e-4, 2e-3, size=(N, B)).astype(np.float16)
    m = rng.uniform(1e-4, 2e-3, size=(N, B)).astype(np.float16)
    sc = rng.integers(0, 64, size=(N, B, 8))
    mn = rng.integers(0, 64, size=(N, B, 8))
    srec = np.stack([[O.pack_record(half_bits(d[n, b]), sc[n, b]) for b in range(B)]
                     for n in range(N)])
    zrec = np.stack([[O.pack_record(half_bits(m[n, b]), mn[n, b]) for b in range(B)]
                     for n in range(N)])
    w = O.dequant(q, srec, zrec, N, K, bits, 32, ASYM)
    for n in range(N):
        for k in range(0, K, 7):
            b, j = k // 256, (k % 256) // 32
            exact = (Fraction(float(d[n, b])) * int(sc[n, b, j]) * int(codes[n, k])
                     - Fraction(float(m[n, b])) * int(mn[n, b, j]))
            # the exact value is a binary64 here; numpy rounds it once to binary32
            assert Fraction(float(exact)) == exact
            assert w[n, k] == np.float32(float(exact)), (n, k)


@pytest.mark.parametrize("bits", [5, 6])
def test_gemv_hi_bits_integer_exact(bits):
    """Power-of-two records and small integer x make every product and sum
    exact: the oracle equals an int64 matmul of the codes."""
    rng = np.random.default_rng(60 + bits)
    N, M, K = 7, 2, 256
    codes = rng.integers(0, 1 << bits, size=(N, K)).astype(np.int8)
    q = O.pack_codes(codes, bits, ASYM)
    one = O.pack_record(half_bits(1.0), np.ones(8, np.uint8))
    zero = O.pack_record(half_bits(0.0), np.zeros(8, np.uint8))
    srec = np.stack([[one]] * N)
    zrec = np.stack([[zero]] * N)
    x = rng.integers(-3, 4, size=(M, K)).astype(np.float16)
    y, _ = O.gemv_ref(q, srec, zrec, x, N, K, bits, 32, ASYM)
    ref = x.astype(np.int64) @ codes.astype(np.int64).T
    assert np.array_equal(y, ref.astype(np.float64))
