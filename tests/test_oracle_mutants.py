"""The pins catch plausible mistakes in the oracle.

Each case copies oracle/rq_oracle.cpp into a temporary directory, plants one
slip by replacing an exact source fragment, builds the copy with g++, points
the oracle module at that build and runs the pins of test_oracle_pins.py.  At
least one pin must fail for every slip.  Nothing here touches a GPU.
"""
import inspect
import json
import os
import shutil
import subprocess

import pytest

import oracle as O
from tests import test_oracle_pins as P

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle")

MUTANTS = {
    "nibbles_swapped": (
        "(k % 2 == 0) ? (byte & 0x0F) : (byte >> 4)",
        "(k % 2 == 0) ? (byte >> 4) : (byte & 0x0F)"),
    "sign_dropped": (
        "return (nibble >= 8) ? nibble - 16 : nibble;",
        "return nibble;"),
    "sign_threshold": (
        "return (nibble >= 8) ? nibble - 16 : nibble;",
        "return (nibble > 8) ? nibble - 16 : nibble;"),
    "int8_unsigned": (
        "return (int)(int8_t)qweight[(size_t)n * K + k];",
        "return (int)qweight[(size_t)n * K + k];"),
    "scale_group_index": (
        "*s = rqo_half_to_double(sc[(size_t)n * (K / group) + k / group]);",
        "*s = rqo_half_to_double(sc[(size_t)n * (K / group) + 0 * (k / group)]);"),
    "scale_row_stride": (
        "*s = rqo_half_to_double(sc[(size_t)n * (K / group) + k / group]);",
        "*s = rqo_half_to_double(sc[(size_t)0 * n + k / group]);"),
    "asym_subgroup_width": (
        "int j = (k % SUPERBLOCK) / SB_GROUP;",
        "int j = (k % SUPERBLOCK) / 64;"),
    "asym_shift_dropped": (
        "double exact = s * q - t;",
        "double exact = s * q;"),
    "asym_shift_sign": (
        "double exact = s * q - t;",
        "double exact = s * q + t;"),
    "asym_scale_for_shift": (
        "*t = rqo_half_to_double(m_bits) * (double)mn[j];",
        "*t = rqo_half_to_double(m_bits) * (double)sc[j];"),
    "record_field_width": (
        "for (int j = 0; j < 8; j++) sub[j] = (uint8_t)((field >> (6 * j)) & 0x3F);",
        "for (int j = 0; j < 8; j++) sub[j] = (uint8_t)((field >> (6 * j)) & 0x1F);"),
    "record_byte_offset": (
        "for (int i = 0; i < 6; i++) field |= (uint64_t)rec[2 + i] << (8 * i);",
        "for (int i = 0; i < 6; i++) field |= (uint64_t)rec[1 + i] << (8 * i);"),
    "half_exponent_bias": (
        "v = ldexp((double)(1024 + f), e - 25);",
        "v = ldexp((double)(1024 + f), e - 24);"),
    "half_subnormal_scale": (
        "v = ldexp((double)f, -24);",
        "v = ldexp((double)f, -25);"),
    "x_transposed": (
        "double p = xd[(size_t)m * K + k] * (double)wrow[k];",
        "double p = xd[(size_t)k * M + m] * (double)wrow[k];"),
    "y_transposed": (
        "y_ref[(size_t)m * N + n] = acc;",
        "y_ref[(size_t)n * M + m] = acc;"),
    "bound_signed": (
        "mag += fabs(p);",
        "mag += p;"),
    "float_accumulator": (
        "double acc = 0.0, mag = 0.0;",
        "float acc = 0.0f; double mag = 0.0;"),
    "weight_rounded_toward_zero": (
        "return (float)exact;",
        "float f = (float)exact;\n"
        "    return (fabs((double)f) > fabs(exact)) ? nextafterf(f, 0.0f) : f;"),
    "check_relative_to_y": (
        "ok = (err <= rtol * bound[i]);",
        "ok = (err <= rtol * fabs(y_ref[i]) + rtol);"),
    "fp8_exponent_bias": (
        "v = ldexp((double)(8 + f), e - 10);",
        "v = ldexp((double)(8 + f), e - 11);"),
    "fp8_subnormal_as_normal": (
        "v = ldexp((double)f, -9);",
        "v = ldexp((double)(8 + f), -10);"),
    "fp8_nan_as_number": (
        "if (e == 15 && f == 7) {",
        "if (e == 16) {"),
    "fp8_sign_dropped": (
        "int s = (b >> 7) & 1;",
        "int s = 0;"),
    "fp8_scale_ignored": (
        "*s = (double)((const float*)scales)[0];",
        "*s = 1.0;"),
    "hi5_shift": (
        "return base + (g == 0 ? i - 4 : i + 4);",
        "return base + (g == 0 ? i - 4 : i + 3);"),
    "hi_plane_offset": (
        "return (size_t)N * (K / 2) + (size_t)n * ((size_t)K * (bits - 4) / 8);",
        "return (size_t)n * ((size_t)K * (bits - 4) / 8);"),
    "hi6_bit_order": (
        "return base + b + s6[i % 2][g];",
        "return base + (1 - b) + s6[i % 2][g];"),
    "hi6_word": (
        "*word = i / 2;",
        "*word = i % 2;"),
    "hi_bits_shift": (
        "q |= (int)((v >> pos) & 1u) << (4 + b);",
        "q |= (int)((v >> pos) & 1u) << (3 + b);"),
    "check_zero_bound_lenient": (
        "ok = (yi == 0.0);",
        "ok = (fabs(yi) < 1e-20);"),
}

# pins that take the golden literals as their only argument
PINS = [f for name, f in sorted(vars(P).items())
        if name.startswith("test_") and callable(f)]


def _run_pins(lit):
    """Run every pin once; return the names of those that fail."""
    failed = []
    for f in PINS:
        params = inspect.signature(f).parameters
        calls = [dict()]
        marks = getattr(f, "pytestmark", [])
        for mk in marks:
            if mk.name == "parametrize":
                names = [s.strip() for s in mk.args[0].split(",")]
                calls = [dict(zip(names, v if isinstance(v, tuple) else (v,)))
                         for v in mk.args[1]]
        for kw in calls:
            if "lit" in params:
                kw = dict(kw, lit=lit)
            try:
                f(**kw)
            except Exception:  # an assertion or a rejected argument
                failed.append(f.__name__)
                break
    return failed


@pytest.fixture(scope="module")
def lit():
    with open(P.GOLDEN) as fh:
        return json.load(fh)


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


def test_unmutated_copy_passes_every_pin(lit, workdir):
    so = _build(workdir, "none", None)
    prev = O.swap_library(O.load_other(so))
    try:
        assert _run_pins(lit) == []
    finally:
        O.swap_library(prev)


def _build(workdir, name, mutation):
    d = workdir / name
    d.mkdir(exist_ok=True)
    src = open(os.path.join(SRC, "rq_oracle.cpp")).read()
    if mutation is not None:
        old, new = mutation
        assert src.count(old) == 1, f"fragment for {name} not found exactly once"
        src = src.replace(old, new)
    (d / "rq_oracle.cpp").write_text(src)
    shutil.copy(os.path.join(SRC, "rq_oracle.h"), d / "rq_oracle.h")
    so = str(d / f"librq_oracle_{name}.so")
    subprocess.run(["g++", "-std=c++17", "-O1", "-fPIC", "-shared",
                    "-ffp-contract=off", "-w", "-o", so, str(d / "rq_oracle.cpp")],
                   check=True)
    return so


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, lit, workdir):
    so = _build(workdir, name, MUTANTS[name])
    prev = O.swap_library(O.load_other(so))
    try:
        failed = _run_pins(lit)
    finally:
        O.swap_library(prev)
    assert failed, f"no pin detects the planted slip '{name}'"
