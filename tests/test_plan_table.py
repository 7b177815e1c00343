"""The matrix-core kernel's plan table, checked on the host (no GPU).

``tests/plan_fits_check.hip`` is compiled host-only with hipcc and run.  For
every format, M-tile count (1..4), group size and plan it asserts that the
host chooser's ``plan_fits`` accepts exactly the plans the kernel instance
accepts (``Mm<...>::FITS``), and that an independent restatement of the fit
conditions (LDS bytes of the copy rings and of the K-slice reduction, the
register cap, the copy layout) agrees with both.  A plan that does not fit is
never launched: the launch template returns an error for it.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def table(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("plan") / "plan_fits_check")
    cmd = [HIPCC, "--offload-host-only", "-std=c++17", "-O1",
           "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "gemm_rwkv_decode_amd", "csrc"),
           os.path.join(ROOT, "tests", "plan_fits_check.hip"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True)
    return r


def test_host_and_kernel_agree_on_every_plan(table):
    assert table.returncode == 0, table.stdout[-3000:]
    assert "mismatches=0" in table.stdout


def test_every_format_has_plans_at_every_m_tile(table):
    lines = [l.split() for l in table.stdout.splitlines() if l.startswith("fits ")]
    have = {(l[1], l[2]) for l in lines}
    for name in ("int4", "int8", "asym4", "asym5", "asym6", "fp8"):
        for mt in (1, 2, 3, 4):
            assert (name, f"mt={mt}") in have, (name, mt)
    # one M-tile with 4 or 8 staged x rows (M <= 4, M <= 8) as well
    xr = {(l[1], l[3]) for l in lines if l[2] == "mt=1"}
    for name in ("int4", "int8", "asym4", "asym5", "asym6", "fp8"):
        for r in ("xr=4", "xr=8", "xr=0"):
            assert (name, r) in xr, (name, r)


def test_lds_within_the_cu(table):
    for l in table.stdout.splitlines():
        if l.startswith("fits "):
            kv = dict(t.split("=") for t in l.split()[2:])
            assert int(kv["lds"]) <= 160 * 1024 and int(kv["red"]) <= 160 * 1024, l


def test_48_row_four_slice_plan_fits_past_48_rows(table):
    """The 48-row, four-K-slice arrangement (plan index 17) fits at four M-tiles
    for int4 group 64: its K-slice reduction takes 48 KiB, well inside the LDS
    (a byte count taken four times too large once excluded it)."""
    assert "fits int4 mt=4 xr=0 g=64 plan=17 " in table.stdout


def test_gpu_tests_cover_every_plan(table):
    """The GPU plan tests force every plan the table holds."""
    import re
    n = int(re.search(r"plans=(\d+)", table.stdout).group(1))
    src = open(os.path.join(ROOT, "tests", "test_gpu_parity.py")).read()
    hi = int(re.search(r"GEMM_PLANS = \[str\(i\) for i in range\(1, (\d+)\)\]", src).group(1))
    assert hi - 1 == n
