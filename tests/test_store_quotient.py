"""The store kernels round x / s with one reciprocal per row and Markstein's correction step instead
of an IEEE division per value (for absmax scales s = fl32(absmax / 127) >= 2^-100).  This checks,
over every pair of a bf16 absmax and a bf16 value it bounds (about 1.05e9 pairs, compiled C on the
host), that the resulting codes are those of the IEEE division, i.e. of the oracle's definition."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_markstein_codes_equal_ieee_division_codes(tmp_path):
    exe = tmp_path / "quotient_check"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-pthread",
                    os.path.join(HERE, "quotient_check.c"), "-o", str(exe), "-lm"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    pairs, bad = (int(v) for v in r.stdout.split()[1::2])
    assert pairs > 1_000_000_000 and bad == 0 and r.returncode == 0
