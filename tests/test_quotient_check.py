"""The quantise-and-append kernel's division-free quotient (one correctly
rounded reciprocal per row plus Markstein's correction) against the IEEE
quotient, code by code: tests/quotient_check.c repeats the kernel's float
arithmetic in C and compares E4M3 codes for a sample of computed descales
amax/448 (every 97th bfloat16 amax, with every x of |x| <= amax) and seeded
descales in [2^-125, 2^125] with every finite bfloat16 x.  `quotient_check
full` runs every amax (about 2.4e9 pairs)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_quotient_codes_match_ieee_division(tmp_path):
    exe = str(tmp_path / "quotient_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "quotient_check.c"), "-lm"], check=True)
    res = subprocess.run([exe, "quick"], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert " 0 mismatches" in res.stdout
