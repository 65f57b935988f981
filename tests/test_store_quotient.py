"""The FP8 and NVFP4 stores divide by a per-thread scale through a correctly
rounded reciprocal and one FMA correction (csrc/store_row.h, Divisor /
quotient). This CPU test restates that arithmetic in C (tests/quotient_check.c,
C99 fmaf) and checks it against the IEEE quotient for every finite BF16 value
and a set of scales, including the bounds past which the store keeps the
uncorrected product."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_reciprocal_quotient_is_correctly_rounded(tmp_path):
    exe = tmp_path / "quotient_check"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe), os.path.join(HERE, "quotient_check.c"), "-lm"],
                   check=True)
    r = subprocess.run([str(exe), "400"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout
    exact, kept, bad = (int(w) for w in r.stdout.split()[1::2])
    assert bad == 0 and exact > 15_000_000 and kept > 1_000_000
