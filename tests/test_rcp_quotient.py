"""The NVFP4 block encoder replaces the 16 divisions |x| / b of a block by one
correctly rounded reciprocal y = 1/b and an FMA correction (Markstein, IBM J.
Res. Dev. 34(1), 1990).  The quantiser must stay bit-exact with the oracle's
float32 division, so this checks, in C on the host, that the E2M1 code never
changes: every positive finite bfloat16 value against every positive E4M3
scale under several per-tensor scales, plus random float32 values."""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_reciprocal_quotient_gives_the_division_codes(tmp_path):
    exe = str(tmp_path / "rcp_quotient_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, os.path.join(HERE, "c", "rcp_quotient_check.c"),
                    "-lm"], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=300).stdout
    m = re.match(r"cases (\d+) code_diffs (\d+) largest_missed_quotient (\S+)", out)
    assert m, out
    assert int(m.group(1)) > 60_000_000
    assert int(m.group(2)) == 0
    # the quotients the correction misses (subnormal |x|) are far below the
    # smallest E2M1 boundary, 0.25
    assert float.fromhex(m.group(3)) < 2.0 ** -50
