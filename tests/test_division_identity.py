"""The W4A8 activation quantiser replaces the per-element IEEE division a / s
by a reciprocal with one residual correction. This CPU test proves the two
agree bit for bit on every (a, s) the quantiser can meet (all fp16 a, all
s = amax / 127 for fp16 amax), so the codes stay those of the plain division
the oracle uses."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_corrected_reciprocal_equals_ieee_division_exhaustively():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "division_identity")
        subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                        os.path.join(HERE, "division_identity.c"), "-o", exe, "-lm"],
                       check=True, capture_output=True)
        out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    pairs, mismatches = map(int, out.stdout.split())
    assert pairs == sum(h + 1 for h in range(1, 0x7BFF + 1))   # every a in [0, amax]
    assert mismatches == 0 and out.returncode == 0
