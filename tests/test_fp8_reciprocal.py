"""The quantising sender takes each value's quotient as |x| * (1 / scale)
plus one FMA correction instead of an IEEE division. This CPU test runs those
operations for every pair of a bf16 value and a bf16 block amax >= 2^-96 and
requires the same e4m3 code as the IEEE quotient in every case (the e4m3
format of "Enabling trillion-parameter models on AWS EFA", section
"Evaluation": block-scaled fp8 dispatch). Tests the kernel's arithmetic, not
the oracle; the two share nothing."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "fp8_reciprocal_check.c")


def test_reciprocal_quotient_gives_the_division_codes(tmp_path):
    exe = str(tmp_path / "fp8_reciprocal_check")
    r = subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, SRC, "-lm", "-lpthread"],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail("could not build the check: " + r.stderr[-2000:])
    out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    pairs, bad = (int(w) for w in out.stdout.split()[1::2])
    assert bad == 0
    # every pair: amax runs over the bf16 patterns 0x0F80 (2^-96) .. 0x7F7F
    # (the largest finite) and |x| over the patterns 0 .. amax's, so the
    # count is sum(h + 1 for h in that range) = 32640*32641/2 - 3968*3969/2
    assert pairs == 32640 * 32641 // 2 - 3968 * 3969 // 2 == 524_826_624
