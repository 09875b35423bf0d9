"""The block scale's divisions in the stochastic-rounding and 1D nearest-even encodes go through
reciprocals: RN(a / b) as q0 = RN(a * RN(1 / b)) followed by two residual corrections with fused
multiply-adds (the second, from a faithful quotient, gives the correctly rounded one: Markstein's
theorem), for a in [2^-90, 2^100] and b = 6 or ts in [2^-100, 2^100].  This checks that claim in
IEEE binary32 on the CPU, against division, on the sample described in the helper's header; the
GPU parity tests compare the kernels' scale bytes with the oracle's, which divides."""
import os
import subprocess

import pytest


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    src = os.path.join(os.path.dirname(__file__), "helpers", "recip_div_check.c")
    exe = str(tmp_path_factory.mktemp("recip") / "recip_div_check")
    # -ffp-contract=off: every product and sum rounds on its own, as in the library's sources
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-std=c11", src, "-o", exe, "-lm"], check=True)
    return exe


def test_corrected_quotients_equal_division(checker):
    # b = 6: every fp32 a in [2^-90, 2^-80) and [1, 2^10), and every 61st one up to 2^100
    runs = [("-90", "-80", "1", "0", "0"), ("0", "10", "1", "0", "0"), ("-90", "100", "61", "300", "400")]
    for args in runs:
        out = subprocess.run([checker, *args], capture_output=True, text=True, check=True).stdout.split()
        counts = [(int(out[i]), int(out[i + 1])) for i in range(0, 6, 2)]
        for n, bad in counts:
            assert bad == 0, (args, counts)
        assert counts[0][0] > 0
    assert counts[1][0] > 50_000_000 and counts[2][0] > 30_000_000
