"""The quantisers' divide-free quotient gives the correctly rounded quotient's codes.

The per-token quantiser (e4m3fn) and the per-tensor one (e4m3fn and e5m2) form x / s
without a divide once amax >= 2^-80: q0 = x * r, e = fma(q0, s, -x), q = fma(-e, r, q0)
with r = fl32(1 / s). The oracle divides (fl32(x / s), correctly rounded). Over every
pair of finite bf16 values (x, amax >= 2^-80), |x| <= amax, `quotient_identity.c` finds
where the two quotients differ at all; this test requires every such quotient to lie
below the format's rounding floor (half its smallest subnormal: 2^-10 for e4m3fn, 2^-17
for e5m2) with the same sign on both sides, so that both encode to the same signed zero.
A statement about the arithmetic, checked exhaustively on the host; the GPU parity tests
check the kernels' codes against the oracle.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
N_PAIRS = 1029203968  # finite bf16 pairs (x, amax) with amax >= 2^-80 and |x| <= amax, both signs of x


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("needs gcc")
    exe = str(tmp_path_factory.mktemp("quotient") / "quotient_identity")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "quotient_identity.c"), "-lm"], check=True)
    return exe


@pytest.mark.parametrize("fmt,fmax,floor", [("e4m3fn", "448", 2.0 ** -10), ("e5m2", "57344", 2.0 ** -17)])
def test_divide_free_quotient_encodes_like_the_division(checker, fmt, fmax, floor):
    out = subprocess.run([checker, fmax], check=True, capture_output=True, text=True).stdout.split()
    pairs, differ, largest, sign_differ = int(out[0]), int(out[1]), float.fromhex(out[2]), int(out[3])
    assert pairs == N_PAIRS
    assert differ > 0  # the two forms do differ somewhere: the check looks where it must
    assert sign_differ == 0, fmt
    assert largest < floor, f"{fmt}: a differing quotient reaches {largest.hex()}"
