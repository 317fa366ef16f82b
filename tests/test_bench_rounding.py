"""The bench's "% correctly rounded" report: fp64 -> bf16 round-to-nearest-
even, taken once (no double rounding through fp32), checked against values
whose bf16 rounding is fixed by the format (8 significant bits, fp32's
exponent range) and against a brute-force nearest search."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _bits(vals):
    return [int(b) for b in bench.bf16_rne_bits(np.array(vals, np.float64))]


def test_known_roundings():
    # ties go to the even mantissa; just above a tie goes up
    assert _bits([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-40]) == \
        [0x3F80, 0x3F80, 0x3F82, 0x3F81]
    assert _bits([-2.5, 0.0, -0.0, np.inf, -np.inf]) == [0xC020, 0x0000, 0x8000, 0x7F80, 0xFF80]
    # subnormal spacing 2^-133; half of it rounds to zero (even)
    assert _bits([3 * 2.0**-133, 2.0**-134, 1.5 * 2.0**-133]) == [0x0003, 0x0000, 0x0002]
    # a carry into the next binade
    assert _bits([2.0 - 2**-9]) == [0x4000]


def test_no_double_rounding():
    # x lies just above a bf16 tie, but rounding to fp32 first lands exactly on
    # the tie and then on the even neighbour (down): one rounding must go up
    x = 1.0 + 2**-8 + 2**-30
    assert float(np.float32(x)) == 1.0 + 2**-8
    assert _bits([x]) == [0x3F81]


def test_brute_force_nearest():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(4000) * np.exp2(rng.integers(-20, 20, 4000))
    got = bench.bf16_rne_bits(x)
    # every bf16 value of the same sign and nearby exponents, nearest (ties to even)
    all_bits = np.arange(0, 0x7F80, dtype=np.uint32)
    table = (all_bits << 16).view(np.float32).astype(np.float64)
    for xi, gi in zip(x[:400], got[:400]):
        d = np.abs(table - abs(xi))
        m = d.min()
        cand = all_bits[d == m]
        best = cand[0] if len(cand) == 1 else cand[(cand & 1) == 0][0]
        if xi < 0:
            best |= 0x8000
        assert gi == best, (xi, hex(gi), hex(best))


def test_share():
    ref = np.array([1.0, 1.0 + 2**-8, 0.5])
    got = bench.bf16_rne_bits(ref)
    assert bench.correctly_rounded_share(got, ref) == 1.0
    got2 = got.copy()
    got2[1] += 1  # one ulp off
    assert abs(bench.correctly_rounded_share(got2, ref) - 2 / 3) < 1e-12
