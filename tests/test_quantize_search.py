"""Host check of the cache write's rounding rule (no GPU).

The cache-write kernel rounds |x| / scale to E2M1 by a binary search of
exact integer comparisons on bf16 bit patterns: every decision boundary
mid * scale (mid in {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5}) is itself a bf16
value; a boundary whose tie goes down to the even code is compared as "> t",
i.e. ">= t + 1" on bit patterns, and every boundary is kept minus one so that
"|x| >= t" is the sign of the 16-bit difference (t - 1) - |x|.  A zero scale
is replaced by 2^100.  This test replays that search, written out here in
numpy, for every E4M3 scale and every finite bf16 magnitude, against the
plain midpoint rule (knowledge note "FP4 main KV": nearest E2M1 value, ties
to even, saturating at 6).
"""
import numpy as np

MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
STRICT = (1, 0, 1, 0, 1, 0, 1)  # ties at 0.25, 1.25, 2.5, 5 go down


def e4m3_value(code):
    e, m = code >> 3, code & 7
    return np.float32(m / 8 * 2.0**-6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))


def midpoint_rule(a, sv):
    t = [np.float32(x) * sv for x in MIDS]
    return ((a > t[0]).astype(int) + (a >= t[1]) + (a > t[2]) + (a >= t[3]) + (a > t[4]) + (a >= t[5]) +
            (a > t[6]))


def bit_search(a_bits, sv, scale_code):
    svb = sv if scale_code != 0 else np.float32(2.0**100)
    bnd = []
    for mid, strict in zip(MIDS, STRICT):
        p = int(np.array([np.float32(mid) * svb], np.float32).view(np.uint32)[0])
        assert p & 0xFFFF == 0, "boundary is a bf16 value"
        t1 = (p >> 16) + strict - 1
        assert 0 <= t1 < 0x8000
        bnd.append(t1)
    t0, t1, t2, t3, t4, t5, t6 = bnd

    def reach(thr):  # sign of the 16-bit difference thr - a
        return (((thr - a_bits) & 0xFFFF) >> 15) & 1

    g1 = reach(t3)
    g2 = reach(np.where(g1 == 1, t5, t1))
    g3 = reach(np.where(g2 == 1, np.where(g1 == 1, t6, t2), np.where(g1 == 1, t4, t0)))
    return 4 * g1 + 2 * g2 + g3


def test_bit_search_matches_midpoint_rule_for_every_scale_and_magnitude():
    a_bits = np.arange(0, 0x7F80, dtype=np.int64)  # every finite non-negative bf16
    a = (a_bits.astype(np.uint32) << 16).view(np.float32)
    for code in range(127):
        sv = e4m3_value(code)
        got = bit_search(a_bits, sv, code)
        if code == 0:
            # scale 0 only for groups with amax / 6 below half the smallest
            # subnormal: every element then rounds to magnitude 0
            sel = a <= np.float32(6 * 2.0**-10)
            assert (got[sel] == 0).all()
        else:
            assert np.array_equal(got, midpoint_rule(a, sv)), code
