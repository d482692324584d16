"""The comparison rules themselves (tests/tiecheck.py), on hand-made cases: which code mismatches
count as rounding ties, the set of quotients that round to a code, and the reduce's float64 bound.
CPU only.  The mismatches made up here stay out of the session's tie statistics (record=False)."""
import numpy as np
import pytest

from tiecheck import (E4M3_VALUES, INT8_VALUES, REDUCE_SUM_REL, TIE_ABS, TIE_REL,
                      assert_codes_within, code_mismatches, reduce_quotient_slack,
                      reduce_sum_bound, rounding_interval)


def _inadmissible(got, ref, quot, int8=False):
    """Inadmissible mismatches among one-element code lists."""
    return code_mismatches(np.array(got, np.uint8), np.array(ref, np.uint8),
                           np.array(quot, np.float64), int8=int8, record=False)[1]


def test_e4m3_table_points():
    # points of the format (bias 7, three mantissa bits, subnormal step 2^-9, 0x7F NaN)
    assert E4M3_VALUES[0x38] == 1.0 and E4M3_VALUES[0x7E] == 448.0 and E4M3_VALUES[0xFE] == -448.0
    assert E4M3_VALUES[0x01] == 2.0 ** -9 and E4M3_VALUES[0x08] == 2.0 ** -6
    assert np.isnan(E4M3_VALUES[0x7F]) and np.isnan(E4M3_VALUES[0xFF])
    assert INT8_VALUES[0x7F] == 127 and INT8_VALUES[0x81] == -127 and INT8_VALUES[0xFF] == -1


def test_adjacent_codes_at_a_midpoint_are_a_tie():
    # 1.0 (0x38) and 1.125 (0x39): midpoint 1.0625, window TIE_REL * 1.0625 + TIE_ABS
    mid = 1.0625
    win = TIE_REL * mid + TIE_ABS
    for t in (mid, mid + 0.5 * win, mid - 0.9 * win):
        assert _inadmissible([0x39], [0x38], [t]) == 0, t
    # just outside the window, or a quotient that rounds plainly
    for t in (mid + 1.1 * win, 1.01):
        assert _inadmissible([0x39], [0x38], [t]) == 1, t


def test_non_adjacent_codes_are_never_a_tie():
    # 1.0 and 1.25 are two steps apart: no quotient makes that a rounding tie
    assert _inadmissible([0x3A], [0x38], [1.125]) == 1
    # opposite signs of the same magnitude are not adjacent either
    assert _inadmissible([0xB8], [0x38], [1.0]) == 1


def test_signed_zero_pair_near_zero():
    # +0 (0x00) against -0 (0x80): admissible when the quotient is within the window of 0
    assert _inadmissible([0x80], [0x00], [-0.5 * TIE_ABS]) == 0
    assert _inadmissible([0x80], [0x00], [-2 * TIE_ABS]) == 1


def test_int8_ties():
    # 5 and 6: midpoint 5.5
    assert _inadmissible([6], [5], [5.5], int8=True) == 0
    assert _inadmissible([6], [5], [5.4], int8=True) == 1
    assert _inadmissible([7], [5], [6.0], int8=True) == 1


def test_return_bad_lists_the_inadmissible_ones():
    got = np.array([0x38, 0x39, 0x3A, 0x38], np.uint8)
    ref = np.array([0x38, 0x38, 0x38, 0x38], np.uint8)
    t = np.array([1.0, 1.0625, 1.0625, 1.0])
    n, bad = code_mismatches(got, ref, t, return_bad=True, record=False)
    assert n == 2 and bad.tolist() == [2]


def test_rounding_interval():
    lo, hi = rounding_interval(np.array([1.0, 448.0, 0.0, -2.0 ** -9]))
    # 1.0: neighbours 0.9375 and 1.125; 448: no upper neighbour (saturation); 0: +-2^-10
    assert lo.tolist()[:3] == [0.96875, 432.0, -2.0 ** -10]
    assert hi.tolist()[0] == 1.0625 and np.isinf(hi[1]) and hi[2] == 2.0 ** -10
    assert lo[3] == -1.5 * 2.0 ** -9 and hi[3] == -0.5 * 2.0 ** -9
    lo, hi = rounding_interval(np.array([5.0, 127.0, -127.0]), int8=True)
    assert lo.tolist()[0] == 4.5 and hi.tolist()[0] == 5.5
    assert lo[1] == 126.5 and np.isinf(hi[1]) and np.isinf(lo[2]) and hi[2] == -126.5
    with pytest.raises(AssertionError):
        rounding_interval(np.array([1.01]))


def test_codes_within_a_slack():
    # code 1.125 (0x39) for an exact quotient of 1.0: its interval [1.0625, 1.1875] is 0.0625 away
    g, t = np.array([0x39], np.uint8), np.array([1.0])
    assert_codes_within(g, t, np.array([0.0625]))
    with pytest.raises(AssertionError):
        assert_codes_within(g, t, np.array([0.0625 - 2 * TIE_ABS]))


def test_reduce_sum_bound_and_slack():
    Q = 448.0
    alpha = np.array([[2.0, 4.0], [2.0, 1.0]])   # [P, nb]
    scale = np.array([[1.0, 0.0], [3.0, 0.0]])   # block 1: every contribution zero
    D = reduce_sum_bound(alpha, scale, Q)
    assert D[0] == REDUCE_SUM_REL * Q * (0.5 + 1.5) and D[1] == 0.0
    # reference peaks M = s Q / alpha: an ordinary block, one inside its noise, an exact zero sum
    D = np.array([1e-3, 1.0, 0.0])
    w, M = reduce_quotient_slack(D, np.array([1.0, 1.0, 1.0]), np.array([1.0, 1e-3, 0.0]), Q)
    assert M[0] == Q and w[0] == pytest.approx(Q * 1e-3 * (1 / Q + 1 / (Q - 1e-3)))
    assert np.isinf(w[1])   # M <= 2 D
    assert w[2] == 0.0      # D = 0: the sum is exactly zero, no slack


def test_reduce_sum_bound_holds(oracle):
    # The bound D between the kernel's and the oracle's float64 reduce sums, against the exact
    # sum.  For random reduces, including a contribution cancelled exactly by a later one with
    # smaller ones between them, and pairs that cancel to 2^-30 of their peaks, the oracle's sum
    # (r = t s' / alpha' from its quotients and scales) and a float64 sum in the kernel's order
    # (factors s_p / alpha_p cut to 46 significant bits, products exact, one rounding per
    # addition) each lie within D / 2 of the exact rotated-domain sum r = sum_p (s_p / alpha_p)
    # dec(q_p), computed with rationals from the stored float32 scales.
    from fractions import Fraction

    from workloads import f32_to_bf16_bits

    rng = np.random.default_rng(4242)
    for case in range(24):
        B = int(rng.choice([64, 128, 256]))
        P = int(rng.integers(2, 7))
        flags = int(rng.integers(0, 2))
        Q = 127.0 if flags else 448.0
        nb = 2
        xs = [rng.laplace(0, 1, nb * B) * 2.0 ** rng.uniform(-20, 20) for _ in range(P)]
        mode = case % 3
        if mode == 1:   # the last contribution cancels the first, huge one, exactly
            xs[0] = xs[0] * 2.0 ** 60
            xs[-1] = -xs[0]
        elif mode == 2:  # the second nearly cancels the first
            xs[1] = -xs[0] * (1 + 2.0 ** -30 * rng.standard_normal(nb * B))
        enc = [oracle.compress(f32_to_bf16_bits(v.astype(np.float32)), B, 1.0, flags=flags)
               for v in xs]
        q = np.stack([e[0] for e in enc])
        a = np.stack([e[1] for e in enc])
        s = np.stack([e[2] for e in enc])
        _, ra, rs, rt = oracle.reduce_fp8(q, a, s, B, 1.0, with_quot=True, flags=flags)
        table = INT8_VALUES if flags else E4M3_VALUES
        dec = table[q].reshape(P, nb, B)
        r_ref = rt.reshape(nb, B) * (rs.astype(np.float64) / ra)[:, None]
        g = s.astype(np.float64) / a.astype(np.float64)
        g = (g.view(np.int64) & ~np.int64(0x7F)).view(np.float64)  # 46 bits: the coarser cut
        r_k = np.zeros((nb, B))
        for p in range(P):
            r_k = r_k + g[p][:, None] * dec[p]
        D = reduce_sum_bound(a, s, Q)
        for k in range(nb):
            fr = [Fraction(float(s[p, k])) / Fraction(float(a[p, k])) for p in range(P)]
            exact = np.array([float(sum(fr[p] * Fraction(float(dec[p, k, i])) for p in range(P)))
                              for i in range(B)])
            assert np.abs(r_ref[k] - exact).max() <= D[k] / 2, (case, k, "oracle")
            assert np.abs(r_k[k] - exact).max() <= D[k] / 2, (case, k, "kernel order")
