"""Comparison helpers shared by the oracle self-tests and the GPU parity tests.

Nothing here computes any part of the compression itself: these functions only decide
whether two results agree to the stated bar.

Code agreement ("identical except at most 1 ULP at rounding ties on <= 1e-4 of elements"):
a mismatch between a code and the reference code is admissible only when

  (i)  the two codes are adjacent E4M3 values (same sign, one step apart) or the +0/-0 pair;
  (ii) the reference's exact quotient t = y/s (the value the reference rounded) lies within
       ``rel * |mid| + abs_`` of the midpoint between the two code values (or of 0 for a
       +0/-0 pair), i.e. it is a rounding tie up to the other side's arithmetic error; and
  (iii) the number of mismatches is at most ``max_frac`` of the elements.
"""
from __future__ import annotations

import numpy as np

# Exact E4M3FN values, written from the format definition (bias 7, 3 mantissa bits,
# subnormal step 2^-9, 0x7F/0xFF NaN); independent of the oracle's decoder and checked
# against torch.float8_e4m3fn in the oracle tests.
_E4M3 = np.empty(256, np.float64)
for _c in range(256):
    _s = -1.0 if _c & 0x80 else 1.0
    _e = (_c >> 3) & 15
    _m = _c & 7
    if _e == 15 and _m == 7:
        _E4M3[_c] = np.nan
    elif _e == 0:
        _E4M3[_c] = _s * _m * 2.0 ** -9
    else:
        _E4M3[_c] = _s * (1 + _m / 8) * 2.0 ** (_e - 7)
E4M3_VALUES = _E4M3
# INT8 codes: two's complement bytes
INT8_VALUES = np.arange(256, dtype=np.int64).astype(np.uint8).view(np.int8).astype(np.float64)

# Window half-width: TIE_REL * |mid| + TIE_ABS code units.  The GPU forms each quotient from a
# float32 transform (a few roundings of 2^-24 relative to the block's peak, 448 code units) and a
# correctly rounded code multiplier, so its quotient errs by ~1e-4 code units at most in absolute
# terms and a few 2^-24 relative.  Measured over the GPU suite and 33 000 sweep cases with a
# window twice as wide (2^-20 |mid| + 2^-11), admitted mismatches sat at most 6.9e-5 code units
# from their midpoints and used at most 16% of that window; this one is half of it, which still
# leaves them at a third of it.
TIE_REL = 2.0 ** -21
TIE_ABS = 2.0 ** -12
MAX_TIE_FRAC = 1e-4

# Variant flags (the values the C ABI and the oracle use for their *_ex entry points).
FLAG_INT8, FLAG_NO_ROTATION = 1, 2


def tie_cap(flags: int) -> float:
    """Largest admissible fraction of tie mismatches.  1e-4 for the method.  With the rotation
    left out (an ablation variant) the codes are taken straight from ratios of bfloat16 inputs
    to the block peak, and those ratios land exactly on rounding midpoints far more often:
    ~2e-3 of the elements for E4M3 (both grids are coarse and dyadic), and for INT8 whenever
    the peak's significand divides evenly (a peak of 127 * 2^k makes every quotient dyadic).
    Such exact ties may round either way depending on the last bit of the fp32 scale, so the
    cap for those variants is 1e-2."""
    return 1e-2 if (flags & FLAG_NO_ROTATION) else MAX_TIE_FRAC


# Over a test session: how much of the tie window the admitted mismatches used (their distance
# from the midpoint over the window's half-width), and their largest distance in code units.
_TIE_STATS = {"admitted": 0, "max_window_frac": 0.0, "max_distance": 0.0, "over_half_window": 0,
              "max_distance_small_mid": 0.0, "max_rel_distance_large_mid": 0.0,
              "window_frac_hist": [0] * 5}
# buckets of the window fraction: [0, 1/64), [1/64, 1/16), [1/16, 1/4), [1/4, 1/2), [1/2, 1]
_HIST_EDGES = np.array([1 / 64, 1 / 16, 1 / 4, 1 / 2])


def tie_window_stats() -> dict:
    st = dict(_TIE_STATS)
    st["window_frac_hist"] = list(_TIE_STATS["window_frac_hist"])
    return st


def code_mismatches(got: np.ndarray, ref: np.ndarray, quot: np.ndarray, rel: float = TIE_REL,
                    abs_: float = TIE_ABS, int8: bool = False, return_bad: bool = False,
                    record: bool = True):
    """Return (n_mismatch, n_inadmissible, first_bad_index or -1), or with return_bad
    (n_mismatch, indices of the inadmissible mismatches).  With record=False the admitted
    mismatches are left out of the session's tie statistics."""
    got = np.asarray(got, np.uint8).reshape(-1)
    ref = np.asarray(ref, np.uint8).reshape(-1)
    quot = np.asarray(quot, np.float64).reshape(-1)
    bad = np.nonzero(got != ref)[0]
    if bad.size == 0:
        return (0, bad) if return_bad else (0, 0, -1)
    g, r, t = got[bad], ref[bad], quot[bad]
    if int8:
        gv, rv = INT8_VALUES[g], INT8_VALUES[r]
        zero_pair = np.zeros(bad.size, bool)
        adjacent = np.abs(gv - rv) == 1
        mid = 0.5 * (gv + rv)
    else:
        gs, rs = g >> 7, r >> 7
        gm, rm = (g & 0x7F).astype(np.int32), (r & 0x7F).astype(np.int32)
        zero_pair = (gm == 0) & (rm == 0)
        adjacent = ((gs == rs) & (np.abs(gm - rm) == 1)) | zero_pair
        mid = np.where(zero_pair, 0.0, 0.5 * (E4M3_VALUES[g] + E4M3_VALUES[r]))
    dist = np.abs(t - mid)
    window = rel * np.abs(mid) + abs_
    near = dist <= window
    ok = adjacent & near
    if ok.any() and record:
        frac = dist[ok] / window[ok]
        _TIE_STATS["admitted"] += int(ok.sum())
        _TIE_STATS["max_window_frac"] = max(_TIE_STATS["max_window_frac"], float(frac.max()))
        _TIE_STATS["max_distance"] = max(_TIE_STATS["max_distance"], float(dist[ok].max()))
        _TIE_STATS["over_half_window"] += int((frac > 0.5).sum())
        small = np.abs(mid[ok]) <= 8.0  # where the absolute term dominates the window
        if small.any():
            _TIE_STATS["max_distance_small_mid"] = max(_TIE_STATS["max_distance_small_mid"],
                                                       float(dist[ok][small].max()))
        if (~small).any():
            _TIE_STATS["max_rel_distance_large_mid"] = max(
                _TIE_STATS["max_rel_distance_large_mid"],
                float((dist[ok][~small] / np.abs(mid[ok][~small])).max()))
        for b in np.searchsorted(_HIST_EDGES, frac, side="right"):
            _TIE_STATS["window_frac_hist"][int(b)] += 1
    if return_bad:
        return int(bad.size), bad[~ok]
    nbad = int((~ok).sum())
    first = int(bad[np.argmax(~ok)]) if nbad else -1
    return int(bad.size), nbad, first


def assert_codes_match(got, ref, quot, max_frac: float = MAX_TIE_FRAC, rel: float = TIE_REL,
                       abs_: float = TIE_ABS, what: str = "codes", int8: bool = False):
    n = np.asarray(ref).size
    nmis, nbad, first = code_mismatches(got, ref, quot, rel, abs_, int8)
    assert nbad == 0, (f"{what}: {nbad} inadmissible code mismatches of {nmis}; first at {first}: "
                       f"got 0x{int(np.asarray(got).reshape(-1)[first]):02x} ref "
                       f"0x{int(np.asarray(ref).reshape(-1)[first]):02x} "
                       f"t={float(np.asarray(quot).reshape(-1)[first])!r}")
    assert nmis <= max_frac * max(n, 1), f"{what}: {nmis} tie mismatches of {n} exceed {max_frac}"
    return nmis


def rounding_interval(values: np.ndarray, int8: bool = False):
    """Lower and upper ends of the set of exact quotients that round to each code value (half the
    gaps to the neighbouring values, ends included; unbounded past the largest values, where
    rounding saturates)."""
    values = np.asarray(values, np.float64)
    table = INT8_VALUES[INT8_VALUES >= -127] if int8 else E4M3_VALUES[np.isfinite(E4M3_VALUES)]
    u = np.unique(table)  # sorted; +0 and -0 are one value
    k = np.searchsorted(u, values)
    assert np.all(u[np.minimum(k, u.size - 1)] == values), "not a code value"
    lo_gap = np.where(k > 0, 0.5 * (u[k] - u[np.maximum(k - 1, 0)]), np.inf)
    hi_gap = np.where(k < u.size - 1, 0.5 * (u[np.minimum(k + 1, u.size - 1)] - u[k]), np.inf)
    return values - lo_gap, values + hi_gap


# The reduce's sum.  Both sides form, per element, r = sum_p g_p dec(q_p) with g_p = s_p / alpha_p
# (the oracle as the float64 sum of the reconstructions in the original domain, the kernel in
# the rotated domain) with float64 roundings: the running sum's (P - 1 of at most 2^-53 of a
# partial sum), the oracle's reconstructions (two divisions) and transforms, and the kernel's
# factor g_p cut to 46 significant bits at least.  Mapped to the rotated domain, the oracle errs
# by at most about sqrt(B) (P + 1) 2^-52 Q sum_p g_p <= 2^-40 Q sum_p g_p (B <= 512, P <= 64; Q
# the code maximum, Q g_p the peak of contribution p) and the kernel by less, so the two differ
# by at most REDUCE_SUM_REL Q sum_p g_p per element, with a margin of about 4.  For blocks whose
# contributions do not cancel that is ~2^-22 code units or less, far inside the tie window; it
# grows only where the sum cancels far below the contributions' peaks.  The reduce's results are
# held to the tie rule first; only a code or scale that fails it may be admitted under this
# bound, and is counted apart from the ties.
REDUCE_SUM_REL = 2.0 ** -38


def reduce_sum_bound(alpha, scale, qmax: float) -> np.ndarray:
    """Per block: the bound D on |r_gpu - r_ref| from the contributions' scales alpha, scale
    [P, nb] (zero blocks contribute nothing)."""
    g = np.asarray(scale, np.float64) / np.asarray(alpha, np.float64)
    return REDUCE_SUM_REL * qmax * g.sum(axis=0)


def reduce_quotient_slack(D, ref_alpha, ref_scale, qmax: float):
    """Per block: (quotient slack w in code units, reference peak M = max|r_ref|).  The GPU's code
    i rounds Q r_gpu,i / M_gpu and the oracle's quotient is Q r_ref,i / M_ref; with both r and the
    peak within D, they differ by at most Q D (1 / M_ref + 1 / (M_ref - D)).  w is infinite where
    0 < D and M_ref <= 2 D: the block's sum is below the rounding noise of its contributions."""
    M = np.asarray(ref_scale, np.float64) * qmax / np.asarray(ref_alpha, np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        w = np.where(M > 2 * D, qmax * D * (1 / M + 1 / (M - D)), np.inf)
    return np.where(D == 0, 0.0, w), M  # D = 0: every contribution zero, the sum exactly zero


def assert_codes_within(got, quot, slack, int8: bool = False, what: str = "codes"):
    """Every code the rounding of some quotient within slack (per element, code units, plus the
    tie window's absolute term) of the reference's exact quotient."""
    g = np.asarray(got, np.uint8).reshape(-1)
    t = np.asarray(quot, np.float64).reshape(-1)
    w = np.asarray(slack, np.float64).reshape(-1) + TIE_ABS
    vals = INT8_VALUES[g] if int8 else E4M3_VALUES[g]
    lo, hi = rounding_interval(vals, int8)
    dist = np.maximum(np.maximum(lo - t, t - hi), 0.0)
    bad = np.nonzero(~(dist <= w))[0]
    assert bad.size == 0, (f"{what}: {bad.size} codes beyond the float64 sum's bound; first at "
                           f"{bad[0]}: got {vals[bad[0]]!r} t={t[bad[0]]!r} slack {w[bad[0]]!r}")


def assert_rel_close(got, ref, rel: float, floor: float = 0.0, what: str = "values"):
    got = np.asarray(got, np.float64).reshape(-1)
    ref = np.asarray(ref, np.float64).reshape(-1)
    err = np.abs(got - ref)
    lim = rel * np.abs(ref) + floor
    bad = np.nonzero(~(err <= lim))[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {ref.size} beyond rel {rel}; first at {bad[0]}: "
                           f"got {got[bad[0]]!r} ref {ref[bad[0]]!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(ref != 0, err / np.abs(ref), 0.0)
    return float(r.max()) if r.size else 0.0
