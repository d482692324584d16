"""Pins of the oracle's variants: INT8 codes (Q_max = 127, the fallback the TACO page keeps for
hardware without FP8, section 5) and the rotation left out (ablation), against library rounding,
closed forms and quantizers written out independently here."""
import math

import numpy as np
import pytest
from scipy.linalg import hadamard

from tiecheck import E4M3_VALUES, INT8_VALUES, assert_codes_match, tie_cap
from workloads import TINY, bf16_bits_to_f32, f32_to_bf16_bits, make_shard, random_bf16_bits

F32_ULP = 2.0 ** -23
INT8, NOROT = 1, 2
FLAG_SETS = [0, INT8, NOROT, INT8 | NOROT]


def _qmax(flags):
    return 127.0 if flags & INT8 else 448.0


def _values(flags):
    return INT8_VALUES if flags & INT8 else E4M3_VALUES


def tight(got, ref, quot, flags):
    return assert_codes_match(got, ref, quot, max_frac=tie_cap(flags), rel=2.0 ** -40, abs_=1e-9,
                              int8=bool(flags & INT8))


# ------------------------------------------------------------------------------ INT8 codec

def test_int8_codec_matches_numpy(oracle):
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(-140, 140, 20000), np.arange(-130, 131) + 0.5,
                        np.arange(-130, 131).astype(np.float64), [0.0, -0.0, 1e-300, -1e-300]])
    enc = oracle.lib().tfp8_ref_int8_encode
    got = np.fromiter((enc(float(t)) for t in v), np.uint8, v.size)
    want = np.clip(np.round(v), -127, 127).astype(np.int8).view(np.uint8)  # numpy: half to even
    assert np.array_equal(got, want)
    dec = np.array([oracle.int8_decode(c) for c in range(256)])
    assert np.array_equal(dec, np.arange(256).astype(np.uint8).view(np.int8).astype(np.float64))


# ------------------------------------------------------------------------------ closed forms

@pytest.mark.parametrize("B", [4, 128, 256])
@pytest.mark.parametrize("flags", FLAG_SETS)
def test_one_hot_block_variants(oracle, B, flags):
    # v = c e_j: alpha = sqrt(T B)/|c| in every variant.  Rotated: every |y_i| = sqrt(T) and all
    # codes are +-Q with the signs of column j.  Not rotated: y = alpha c e_j, one code +-Q.
    T, c, j = 2.0, -0.75, 1
    v = np.zeros(B, np.float32)
    v[j] = c
    x = f32_to_bf16_bits(v)
    codes, alpha, scale = oracle.compress(x, B, T, flags=flags)
    Q = _qmax(flags)
    assert abs(alpha[0] - math.sqrt(T * B) / abs(c)) <= 0.5 * F32_ULP * alpha[0] * 1.0000001
    vals = _values(flags)[codes]
    if flags & NOROT:
        assert abs(scale[0] * Q - math.sqrt(T * B)) <= 2 * F32_ULP * math.sqrt(T * B)
        want = np.zeros(B)
        want[j] = -Q
    else:
        assert abs(scale[0] * Q - math.sqrt(T)) <= 2 * F32_ULP * math.sqrt(T)
        want = -Q * hadamard(B)[:, j]
    assert np.array_equal(vals, want)
    xh = oracle.decompress_f64(codes, alpha, scale, B, flags=flags)
    assert abs(xh[j] - c) <= 4 * F32_ULP * abs(c)
    assert np.all(xh[np.arange(B) != j] == 0.0)


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_constant_block_variants(oracle, flags):
    B, T, c = 64, 1.0, 0.5
    x = f32_to_bf16_bits(np.full(B, c, np.float32))
    codes, alpha, scale = oracle.compress(x, B, T, flags=flags)
    Q = _qmax(flags)
    vals = _values(flags)[codes]
    if flags & NOROT:  # every element is the block's peak
        assert np.all(vals == Q)
    else:              # all energy in coefficient 0
        assert vals[0] == Q and np.all(vals[1:] == 0)


# ------------------------------------------------------------------------------ independent quantizers

def _nearest_codes(t, flags):
    """Nearest code to each quotient by search (ties: even code / even integer)."""
    if flags & INT8:
        return np.clip(np.round(t), -127, 127).astype(np.int8).view(np.uint8)
    finite = np.array([c for c in range(256) if not np.isnan(E4M3_VALUES[c])])
    vals = E4M3_VALUES[finite]
    out = np.empty(t.size, np.uint8)
    for i, ti in enumerate(t):
        d = np.abs(vals - ti)
        cands = finite[d == d.min()]
        if cands.size > 1:
            same_sign = [c for c in cands if (c >> 7) == (1 if np.signbit(ti) else 0)]
            cands = np.array(same_sign or list(cands))
            even = [c for c in cands if c % 2 == 0]
            cands = np.array(even or list(cands))
        out[i] = cands[0]
    return out


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_codes_equal_plain_absmax_quantizer_of_the_rotated_block(oracle, flags):
    """Whatever alpha is, the codes are those of a plain per-block absmax quantizer applied to
    H x (or to x without the rotation): t = Q w / max|w|.  Computed here with scipy's Hadamard
    matrix and no alpha at all."""
    B = 64
    x = random_bf16_bits(40 * B, seed=21, scale=0.05)
    q, a, s, t = oracle.compress(x, B, 1.0, with_quot=True, flags=flags)
    v = bf16_bits_to_f32(x).astype(np.float64).reshape(-1, B)
    w = v if flags & NOROT else v @ hadamard(B).astype(np.float64)
    tq = _qmax(flags) * w / np.abs(w).max(axis=1, keepdims=True)
    want = _nearest_codes(tq.reshape(-1), flags)
    # The oracle divides by the fp32-rounded s, so quotients that are exact rounding midpoints
    # may round either way.  Without the rotation such exact ties are common (bfloat16 inputs
    # and E4M3 midpoints share a dyadic grid), hence the larger cap for that variant.
    assert_codes_match(q, want, tq.reshape(-1), max_frac=tie_cap(flags), rel=2.0 ** -22, abs_=1e-9,
                       int8=bool(flags & INT8))


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_error_bound_and_reconstruction_identity(oracle, flags):
    B = 128
    x = make_shard(TINY).reshape(-1)
    q, a, s, t = oracle.compress(x, B, 1.0, with_quot=True, flags=flags)
    vals = _values(flags)[q]
    if flags & INT8:
        assert np.all(np.abs(vals - t) <= 0.5 * (1 + 1e-12))
    assert np.all(np.abs(t) <= _qmax(flags) * (1 + 2.0 ** -23))
    xh = oracle.decompress_f64(q, a, s, B, flags=flags).reshape(-1, B)
    xv = bf16_bits_to_f32(x).astype(np.float64).reshape(-1, B)
    s64 = s.astype(np.float64)[:, None]
    lhs = np.linalg.norm(xh - xv, axis=1)
    rhs = np.linalg.norm(s64 * (vals.reshape(-1, B) - t.reshape(-1, B)), axis=1) / a
    assert np.all(np.abs(lhs - rhs) <= 1e-9 * np.maximum(rhs, 1e-300))


@pytest.mark.parametrize("flags", [INT8, INT8 | NOROT, NOROT])
def test_codes_invariant_to_target_variants(oracle, flags):
    x = make_shard(TINY).reshape(-1)
    q1, a1, s1, t1 = oracle.compress(x, 128, 1.0, with_quot=True, flags=flags)
    qT, aT, sT = oracle.compress(x, 128, 37.5, flags=flags)
    # a different T changes the fp32 roundings of alpha and s, which moves every quotient by a
    # few 2^-24 of itself: only near-ties within that may flip
    assert_codes_match(qT, q1, t1, max_frac=tie_cap(flags), rel=2.0 ** -21, abs_=1e-9,
                       int8=bool(flags & INT8))


# ------------------------------------------------------------------------------ reduce

def _negate(q, flags):
    if flags & INT8:
        return (-q.view(np.int8).astype(np.int16)).astype(np.int8).view(np.uint8)
    return q ^ 0x80


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_reduce_routes_and_identities_variants(oracle, flags):
    B, P = 128, 4
    xs = [random_bf16_bits(24 * B, seed=30 + p, scale=0.02) for p in range(P)]
    enc = [oracle.compress(x, B, 1.0, flags=flags) for x in xs]
    q = np.stack([e[0] for e in enc]); a = np.stack([e[1] for e in enc]); s = np.stack([e[2] for e in enc])
    qa, aa, sa, ta = oracle.reduce_fp8(q, a, s, B, 1.0, with_quot=True, flags=flags)
    qb, ab, sb, tb = oracle.reduce_fp8_rotated(q, a, s, B, 1.0, with_quot=True, flags=flags)
    tight(qb, qa, ta, flags)
    assert np.all(np.abs(sb.astype(np.float64) - sa) <= F32_ULP * sa)
    # P = 1 leaves the codes (up to the sign of zero) and s/alpha as they are
    q1, a1, s1, t1 = oracle.reduce_fp8(q[:1], a[:1], s[:1], B, 1.0, with_quot=True, flags=flags)
    norm = (lambda c: c) if flags & INT8 else (lambda c: np.where(c == 0x80, 0, c))
    assert np.array_equal(norm(q1), norm(q[0]))
    r_in = s[0].astype(np.float64) / a[0]
    assert np.all(np.abs(s1.astype(np.float64) / a1 - r_in) <= 4 * F32_ULP * r_in)
    # a contribution and its negation cancel
    q2 = np.stack([q[0], _negate(q[0], flags)])
    qo, ao, so = oracle.reduce_fp8(q2, np.repeat(a[:1], 2, 0), np.repeat(s[:1], 2, 0), B, 1.0,
                                   flags=flags)
    assert np.all(qo == 0) and np.all(ao == 1.0) and np.all(so == 0.0)


def test_flag_validation(oracle):
    x = np.zeros(256, np.uint16)
    with pytest.raises(ValueError, match="-6"):
        oracle.compress(x, 128, 1.0, flags=4)
