"""Pins of the oracle's compress / decompress / reduce against closed forms, invariants,
brute force on tiny blocks and exact identities (no GPU).

Each closed form below is derived by hand from the method on the TACO summary page
(section 2.B.1 adaptive scale-Hadamard, section 2.B.2 dual scale) under the stated readings:
m2 = mean(v^2), alpha = sqrt(T/m2), y = H(alpha v)/sqrt(B) (Sylvester, natural order),
s = max|y|/448, q = E4M3FN(y/s).
"""
import math

import numpy as np
import pytest
from scipy.linalg import hadamard

from tiecheck import E4M3_VALUES, assert_codes_match, code_mismatches
from workloads import TINY, bf16_bits_to_f32, f32_to_bf16_bits, make_shard, random_bf16_bits

F32_ULP = 2.0 ** -23


def bf(values):
    """float values that are exactly bfloat16 -> bits."""
    f = np.asarray(values, np.float32)
    bits = f32_to_bf16_bits(f)
    assert np.array_equal(bf16_bits_to_f32(bits), f), "test value is not a bfloat16 number"
    return bits


def tight(got, ref, quot):
    # oracle-vs-oracle: only float64 rounding separates the two sides
    return assert_codes_match(got, ref, quot, max_frac=1e-4, rel=2.0 ** -40, abs_=1e-9)


# ------------------------------------------------------------------------------ closed forms

@pytest.mark.parametrize("B", [2, 4, 8, 128, 256])
@pytest.mark.parametrize("T", [1.0, 37.5])
@pytest.mark.parametrize("c", [2.0, -0.375, 0.0029296875])
def test_one_hot_block(oracle, B, T, c):
    # v = c e_j: m2 = c^2/B, alpha = sqrt(T B)/|c|, y = alpha c H[:, j]/sqrt(B) so every
    # |y_i| = sqrt(T): all codes are +-448 with the signs of column j times sign(c), and the
    # reconstruction puts c back at j and exact zeros elsewhere.
    j = B // 2 + 1 if B > 2 else 1
    v = np.zeros(B, np.float32)
    v[j] = c
    x = bf(v)
    cval = float(bf16_bits_to_f32(x)[j])
    codes, alpha, scale = oracle.compress(x, B, T)
    assert abs(alpha[0] - math.sqrt(T * B) / abs(cval)) <= 0.5 * F32_ULP * alpha[0] * 1.0000001
    assert abs(scale[0] * 448.0 - math.sqrt(T)) <= 2 * F32_ULP * math.sqrt(T)
    signs = hadamard(B)[:, j] * np.sign(cval)
    want = np.where(signs > 0, 0x7E, 0xFE).astype(np.uint8)
    assert np.array_equal(codes, want)
    xh = oracle.decompress_f64(codes, alpha, scale, B)
    assert abs(xh[j] - cval) <= 4 * F32_ULP * abs(cval)
    assert np.all(xh[np.arange(B) != j] == 0.0)


@pytest.mark.parametrize("B", [4, 8, 128, 256])
@pytest.mark.parametrize("c", [0.5, -3.0, 2.0 ** -100])
def test_constant_block(oracle, B, c):
    # v = c * 1: m2 = c^2, alpha = sqrt(T)/|c|, y = (sign(c) sqrt(T B), 0, ..., 0).
    T = 4.0
    x = bf(np.full(B, c, np.float32))
    codes, alpha, scale = oracle.compress(x, B, T)
    assert abs(alpha[0] - math.sqrt(T) / abs(c)) <= 0.5 * F32_ULP * alpha[0] * 1.0000001
    assert abs(scale[0] * 448.0 - math.sqrt(T * B)) <= 2 * F32_ULP * math.sqrt(T * B)
    want = np.zeros(B, np.uint8)
    want[0] = 0x7E if c > 0 else 0xFE
    assert np.array_equal(codes, want)
    xh = oracle.decompress_f64(codes, alpha, scale, B)
    assert np.all(np.abs(xh - c) <= 4 * F32_ULP * abs(c))


@pytest.mark.parametrize("B", [8, 128])
def test_hadamard_row_block(oracle, B):
    # v = c H[r, :]: m2 = c^2, y = alpha c H H[r,:]^T / sqrt(B) = sign(c) sqrt(T B) e_r.
    r, c, T = 5, -0.25, 1.0
    x = bf(c * hadamard(B)[r].astype(np.float32))
    codes, alpha, scale = oracle.compress(x, B, T)
    want = np.zeros(B, np.uint8)
    want[r] = 0xFE
    assert np.array_equal(codes, want)
    assert abs(alpha[0] - 4.0) <= 0.5 * F32_ULP * 4.0


def test_zero_block(oracle):
    B = 128
    x = np.zeros(3 * B, np.uint16)
    x[B + 7] = bf([0.125])[0]
    codes, alpha, scale = oracle.compress(x, B, 1.0)
    for k in (0, 2):
        assert alpha[k] == 1.0 and scale[k] == 0.0
        assert np.all(codes[k * B:(k + 1) * B] == 0)
    assert scale[1] > 0
    out16 = oracle.decompress(codes, alpha, scale, B, np.uint16)
    out32 = oracle.decompress(codes, alpha, scale, B, np.float32)
    for k in (0, 2):
        assert np.all(out16[k * B:(k + 1) * B] == 0)  # +0 bits
        assert np.all(out32[k * B:(k + 1) * B].view(np.uint32) == 0)


def test_negative_zero_only_block_is_zero(oracle):
    B = 8
    x = np.full(B, 0x8000, np.uint16)  # -0.0
    codes, alpha, scale = oracle.compress(x, B, 1.0)
    assert alpha[0] == 1.0 and scale[0] == 0.0 and np.all(codes == 0)


def test_subnormal_block_clamps_alpha(oracle):
    # absmax 2^-127 (bfloat16 subnormal): sqrt(1/m2) >= 2^127 exceeds the clamp 2^126.
    B = 128
    rng = np.random.default_rng(3)
    k = rng.integers(-(2 ** 6), 2 ** 6, B)
    k[0] = 2 ** 6
    v = k.astype(np.float64) * 2.0 ** -133
    x = f32_to_bf16_bits(v.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f32(x).astype(np.float64), v)
    codes, alpha, scale, quot = oracle.compress(x, B, 1.0, with_quot=True)
    assert alpha[0] == np.float32(2.0 ** 126)
    assert np.any((codes == 0x7E) | (codes == 0xFE))
    # the reconstruction error identity holds there too
    xh = oracle.decompress_f64(codes, alpha, scale, B)
    y = scale.astype(np.float64)[0] * quot
    lhs = np.linalg.norm(xh - v)
    rhs = np.linalg.norm(scale.astype(np.float64)[0] * E4M3_VALUES[codes] - y) / float(alpha[0])
    assert abs(lhs - rhs) <= 1e-9 * rhs


# ------------------------------------------------------------------------------ invariants

def _tiny_shard(oracle):
    return make_shard(TINY).reshape(-1)


def test_codes_invariant_to_target(oracle):
    x = _tiny_shard(oracle)
    B = 128
    q1, a1, s1, t1 = oracle.compress(x, B, 1.0, with_quot=True)
    for T in (37.5, 2.0 ** -10, 2.0 ** 20):
        qT, aT, sT = oracle.compress(x, B, T)
        tight(qT, q1, t1)
        nz = s1 > 0
        r1 = s1[nz].astype(np.float64) / a1[nz]
        rT = sT[nz].astype(np.float64) / aT[nz]
        assert np.all(np.abs(rT - r1) <= 4 * F32_ULP * r1)


def test_power_of_two_scaling(oracle):
    x = random_bf16_bits(64 * 128, seed=4, scale=0.01)
    B = 128
    q, a, s = oracle.compress(x, B, 1.0)
    for k in (-20, 13):
        xs = f32_to_bf16_bits(bf16_bits_to_f32(x) * np.float32(2.0 ** k))
        assert np.array_equal(bf16_bits_to_f32(xs), bf16_bits_to_f32(x) * np.float32(2.0 ** k))
        qk, ak, sk = oracle.compress(xs, B, 1.0)
        assert np.array_equal(qk, q)
        assert np.array_equal(sk, s)
        assert np.array_equal(ak, (a.astype(np.float64) * 2.0 ** -k).astype(np.float32))


def test_negation_flips_signs(oracle):
    x = _tiny_shard(oracle)
    B = 128
    q, a, s, t = oracle.compress(x, B, 1.0, with_quot=True)
    qn, an, sn = oracle.compress(x ^ np.uint16(0x8000), B, 1.0)
    assert np.array_equal(an, a) and np.array_equal(sn, s)
    exact_zero = t == 0.0
    assert np.array_equal(qn[~exact_zero], q[~exact_zero] ^ 0x80)
    assert np.all(qn[exact_zero] == 0) and np.all(q[exact_zero] == 0)


def test_block_permutation_equivariance(oracle):
    B = 64
    x = random_bf16_bits(32 * B, seed=5)
    perm = np.random.default_rng(6).permutation(32)
    xp = x.reshape(32, B)[perm].reshape(-1)
    q, a, s = oracle.compress(x, B, 1.0)
    qp, ap, sp = oracle.compress(xp, B, 1.0)
    assert np.array_equal(qp.reshape(32, B), q.reshape(32, B)[perm])
    assert np.array_equal(ap, a[perm]) and np.array_equal(sp, s[perm])


def test_every_nonzero_block_reaches_qmax_and_no_nan(oracle):
    x = _tiny_shard(oracle)
    B = 128
    q, a, s = oracle.compress(x, B, 1.0)
    qb = q.reshape(-1, B)
    has_max = np.any((qb == 0x7E) | (qb == 0xFE), axis=1)
    assert np.array_equal(has_max, s > 0)
    assert not np.any((q == 0x7F) | (q == 0xFF))
    assert np.sum(s == 0) == 4  # the four all-zero blocks of this input


# ------------------------------------------------------------------------------ brute force

_GRID = np.array([0.0, 2.0 ** -133, 2.0 ** -127, 2.0 ** -20, 0.5, 1.0, 1.5, 448.0, 3.0e38])


def _brute_block(v64, T):
    """Explicit-matrix route with exhaustive nearest-code search (independent of the oracle's
    FWHT and encoder)."""
    B = v64.size
    finite = np.array([c for c in range(256) if not np.isnan(E4M3_VALUES[c])])
    if np.max(np.abs(v64)) == 0:
        return np.zeros(B, np.uint8), np.float32(1), np.float32(0), np.zeros(B)
    m2 = np.mean(v64 * v64)
    T = float(np.float32(T))  # the target crosses the boundary as an fp32
    a = np.float32(min(max(math.sqrt(T / m2), 2.0 ** -126), 2.0 ** 126))
    y = (hadamard(B).astype(np.float64) @ (float(a) * v64)) / math.sqrt(B)
    s = np.float32(np.max(np.abs(y)) / 448.0)
    t = y / float(s)
    d = np.abs(E4M3_VALUES[finite][None, :] - t[:, None])
    best = d.min(axis=1, keepdims=True)
    cand = np.where(d == best, finite[None, :], 999)
    codes = np.empty(B, np.uint8)
    for i in range(B):
        cs = sorted(c for c in cand[i] if c != 999)
        if len(cs) == 1:
            codes[i] = cs[0]
        else:  # equidistant pair: even mantissa; sign of the quotient on a +-0 pair
            cs = [c for c in cs if (c & 0x80) == (0x80 if np.signbit(t[i]) else 0)] or cs
            codes[i] = [c for c in cs if c % 2 == 0][0] if len(cs) > 1 else cs[0]
    return codes, a, s, t


@pytest.mark.parametrize("B", [2, 4, 8])
def test_tiny_blocks_brute_force(oracle, B):
    rng = np.random.default_rng(B)
    grid = np.concatenate([_GRID, -_GRID[1:]])
    if B == 2:
        blocks = np.array([[a, b] for a in grid for b in grid])
    else:
        blocks = grid[rng.integers(0, grid.size, (1500, B))]
        # mixtures of magnitudes across the whole range are the interesting cases
    v32 = blocks.astype(np.float32)
    x = f32_to_bf16_bits(v32.reshape(-1))
    v64 = bf16_bits_to_f32(x).astype(np.float64).reshape(-1, B)
    for T in (1.0, 0.01):
        q, a, s, t = oracle.compress(x, B, T, with_quot=True)
        for k in range(v64.shape[0]):
            cq, ca, cs, ct = _brute_block(v64[k], T)
            assert a[k] == ca, (k, v64[k], a[k], ca)
            assert abs(float(s[k]) - float(cs)) <= F32_ULP * float(cs), (k, s[k], cs)
            assert code_mismatches(q[k * B:(k + 1) * B], cq, ct, 2.0 ** -40, 1e-12)[1] == 0, (
                k, v64[k], q[k * B:(k + 1) * B], cq)


# ------------------------------------------------------------------------------ error identities

def _half_step(t):
    a = np.abs(t)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.where(a < 2.0 ** -6, 2.0 ** -10, 2.0 ** (e - 4))


def test_quantization_error_bound(oracle):
    x = _tiny_shard(oracle)
    B = 128
    q, a, s, t = oracle.compress(x, B, 1.0, with_quot=True)
    err = np.abs(E4M3_VALUES[q] - t)
    assert np.all(err <= _half_step(t) * (1 + 1e-12))
    # s is max|y|/448 rounded to fp32, so |y/s| may exceed 448 by that one rounding
    assert np.all(np.abs(t) <= 448.0 * (1 + 2.0 ** -23))
    assert np.max(np.abs(t)) > 448.0 * (1 - 2.0 ** -23)


def test_reconstruction_error_identity(oracle):
    # ||xh - x||_2 = ||s dec(q) - y||_2 / alpha per block (the rotation is orthogonal)
    x = _tiny_shard(oracle)
    B = 128
    q, a, s, t = oracle.compress(x, B, 1.0, with_quot=True)
    xh = oracle.decompress_f64(q, a, s, B).reshape(-1, B)
    xv = bf16_bits_to_f32(x).astype(np.float64).reshape(-1, B)
    s64 = s.astype(np.float64)[:, None]
    lhs = np.linalg.norm(xh - xv, axis=1)
    rhs = np.linalg.norm(s64 * E4M3_VALUES[q].reshape(-1, B) - s64 * t.reshape(-1, B), axis=1)
    rhs = rhs / a.astype(np.float64)
    assert np.all(np.abs(lhs - rhs) <= 1e-9 * np.maximum(rhs, 1e-300))
    # and the round trip is close: relative L2 error per nonzero block bounded by E4M3's
    # half-step relative precision (2^-4) at worst
    nz = s > 0
    rel = lhs[nz] / np.linalg.norm(xv[nz], axis=1)
    assert rel.max() < 2.0 ** -4


@pytest.mark.parametrize("B", [2, 16, 128, 256])
def test_exact_inverse_without_rounding(oracle, B):
    x = random_bf16_bits(40 * B, seed=B, scale=0.3)
    x[:B] = 0
    t, a, s = oracle.compress_unrounded(x, B, 1.0)
    back = oracle.decompress_unrounded(t, a, s, B).reshape(-1, B)
    xv = bf16_bits_to_f32(x).astype(np.float64).reshape(-1, B)
    scale = np.maximum(np.abs(xv).max(axis=1, keepdims=True), 1e-300)
    assert np.all(np.abs(back - xv) <= 1e-14 * scale)


def test_decompress_bf16_rounds_once(oracle):
    # The bfloat16 output is the exact reconstruction rounded once.  With alpha = float32(256/257),
    # s = 1 and the code of 1.0 (no rotation: x = s dec(q) / alpha), the reconstruction 1/alpha
    # lies 2.3e-10 above 1 + 2^-8, the midpoint between the bfloat16 neighbours 1 and 1 + 2^-7.
    # Rounded once it is 1 + 2^-7; rounded to float32 first it would become the midpoint itself
    # and then round to even, 1.
    from fractions import Fraction

    from tiecheck import FLAG_NO_ROTATION

    B = 64
    alpha = np.float32(256 / 257)
    eps = 1 / Fraction(float(alpha)) - Fraction(257, 256)
    assert 0 < eps < Fraction(1, 2 ** 25)  # the case is the one described
    one = int(np.flatnonzero(E4M3_VALUES == 1.0)[0])
    q = np.full(2 * B, one, np.uint8)
    q[B:] |= 0x80  # block 1: the code of -1.0
    a, s = np.full(2, alpha, np.float32), np.ones(2, np.float32)
    out16 = oracle.decompress(q, a, s, B, np.uint16, flags=FLAG_NO_ROTATION)
    assert np.all(out16[:B] == 0x3F81) and np.all(out16[B:] == 0xBF81)
    out32 = oracle.decompress(q, a, s, B, np.float32, flags=FLAG_NO_ROTATION)
    assert np.all(out32[:B] == np.float32(1 + 2.0 ** -8))


def test_decompress_dtypes_agree_with_f64(oracle):
    x = _tiny_shard(oracle)
    B = 128
    q, a, s = oracle.compress(x, B, 1.0)
    r64 = oracle.decompress_f64(q, a, s, B)
    assert np.array_equal(oracle.decompress(q, a, s, B, np.float32), r64.astype(np.float32))
    import torch
    via_torch = torch.from_numpy(r64).to(torch.bfloat16)  # may double round via float32
    ours = oracle.decompress(q, a, s, B, np.uint16)
    diff = ours != via_torch.view(torch.int16).numpy().view(np.uint16)
    assert diff.mean() < 1e-4


# ------------------------------------------------------------------------------ reduce

def _shards(oracle, P, B=128, nblk=48, seed=10):
    xs = [random_bf16_bits(nblk * B, seed=seed + p, scale=0.02) for p in range(P)]
    out = [oracle.compress(x, B, 1.0) for x in xs]
    return (np.stack([o[0] for o in out]), np.stack([o[1] for o in out]),
            np.stack([o[2] for o in out]))


def test_reduce_single_contribution_is_identity(oracle):
    q, a, s = _shards(oracle, 1)
    qo, ao, so, t = oracle.reduce_fp8(q, a, s, 128, 1.0, with_quot=True)
    tight(qo, q[0], t)
    r_in = s[0].astype(np.float64) / a[0]
    r_out = so.astype(np.float64) / ao
    assert np.all(np.abs(r_out - r_in) <= 4 * F32_ULP * r_in)


@pytest.mark.parametrize("P", [2, 3, 8])
def test_reduce_identical_copies(oracle, P):
    q, a, s = _shards(oracle, 1)
    qP, aP, sP = np.repeat(q, P, 0), np.repeat(a, P, 0), np.repeat(s, P, 0)
    qo, ao, so, t = oracle.reduce_fp8(qP, aP, sP, 128, 1.0, with_quot=True)
    tight(qo, q[0], t)
    r_in = P * s[0].astype(np.float64) / a[0]
    r_out = so.astype(np.float64) / ao
    assert np.all(np.abs(r_out - r_in) <= 4 * F32_ULP * r_in)


def test_reduce_contribution_and_its_negation_cancel(oracle):
    q, a, s = _shards(oracle, 1)
    q2 = np.stack([q[0], q[0] ^ 0x80])
    qo, ao, so = oracle.reduce_fp8(q2, np.repeat(a, 2, 0), np.repeat(s, 2, 0), 128, 1.0)
    assert np.all(ao == 1.0) and np.all(so == 0.0) and np.all(qo == 0)
    qo, ao, so = oracle.reduce_fp8_rotated(q2, np.repeat(a, 2, 0), np.repeat(s, 2, 0), 128, 1.0)
    assert np.all(ao == 1.0) and np.all(so == 0.0) and np.all(qo == 0)


@pytest.mark.parametrize("route", ["definition", "rotated"])
def test_reduce_sums_in_contribution_order(oracle, route):
    # The sum runs over p = 0, 1, ..., P - 1.  With a large contribution x first, its exact
    # negation second and a contribution y 2^40 times smaller last, x + (-x) is exactly zero
    # before y is added, so the reduce of [x, -x, y] is the reduce of [y] alone, bit for bit.
    # In any other order y would meet x or -x first and lose its low bits to the rounding.
    B = 128
    q, a, s = _shards(oracle, 2, B=B, nblk=24)
    big = s[0] * np.float32(2.0 ** 20)
    small = s[1] * np.float32(2.0 ** -20)
    q3 = np.stack([q[0], q[0] ^ 0x80, q[1]])
    a3 = np.stack([a[0], a[0], a[1]])
    s3 = np.stack([big, big, small])
    f = oracle.reduce_fp8 if route == "definition" else oracle.reduce_fp8_rotated
    q1, a1, s1, t1 = f(q3[2:], a3[2:], s3[2:], B, 1.0, with_quot=True)
    qr, ar, sr, tr = f(q3, a3, s3, B, 1.0, with_quot=True)
    assert np.array_equal(qr, q1) and np.array_equal(tr, t1)
    assert np.array_equal(ar, a1) and np.array_equal(sr, s1)
    # the pin has teeth: summed from the last contribution down, the result differs
    qb, ab, sb, tb = f(q3[::-1].copy(), a3[::-1].copy(), s3[::-1].copy(), B, 1.0, with_quot=True)
    assert not (np.array_equal(tb, t1) and np.array_equal(ab, a1))


def test_reduce_rotated_route_scales_by_the_stored_alpha(oracle):
    # With one contribution the rotated route's sum is r = (s / alpha) dec(q), formed here in
    # float64 as the definition states it.  Requantising r uses the stored (float32) prescale:
    # y = alpha' r, s' = max|y| / Q rounded to float32, and the quotients y / s'.  So the
    # quotients must be alpha' r / s' and s' must be float32(alpha' max|r| / Q) exactly, with
    # alpha' = float32(sqrt(T / mean(r^2))) to within its last bit (the sum of squares may round
    # in another order).  A route that scaled by the unrounded alpha would miss both.
    B, Q = 128, 448.0
    q, a, s = _shards(oracle, 1, B=B, nblk=48)
    qo, ao, so, t = oracle.reduce_fp8_rotated(q, a, s, B, 1.0, with_quot=True)
    r = (s[0].astype(np.float64) / a[0].astype(np.float64))[:, None] * \
        E4M3_VALUES[q[0]].reshape(-1, B)
    a64 = ao.astype(np.float64)
    assert np.all(s[0] > 0)
    assert np.array_equal(so, (a64 * np.abs(r).max(axis=1) / Q).astype(np.float32))
    assert np.array_equal(t.reshape(-1, B), a64[:, None] * r / so.astype(np.float64)[:, None])
    alpha_def = np.sqrt(1.0 / np.mean(r * r, axis=1)).astype(np.float32)
    assert np.all(np.abs(ao.view(np.int32) - alpha_def.view(np.int32)) <= 1)


def _subnormal_blocks(rng, nb, B):
    # bfloat16-subnormal blocks k * 2^-133, |k| <= 64, each with a peak of 2^-127: their
    # sqrt(1/m2) passes 2^126, so compress clamps alpha there
    k = rng.integers(-(2 ** 6), 2 ** 6, (nb, B))
    k[:, 0] = 2 ** 6
    return f32_to_bf16_bits((k.astype(np.float64) * 2.0 ** -133).astype(np.float32).reshape(-1))


@pytest.mark.parametrize("route", ["definition", "rotated"])
def test_reduce_clamps_alpha_of_tiny_sums(oracle, route):
    # two contributions compressed from bfloat16-subnormal blocks: their sum's mean square is
    # still below 2^-252, so the reduce's alpha is clamped at 2^126 too, in either route
    B, nb = 128, 8
    rng = np.random.default_rng(31)
    enc = [oracle.compress(_subnormal_blocks(rng, nb, B), B, 1.0) for _ in range(2)]
    q, a, s = (np.stack([e[i] for e in enc]) for i in range(3))
    assert np.all(a == np.float32(2.0 ** 126))
    f = oracle.reduce_fp8 if route == "definition" else oracle.reduce_fp8_rotated
    qo, ao, so = f(q, a, s, B, 1.0)
    z = sum(oracle.decompress_f64(q[p], a[p], s[p], B) for p in range(2)).reshape(nb, B)
    assert np.all(np.sqrt(1.0 / np.mean(z * z, axis=1)) > 2.0 ** 126)
    assert np.all(ao == np.float32(2.0 ** 126)) and np.all(so > 0)


@pytest.mark.parametrize("P,B", [(4, 256), (8, 128), (3, 64)])
def test_reduce_two_routes_agree(oracle, P, B):
    q, a, s = _shards(oracle, P, B=B, nblk=40)
    q[:, :B] = 0            # block 0 zero in every contribution
    s[:, 0] = 0.0
    a[:, 0] = 1.0
    s[1, 3] = 0.0           # block 3 zero in one contribution only
    a[1, 3] = 1.0
    q[1, 3 * B:4 * B] = 0
    qa, aa, sa, ta = oracle.reduce_fp8(q, a, s, B, 1.0, with_quot=True)
    qb, ab, sb, tb = oracle.reduce_fp8_rotated(q, a, s, B, 1.0, with_quot=True)
    tight(qb, qa, ta)
    assert np.all(np.abs(ab.astype(np.float64) - aa) <= F32_ULP * aa)
    assert np.all(np.abs(sb.astype(np.float64) - sa) <= F32_ULP * np.abs(sa))
    assert aa[0] == 1.0 and sa[0] == 0.0


@pytest.mark.parametrize("route", ["definition", "rotated"])
def test_reduce_target_scaling(oracle, route):
    # alpha = clamp(sqrt(T / m2)) with m2 the sum's second moment, which does not depend on T:
    # a target 4 times larger doubles alpha exactly (sqrt(4 x) = 2 sqrt(x) in binary), hence y and
    # s, and leaves every quotient and code as it was (no block here reaches the clamp)
    P, B = 4, 128
    q, a, s = _shards(oracle, P, B=B, nblk=24)
    f = oracle.reduce_fp8 if route == "definition" else oracle.reduce_fp8_rotated
    for T in (1.0, 2.0 ** -6, 37.5):
        q1, a1, s1, t1 = f(q, a, s, B, T, with_quot=True)
        q4, a4, s4, t4 = f(q, a, s, B, 4 * T, with_quot=True)
        assert np.array_equal(q4, q1) and np.array_equal(t4, t1)
        assert np.array_equal(a4, 2 * a1) and np.array_equal(s4, 2 * s1)


def test_reduce_reconstruction_identity(oracle):
    # the reduce's output reconstructs the float64 sum of the reconstructions up to exactly
    # its own requantisation error
    P, B = 4, 128
    q, a, s = _shards(oracle, P)
    qo, ao, so, t = oracle.reduce_fp8(q, a, s, B, 1.0, with_quot=True)
    z = sum(oracle.decompress_f64(q[p], a[p], s[p], B) for p in range(P)).reshape(-1, B)
    xh = oracle.decompress_f64(qo, ao, so, B).reshape(-1, B)
    s64 = so.astype(np.float64)[:, None]
    lhs = np.linalg.norm(xh - z, axis=1)
    rhs = np.linalg.norm(s64 * (E4M3_VALUES[qo].reshape(-1, B) - t.reshape(-1, B)), axis=1) / ao
    assert np.all(np.abs(lhs - rhs) <= 1e-9 * rhs)


# ------------------------------------------------------------------------------ arguments

def test_argument_bounds(oracle):
    # the target's contract is [2^-64, 2^64] with both ends included (the next float32 outside
    # either end is rejected), and a reduce needs P >= 1
    B = 128
    x = random_bf16_bits(2 * B, seed=12)
    q, a, s = oracle.compress(x, B, 1.0)
    below = float(np.nextafter(np.float32(2.0 ** -64), np.float32(0)))
    above = float(np.nextafter(np.float32(2.0 ** 64), np.float32(np.inf)))
    for T in (2.0 ** -64, 2.0 ** 64):
        oracle.compress(x, B, T)
        oracle.reduce_fp8(q[None], a[None], s[None], B, T)
        oracle.accumulate(q, a, s, x, B, T)
    for T in (below, above):
        with pytest.raises(ValueError, match="-6"):
            oracle.compress(x, B, T)
        with pytest.raises(ValueError, match="-6"):
            oracle.reduce_fp8(q[None], a[None], s[None], B, T)
        with pytest.raises(ValueError, match="-6"):
            oracle.accumulate(q, a, s, x, B, T)
    out_q, out_f = np.zeros(2 * B, np.uint8), np.zeros(2, np.float32)
    for P, want in ((0, -6), (-1, -6), (1, 0)):
        st = oracle.raw_status("tfp8_ref_reduce_ex", q.ctypes.data, a.ctypes.data, s.ctypes.data,
                               P, 2 * B, B, 1.0, 0, out_q.ctypes.data, out_f.ctypes.data,
                               out_f.ctypes.data, None)
        assert st == want, (P, st)


def test_argument_errors(oracle):
    x = np.zeros(256, np.uint16)
    with pytest.raises(ValueError, match="-3"):
        oracle.compress(x, 96, 1.0)           # block not a power of two
    with pytest.raises(ValueError, match="-2"):
        oracle.compress(x[:200], 128, 1.0)    # n % block != 0
    with pytest.raises(ValueError, match="-6"):
        oracle.compress(x, 128, 0.0)          # target <= 0
    with pytest.raises(ValueError, match="-6"):
        oracle.compress(x, 128, float("inf"))
    st = oracle.raw_status("tfp8_ref_compress", None, 0, 256, 128, 1.0, None, None, None, None)
    assert st == -1
    st = oracle.raw_status("tfp8_ref_compress", x.ctypes.data, 7, 256, 128, 1.0, None, None, None, None)
    assert st == -4
    # n = 0 is a no-op
    assert oracle.raw_status("tfp8_ref_compress", None, 0, 0, 128, 1.0, None, None, None, None) == 0
