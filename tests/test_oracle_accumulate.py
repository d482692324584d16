"""Pins of the oracle's local gradient accumulation (AGoQ page, section 2.B: dequantize the FP8
main gradient, add the local gradient, quantize again)."""
import numpy as np
import pytest

from tiecheck import E4M3_VALUES, INT8_VALUES, assert_codes_match, tie_cap
from workloads import TINY, bf16_bits_to_f32, make_shard, random_bf16_bits

F32_ULP = 2.0 ** -23
FLAG_SETS = [0, 1, 2, 3]


def _main(oracle, flags, B=128):
    x = make_shard(TINY).reshape(-1)
    return oracle.compress(x, B, 1.0, flags=flags)


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_zero_local_gradient_keeps_the_codes(oracle, flags):
    q, a, s = _main(oracle, flags)
    g = np.zeros(q.size, np.uint16)
    qo, ao, so = oracle.accumulate(q, a, s, g, 128, 1.0, flags=flags)
    norm = (lambda c: c) if flags & 1 else (lambda c: np.where(c == 0x80, 0, c))
    assert np.array_equal(norm(qo), norm(q))
    nz = s > 0
    r_in = s[nz].astype(np.float64) / a[nz]
    assert np.all(np.abs(so[nz].astype(np.float64) / ao[nz] - r_in) <= 4 * F32_ULP * r_in)


@pytest.mark.parametrize("flags", FLAG_SETS)
@pytest.mark.parametrize("gdtype", ["bf16", "f32"])
def test_zero_main_gradient_equals_compressing_the_local_gradient(oracle, flags, gdtype):
    n, B = 64 * 128, 128
    q = np.zeros(n, np.uint8)
    a = np.ones(n // B, np.float32)
    s = np.zeros(n // B, np.float32)
    g = random_bf16_bits(n, seed=8, scale=0.3)
    if gdtype == "f32":
        g = bf16_bits_to_f32(g) * np.float32(1.0 + 2.0 ** -10)
    got = oracle.accumulate(q, a, s, g, B, 1.0, flags=flags)
    want = oracle.compress(g, B, 1.0, flags=flags)
    for u, v in zip(got, want):
        assert np.array_equal(u, v)


@pytest.mark.parametrize("flags", FLAG_SETS)
@pytest.mark.parametrize("gdtype", ["bf16", "f32"])
def test_two_routes_agree(oracle, flags, gdtype):
    q, a, s = _main(oracle, flags)
    g = random_bf16_bits(q.size, seed=9, scale=0.02)
    if gdtype == "f32":
        g = bf16_bits_to_f32(g) * np.float32(0.75)
    qa, aa, sa, ta = oracle.accumulate(q, a, s, g, 128, 1.0, with_quot=True, flags=flags)
    qb, ab, sb, tb = oracle.accumulate_rotated(q, a, s, g, 128, 1.0, with_quot=True, flags=flags)
    assert_codes_match(qb, qa, ta, max_frac=tie_cap(flags), rel=2.0 ** -40, abs_=1e-9,
                       int8=bool(flags & 1))
    assert np.all(np.abs(sb.astype(np.float64) - sa) <= F32_ULP * sa)
    assert np.all(np.abs(ab.astype(np.float64) - aa) <= F32_ULP * aa)


@pytest.mark.parametrize("route", ["definition", "rotated"])
def test_clamps_alpha_of_tiny_sums(oracle, route):
    # a main gradient compressed from bfloat16-subnormal blocks plus a local gradient of the
    # same kind: the sum's mean square is below 2^-252, so alpha is clamped at 2^126, in either
    # route
    from workloads import f32_to_bf16_bits

    B, nb = 128, 8
    rng = np.random.default_rng(32)

    def tiny():
        k = rng.integers(-(2 ** 6), 2 ** 6, (nb, B))
        k[:, 0] = 2 ** 6
        return f32_to_bf16_bits((k.astype(np.float64) * 2.0 ** -133).astype(np.float32).reshape(-1))

    q, a, s = oracle.compress(tiny(), B, 1.0)
    g = tiny()
    f = oracle.accumulate if route == "definition" else oracle.accumulate_rotated
    qo, ao, so = f(q, a, s, g, B, 1.0)
    z = (oracle.decompress_f64(q, a, s, B) + bf16_bits_to_f32(g)).reshape(nb, B)
    assert np.all(np.sqrt(1.0 / np.mean(z * z, axis=1)) > 2.0 ** 126)
    assert np.all(ao == np.float32(2.0 ** 126)) and np.all(so > 0)


@pytest.mark.parametrize("flags", FLAG_SETS)
@pytest.mark.parametrize("route", ["definition", "rotated"])
def test_target_scaling(oracle, flags, route):
    # alpha = clamp(sqrt(T / m2)) with m2 the second moment of the sum, which does not depend on
    # T: a target 4 times larger doubles alpha exactly, hence y and s, and leaves every quotient
    # and code as it was (no block here reaches the clamp)
    q, a, s = _main(oracle, flags)
    g = random_bf16_bits(q.size, seed=11, scale=0.02)
    f = oracle.accumulate if route == "definition" else oracle.accumulate_rotated
    for T in (1.0, 2.0 ** -6, 37.5):
        q1, a1, s1, t1 = f(q, a, s, g, 128, T, with_quot=True, flags=flags)
        q4, a4, s4, t4 = f(q, a, s, g, 128, 4 * T, with_quot=True, flags=flags)
        assert np.array_equal(q4, q1) and np.array_equal(t4, t1)
        assert np.array_equal(a4, 2 * a1) and np.array_equal(s4, 2 * s1)


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_requantisation_error_identity(oracle, flags):
    # ||xhat_out - (xhat_in + g)|| = ||s' (dec q' - t')|| / alpha' per block
    B = 128
    q, a, s = _main(oracle, flags, B)
    g = random_bf16_bits(q.size, seed=10, scale=0.05)
    qo, ao, so, t = oracle.accumulate(q, a, s, g, B, 1.0, with_quot=True, flags=flags)
    z = (oracle.decompress_f64(q, a, s, B, flags=flags) + bf16_bits_to_f32(g)).reshape(-1, B)
    xh = oracle.decompress_f64(qo, ao, so, B, flags=flags).reshape(-1, B)
    vals = (INT8_VALUES if flags & 1 else E4M3_VALUES)[qo].reshape(-1, B)
    lhs = np.linalg.norm(xh - z, axis=1)
    rhs = np.linalg.norm(so.astype(np.float64)[:, None] * (vals - t.reshape(-1, B)), axis=1) / ao
    assert np.all(np.abs(lhs - rhs) <= 1e-9 * np.maximum(rhs, 1e-300))


def test_accumulate_argument_errors(oracle):
    q = np.zeros(256, np.uint8)
    a, s = np.ones(2, np.float32), np.zeros(2, np.float32)
    st = oracle.raw_status("tfp8_ref_accumulate_ex", q.ctypes.data, a.ctypes.data, s.ctypes.data,
                           q.ctypes.data, 3, 256, 128, 1.0, 0, q.ctypes.data, a.ctypes.data,
                           s.ctypes.data, None)
    assert st == -4  # grad dtype
    st = oracle.raw_status("tfp8_ref_accumulate_ex", q.ctypes.data, a.ctypes.data, s.ctypes.data,
                           q.ctypes.data, 0, 256, 128, 1.0, 4, q.ctypes.data, a.ctypes.data,
                           s.ctypes.data, None)
    assert st == -6  # unknown flag
