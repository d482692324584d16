"""Pins of the oracle's E4M3FN codec, bfloat16 rounding and Hadamard against things other
than itself: the OCP format's printed points, torch's float8_e4m3fn / bfloat16 casts,
brute-force nearest-value search, and scipy's Hadamard matrix."""
import math
import os

import numpy as np
import pytest
import torch
from scipy.linalg import hadamard

from tiecheck import E4M3_VALUES

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_decode_table():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_ocp_points(oracle):
    for line in open(os.path.join(GOLDEN, "e4m3fn_points.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        got = oracle.e4m3_decode(int(code, 16))
        if val == "nan":
            assert math.isnan(got), code
        else:
            want = float.fromhex(val) if "0x" in val else float(val)
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)


def test_decode_table_matches_torch(oracle):
    ours = oracle.e4m3_decode_table()
    ref = _torch_decode_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    assert np.array_equal(E4M3_VALUES[~nan], ref[~nan])


def _brute_encode(v: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3FN value by search; ties to the even code; saturate at 448;
    sign from the input (so -0 and tiny negatives give 0x80)."""
    grid = _torch_decode_table()[:0x7F]  # codes 0x00..0x7E, ascending values
    a = np.abs(v)
    idx = np.clip(np.searchsorted(grid, a), 1, 0x7E)
    lo, hi = idx - 1, idx
    dlo, dhi = a - grid[lo], grid[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a >= grid[0x7E], 0x7E, pick)
    return (pick | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def _oracle_encode_many(oracle, v):
    enc = oracle.lib().tfp8_ref_e4m3_encode
    return np.fromiter((enc(float(x)) for x in v), dtype=np.uint8, count=len(v))


def test_encode_matches_brute_force_at_midpoints(oracle):
    grid = _torch_decode_table()[:0x7F]
    mids = 0.5 * (grid[1:] + grid[:-1])
    pts = [mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf), grid,
           np.nextafter(grid, np.inf), np.nextafter(grid, -np.inf),
           np.array([0.0, 448.0, 449.0, 463.999, 464.0, 464.001, 480.0, 1e30, 5e-324, 2.0 ** -10,
                     2.0 ** -10 * (1 + 2 ** -52), 3 * 2.0 ** -10])]
    v = np.concatenate(pts)
    v = v[np.isfinite(v)]
    v = np.concatenate([v, -v])
    assert np.array_equal(_oracle_encode_many(oracle, v), _brute_encode(v))


def test_encode_matches_brute_force_random(oracle):
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.uniform(-500, 500, 20000),
                        np.exp2(rng.uniform(-14, 9.2, 40000)) * rng.choice([-1.0, 1.0], 40000)])
    assert np.array_equal(_oracle_encode_many(oracle, v), _brute_encode(v))


def test_encode_matches_torch_cast_structured(oracle):
    # float32 inputs over every binade from 2^-12 to 2^8, all top-7 mantissa patterns and the
    # low-bit patterns around each E4M3 rounding midpoint; torch's cast is round-to-nearest-even
    # (and returns NaN above 464, so the range stops at 448).
    exps = np.arange(-12, 9)
    top = np.arange(128)
    low = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF])
    e, t, l = np.meshgrid(exps + 127, top, low, indexing="ij")
    bits = (e.astype(np.uint32) << 23) | (t.astype(np.uint32) << 16) | l.astype(np.uint32)
    f = bits.reshape(-1).view(np.float32)
    f = f[f <= 448.0]
    f = np.concatenate([f, -f])
    ref = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(_oracle_encode_many(oracle, f.astype(np.float64)), ref)


def test_encode_sign_of_zero(oracle):
    assert oracle.e4m3_encode(-1e-5) == 0x80
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(0.0) == 0x00
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00      # exact tie between 0 and 2^-9 -> even (0)
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02  # tie between 1 and 2 (x 2^-9) -> even
    assert oracle.e4m3_encode(1.0625) == 0x38          # tie between 1 and 1.125 -> even
    assert oracle.e4m3_encode(1.1875) == 0x3A
    assert oracle.e4m3_encode(464.0) == 0x7E           # tie 448/480 -> even mantissa (448)


def test_round_bf16_matches_torch(oracle):
    rng = np.random.default_rng(2)
    f = np.concatenate([rng.standard_normal(20000) * np.exp2(rng.integers(-140, 120, 20000)),
                        np.exp2(rng.uniform(-133, -120, 5000))]).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    rb = oracle.lib().tfp8_ref_round_bf16
    got = np.fromiter((rb(float(x)) for x in f), dtype=np.uint16, count=f.size)
    assert np.array_equal(got, ref)


def test_round_bf16_single_rounding(oracle):
    # A float64 value just above a bfloat16 midpoint must round up, even though rounding it
    # to float32 first would land exactly on the midpoint and then round to even (down).
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert oracle.round_bf16(v) == 0x3F81
    assert oracle.round_bf16(1.0 + 2.0 ** -8) == 0x3F80  # exact tie -> even


@pytest.mark.parametrize("B", [2, 4, 8, 16, 32, 64, 128, 256, 512, 1024])
def test_hadamard_entries_match_scipy(oracle, B):
    H = np.array([[oracle.hadamard_entry(i, j) for j in range(B)] for i in range(B)])
    assert np.array_equal(H, hadamard(B))
    assert np.array_equal(H @ H.T, B * np.eye(B, dtype=H.dtype))


@pytest.mark.parametrize("B", [2, 8, 64, 128, 256, 1024])
def test_fwht_matches_matrix_product(oracle, B):
    rng = np.random.default_rng(B)
    v = rng.standard_normal(B)
    ref = hadamard(B).astype(np.float64) @ v
    got = oracle.fwht(v)
    assert np.allclose(got, ref, rtol=0, atol=1e-12 * np.abs(v).sum())
    assert np.allclose(oracle.hadamard_dense(v), ref, rtol=0, atol=1e-12 * np.abs(v).sum())
    # (H / sqrt(B))^2 = I and energy preservation
    back = oracle.fwht(got) / B
    assert np.allclose(back, v, rtol=0, atol=1e-13 * np.abs(v).max())
    assert abs(np.dot(got, got) / B - np.dot(v, v)) <= 1e-13 * np.dot(v, v)
