"""The synthetic inputs are deterministic and have the structure their recipes state."""
import os

import numpy as np
import pytest

from workloads import (GPT2_7B, GPT6_7B, GPT13B_GRAD, TINY, WORKLOADS, bf16_bits_to_f32, make_shard,
                       make_shards, sha256_bits)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "workload_sha256.txt")


def _recorded():
    out = []
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            c, p, h = line.split()
            out.append((c, int(p), h))
    return out


@pytest.mark.parametrize("key,shard,digest", _recorded())
def test_shard_hash_is_stable(key, shard, digest):
    x = make_shard(key, shard)
    assert x.shape == WORKLOADS[key].shape and x.dtype == np.uint16
    assert sha256_bits(x) == digest


def test_shapes_divide_into_blocks():
    for wl in WORKLOADS.values():
        assert wl.shape[-1] % wl.block == 0
        assert wl.n % wl.block == 0


def test_tiny_structure():
    wl = WORKLOADS[TINY]
    v = bf16_bits_to_f32(make_shard(TINY)).reshape(-1, wl.block)
    zero = np.all(v == 0, axis=1)
    assert sorted(np.nonzero(zero)[0].tolist()) == [0, 1, 2048, 4095]
    a = np.abs(v[~zero]).reshape(-1)
    big = a >= 5.0
    assert 0.008 < big.mean() < 0.012  # ~1% outliers from +-U(5, 50)
    assert a.max() <= 50.0


def test_gpt2_7b_outlier_channels():
    wl = WORKLOADS[GPT2_7B]
    v = bf16_bits_to_f32(make_shard(GPT2_7B)).reshape(-1, wl.shape[-1])
    big = np.abs(v) >= 10.0
    cols = np.nonzero(big.all(axis=0))[0]
    assert cols.size == 8
    assert big.sum() == 8 * v.shape[0]


def test_gpt13b_grad_subnormal_and_zero_blocks():
    wl = WORKLOADS[GPT13B_GRAD]
    v = bf16_bits_to_f32(make_shard(GPT13B_GRAD)).reshape(-1, wl.block)
    amax = np.abs(v).max(axis=1)
    assert int(np.sum(amax == 0)) == wl.nblocks // 100
    sub = (amax > 0) & (amax <= 2.0 ** -127)
    assert int(sub.sum()) == wl.nblocks * 5 // 100
    assert np.all(amax[sub] >= 2.0 ** -128)  # (2^-128, 2^-127] before rounding to the grid


def test_shards_differ_and_pool_matches_serial():
    a = make_shards(GPT6_7B, count=2, workers=1)
    b = make_shards(GPT6_7B, count=2, workers=2)
    assert np.array_equal(a, b)
    assert not np.array_equal(a[0], a[1])
