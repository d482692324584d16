"""The synthetic inputs are deterministic and have the structure their recipes state."""
import os

import numpy as np
import pytest

from workloads import CONFIGS, bf16_bits_to_f32, make_shard, make_shards, sha256_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "workload_sha256.txt")


def _recorded():
    out = []
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            c, p, h = line.split()
            out.append((int(c), int(p), h))
    return out


@pytest.mark.parametrize("cid,shard,digest", _recorded())
def test_shard_hash_is_stable(cid, shard, digest):
    x = make_shard(cid, shard)
    assert x.shape == CONFIGS[cid].shape and x.dtype == np.uint16
    assert sha256_bits(x) == digest


def test_shapes_divide_into_blocks():
    for cfg in CONFIGS.values():
        assert cfg.shape[-1] % cfg.block == 0
        assert cfg.n % cfg.block == 0


def test_cfg1_structure():
    cfg = CONFIGS[1]
    v = bf16_bits_to_f32(make_shard(1)).reshape(-1, cfg.block)
    zero = np.all(v == 0, axis=1)
    assert sorted(np.nonzero(zero)[0].tolist()) == [0, 1, 2048, 4095]
    a = np.abs(v[~zero]).reshape(-1)
    big = a >= 5.0
    assert 0.008 < big.mean() < 0.012  # ~1% outliers from +-U(5, 50)
    assert a.max() <= 50.0


def test_cfg2_outlier_channels():
    cfg = CONFIGS[2]
    v = bf16_bits_to_f32(make_shard(2)).reshape(-1, cfg.shape[-1])
    big = np.abs(v) >= 10.0
    cols = np.nonzero(big.all(axis=0))[0]
    assert cols.size == 8
    assert big.sum() == 8 * v.shape[0]


def test_cfg4_subnormal_and_zero_blocks():
    cfg = CONFIGS[4]
    v = bf16_bits_to_f32(make_shard(4)).reshape(-1, cfg.block)
    amax = np.abs(v).max(axis=1)
    assert int(np.sum(amax == 0)) == cfg.nblocks // 100
    sub = (amax > 0) & (amax <= 2.0 ** -127)
    assert int(sub.sum()) == cfg.nblocks * 5 // 100
    assert np.all(amax[sub] >= 2.0 ** -128)  # (2^-128, 2^-127] before rounding to the grid


def test_shards_differ_and_pool_matches_serial():
    a = make_shards(3, count=2, workers=1)
    b = make_shards(3, count=2, workers=2)
    assert np.array_equal(a, b)
    assert not np.array_equal(a[0], a[1])
