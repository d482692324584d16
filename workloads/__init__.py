"""Seeded synthetic input tensors for the FP8 (ASH + DS) compression path.

This module only draws random numbers and rounds them to bfloat16.  It holds
none of the compression arithmetic, so both the CPU oracle's tests and the HIP
path's tests and benchmark can take their inputs from it without sharing any
part of the method.

The tensors stand in for tensor-parallel activations and backward gradients of
the models the TACO page evaluates (GPT 2.7B / 6.7B / 13B and Qwen2.5-7B, page
"TACO: Efficient Communication Compression of Intermediate Tensors for Scalable
Tensor-Parallel LLM Training", section 4).  That page describes such tensors as
a dense cluster near zero with a long tail (section 1), which is the shape of
every recipe below.  No dataset is used.

Recipe (fixed draw order, numpy PCG64 ``default_rng(seed)``):

* values are drawn in float64, rounded to float32 (round-to-nearest-even) and
  then to bfloat16 (round-to-nearest-even); subnormals are kept;
* ``Laplace(0, b)`` is ``rng.laplace(0, b)``, ``t(nu)*c`` is
  ``rng.standard_t(nu) * c``, ``+-U(a, b)`` is ``rng.uniform(a, b)`` times a
  sign drawn as ``rng.integers(0, 2)``;
* mixtures are per element: one ``rng.random()`` draw picks the component.

Everything is returned as raw bfloat16 bit patterns (``numpy.uint16``) in the
row-major order of the workload's shape, so a flat view is the buffer the library
compresses.
"""
from __future__ import annotations

import hashlib
import os
from dataclasses import dataclass
from typing import Tuple

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "TINY",
    "GPT2_7B",
    "GPT6_7B",
    "GPT13B_GRAD",
    "QWEN7B",
    "make_shard",
    "make_shards",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "sha256_bits",
    "random_bf16_bits",
]


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: tensor shape, block size and reduce width."""

    key: str
    label: str
    shape: Tuple[int, ...]
    block: int
    shards: int  # P: number of simulated rank shards (1 = no reduce)

    @property
    def n(self) -> int:
        out = 1
        for d in self.shape:
            out *= d
        return out

    @property
    def nblocks(self) -> int:
        return self.n // self.block


TINY = "tiny"
GPT2_7B = "gpt2.7b-act"
GPT6_7B = "gpt6.7b-act"
GPT13B_GRAD = "gpt13b-grad"
QWEN7B = "qwen2.5-7b-act"

WORKLOADS = {w.key: w for w in (
    Workload(TINY, "tiny-roundtrip 512x1024", (512, 1024), 128, 1),
    Workload(GPT2_7B, "gpt-2.7b tp activation [1,2048,2560]", (1, 2048, 2560), 128, 1),
    Workload(GPT6_7B, "gpt-6.7b tp activation [4,2048,4096]", (4, 2048, 4096), 256, 4),
    Workload(GPT13B_GRAD, "gpt-13b tp gradient [4,4096,5120]", (4, 4096, 5120), 128, 1),
    Workload(QWEN7B, "qwen2.5-7b tp activation [8,4096,3584]", (8, 4096, 3584), 128, 8),
)}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even, and return the bits.

    Inputs are finite (the recipes never produce NaN or Inf)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def sha256_bits(b: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(b).tobytes()).hexdigest()


def _signs(rng: np.random.Generator, k: int) -> np.ndarray:
    return rng.integers(0, 2, size=k).astype(np.float64) * 2.0 - 1.0


def _to_bits(v64: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(v64.astype(np.float32))


def _tiny(shard: int) -> np.ndarray:
    # 90% Laplace(0, 0.01), 9% 0.05 * t(3), 1% +-U(5, 50); blocks 0, 1, 2048 and 4095 all-zero.
    wl = WORKLOADS[TINY]
    n = wl.n
    rng = np.random.default_rng(shard)
    cat = rng.random(n)
    v = rng.laplace(0.0, 0.01, n)
    tail = cat >= 0.90
    out = (cat >= 0.99)
    mid = tail & ~out
    v[mid] = rng.standard_t(3.0, int(mid.sum())) * 0.05
    k = int(out.sum())
    v[out] = rng.uniform(5.0, 50.0, k) * _signs(rng, k)
    bits = _to_bits(v)
    B = wl.block
    for b in (0, 1, 2048, 4095):
        bits[b * B:(b + 1) * B] = 0
    return bits.reshape(wl.shape)


def _gpt2_7b(shard: int) -> np.ndarray:
    # Laplace(0, 0.02) body, 8 fixed outlier channels of +-U(10, 100) in every row.
    wl = WORKLOADS[GPT2_7B]
    rows, cols = wl.shape[0] * wl.shape[1], wl.shape[2]
    rng = np.random.default_rng(shard)
    ch = np.sort(rng.choice(cols, 8, replace=False))
    v = rng.laplace(0.0, 0.02, rows * cols).reshape(rows, cols)
    k = rows * ch.size
    v[:, ch] = (rng.uniform(10.0, 100.0, k) * _signs(rng, k)).reshape(rows, ch.size)
    return _to_bits(v.reshape(-1)).reshape(wl.shape)


def _gpt6_7b(shard: int) -> np.ndarray:
    # Laplace(0, 0.02) body with 9% of elements replaced by a 0.05 * t(2.5) tail.
    wl = WORKLOADS[GPT6_7B]
    n = wl.n
    rng = np.random.default_rng(shard)
    cat = rng.random(n)
    v = rng.laplace(0.0, 0.02, n)
    tail = cat >= 0.91
    v[tail] = rng.standard_t(2.5, int(tail.sum())) * 0.05
    return _to_bits(v).reshape(wl.shape)


def _gpt13b_grad(shard: int) -> np.ndarray:
    # Laplace(0, 1e-4) with 0.1% spikes +-U(1e-2, 1); then 5% of blocks moved into the
    # bfloat16 subnormal range and 1% of blocks (disjoint) set to zero.
    wl = WORKLOADS[GPT13B_GRAD]
    n, B, nb = wl.n, wl.block, wl.nblocks
    rng = np.random.default_rng(shard)
    cat = rng.random(n)
    v = rng.laplace(0.0, 1e-4, n)
    spike = cat >= 0.999
    k = int(spike.sum())
    v[spike] = rng.uniform(1e-2, 1.0, k) * _signs(rng, k)
    bits = _to_bits(v)
    sel = rng.permutation(nb)
    n_sub = nb * 5 // 100
    n_zero = nb // 100
    sub_blocks = np.sort(sel[:n_sub])
    zero_blocks = np.sort(sel[n_sub:n_sub + n_zero])
    blk = bits.reshape(nb, B)
    vals = bf16_bits_to_f32(blk[sub_blocks]).astype(np.float64)
    amax = np.abs(vals).max(axis=1)
    # Scale each chosen block by 2^(-127 - ceil(log2 absmax)) so its absmax lands in
    # (2^-128, 2^-127]; then round exactly onto the bfloat16 subnormal grid (step 2^-133).
    e = np.ceil(np.log2(amax))
    scaled = vals * np.exp2(-127.0 - e)[:, None]
    q = np.round(scaled * 2.0 ** 133) * 2.0 ** -133  # numpy rounds half to even
    blk[sub_blocks] = f32_to_bf16_bits(q.astype(np.float32))  # exact: q is on the grid
    blk[zero_blocks] = 0
    return blk.reshape(wl.shape)


def _qwen7b(shard: int) -> np.ndarray:
    # Laplace(0, 0.02) body with 16 outlier channels +-U(20, 200); the channel set is a
    # property of the model, drawn once from seed 0 and shared by all shards.
    wl = WORKLOADS[QWEN7B]
    rows, cols = wl.shape[0] * wl.shape[1], wl.shape[2]
    ch = np.sort(np.random.default_rng(0).choice(cols, 16, replace=False))
    rng = np.random.default_rng(shard)
    v = rng.laplace(0.0, 0.02, rows * cols).reshape(rows, cols)
    k = rows * ch.size
    v[:, ch] = (rng.uniform(20.0, 200.0, k) * _signs(rng, k)).reshape(rows, ch.size)
    return _to_bits(v.reshape(-1)).reshape(wl.shape)


_MAKERS = {TINY: _tiny, GPT2_7B: _gpt2_7b, GPT6_7B: _gpt6_7b, GPT13B_GRAD: _gpt13b_grad,
           QWEN7B: _qwen7b}


def make_shard(key: str, shard: int = 0) -> np.ndarray:
    """bfloat16 bits (uint16, the workload's shape) of shard ``shard`` of workload ``key``."""
    if key not in _MAKERS:
        raise ValueError(f"unknown workload {key!r}")
    return _MAKERS[key](shard)


def make_shards(key: str, count: int | None = None, workers: int | None = None) -> np.ndarray:
    """All P shards of a workload stacked as [P, *shape] (shard p uses seed p).

    Shards are independent, so they are drawn by a pool of ``workers`` threads (default: up to
    8, bounded by the CPUs this process may use): numpy's bulk generators and array operations
    release the GIL.  Threads rather than processes, so that nothing is forked (forking under a
    profiler's injected runtime, or after the GPU runtime is up, is unsafe)."""
    wl = WORKLOADS[key]
    P = wl.shards if count is None else count
    if workers is None:
        workers = min(8, P, len(os.sched_getaffinity(0)))
    out = np.empty((P,) + wl.shape, dtype=np.uint16)
    if workers <= 1 or P == 1:
        for p in range(P):
            out[p] = make_shard(key, p)
        return out
    from concurrent.futures import ThreadPoolExecutor

    def fill(p):
        out[p] = make_shard(key, p)

    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(fill, range(P)))
    return out


def random_bf16_bits(n: int, seed: int, scale: float = 1.0) -> np.ndarray:
    """Plain Laplace(0, scale) bfloat16 bits for ad-hoc sizes (edge-case tests)."""
    rng = np.random.default_rng(seed)
    return _to_bits(rng.laplace(0.0, scale, n))
