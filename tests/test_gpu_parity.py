"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded inputs.

Each stage is fed the oracle's output of the stage before it, so a mismatch names the stage;
the end-to-end test of the Qwen-shaped workload alone chains the GPU's own outputs, against the
oracle's chain, within a bound derived from the per-stage bars.  Bars: codes identical except
admissible rounding ties on <= 1e-4 of the elements; alpha and s within 1e-6 relative (zero
blocks exact, alpha inside its clamp range); float32 reconstructions within 1e-6 relative (+ 2^-149
absolute for subnormal results); bfloat16 reconstructions identical except double-rounding
ties.
"""
import os

import numpy as np
import pytest
import torch

from gpu_helpers import (DEV, assert_codes_match_every_block, assert_reduce_matches, assert_scales,
                         assert_periodic_codes, assert_periodic_decompress, fill_periodic,
                         bits_to_gpu, check_compress, check_decompress, check_reduce, cpu,
                         f32_to_gpu, gpu_bf16_bits, say, u8_to_gpu)
from tiecheck import (E4M3_VALUES, FLAG_INT8, FLAG_NO_ROTATION, assert_codes_match,
                      assert_rel_close, rounding_interval, tie_cap)
from workloads import (GPT2_7B, GPT6_7B, GPT13B_GRAD, QWEN7B, TINY, WORKLOADS, bf16_bits_to_f32,
                       f32_to_bf16_bits, make_shard, make_shards, random_bf16_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tfp8():
    import fp8_compression_tensor_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()  # raises if the HIP library is not built
    return m


@pytest.fixture(scope="module", autouse=True)
def _threads(oracle):
    oracle.set_threads(min(16, len(os.sched_getaffinity(0))))


# ----------------------------------------------------------------------------- single-shard workloads

@pytest.mark.parametrize("key", [TINY, GPT2_7B, GPT13B_GRAD])
def test_workload_compress_decompress(oracle, tfp8, key):
    wl = WORKLOADS[key]
    say(f"{key} ({wl.label}), block {wl.block}")
    x = make_shard(key).reshape(-1)
    q, a, s = check_compress(oracle, tfp8, x, wl.block, what=f"{key} compress")
    check_decompress(oracle, tfp8, q, a, s, wl.block, what=f"{key} decompress")


# ----------------------------------------------------------------------------- GPT-6.7B shards, P = 4

def test_gpt6_7b_compress_reduce_decompress(oracle, tfp8):
    wl = WORKLOADS[GPT6_7B]
    B, P = wl.block, wl.shards
    say(f"{GPT6_7B} ({wl.label}), block {B}, P={P}")
    xs = make_shards(GPT6_7B)  # [4, 4, 2048, 4096]
    # one call compresses the stacked shards (blocks never straddle shards)
    q, a, s = check_compress(oracle, tfp8, xs.reshape(-1), B, what="gpt6.7b compress of 4 stacked shards")
    n = wl.n
    q, a, s = q.reshape(P, n), a.reshape(P, -1), s.reshape(P, -1)
    check_decompress(oracle, tfp8, q[0], a[0], s[0], B, what="gpt6.7b decompress shard 0")
    _check_reduce(oracle, tfp8, q, a, s, B, what="gpt6.7b reduce P=4")


def _check_reduce(oracle, tfp8, q, a, s, B, T=1.0, what="reduce"):
    return check_reduce(oracle, tfp8, q, a, s, B, T, what=what)


# ----------------------------------------------------------------------------- Qwen2.5-7B shards, P = 8

def _stacked_compressed(oracle, tfp8, key, flags=0):
    """The P stacked shards of a workload compressed by the GPU in one call and by the oracle,
    with the GPU's codes checked on every block and its scales on every block.  For the 8
    Qwen2.5-7B-shaped shards this is the launch that bench.py times (1.88 GB of input, the
    XCD-remapped shape)."""
    wl = WORKLOADS[key]
    B, P, n = wl.block, wl.shards, wl.n
    nbt = P * wl.nblocks
    say(f"{key} ({wl.label}), block {B}, P={P}: generating {P} shards")
    xs = make_shards(key).reshape(P, n)
    say(f"  compress of the {P} stacked shards (one call), checked on every block")
    xg = bits_to_gpu(xs.reshape(-1))
    qg, ag, sg = tfp8.compress(xg, B, 1.0, flags=flags)
    torch.cuda.synchronize()
    del xg
    q, a, s = cpu(qg), cpu(ag), cpu(sg)
    qr, ar, sr = oracle.compress(xs.reshape(-1), B, 1.0, flags=flags)
    xb = xs.reshape(nbt, B)
    nmis = assert_codes_match_every_block(
        q, qr, B, lambda idx: oracle.compress(xb[idx], B, 1.0, with_quot=True, flags=flags)[3],
        max_frac=tie_cap(flags), what=f"{key} compress codes (every block)",
        int8=bool(flags & FLAG_INT8))
    ea, es = assert_scales(a, s, ar, sr, what=f"{key} compress (every block)")
    say(f"  {key} compress: {nbt} blocks, code tie mismatches {nmis} ({nmis / q.size:.2e}), "
        f"max rel err alpha {ea:.2e} scale {es:.2e}")
    return xs, (qg, ag, sg), (q, a, s), (qr, ar, sr)


def _qwen7b_compressed(oracle, tfp8):
    return _stacked_compressed(oracle, tfp8, QWEN7B)


def test_qwen7b_pipeline(oracle, tfp8):
    wl = WORKLOADS[QWEN7B]
    B, P, n = wl.block, wl.shards, wl.n
    xs, _, _, (q, a, s) = _qwen7b_compressed(oracle, tfp8)
    del xs
    # reduce of the oracle's codes of all 8 shards, then decompress of the oracle's reduced
    # tensor, each checked in full
    q, a, s = q.reshape(P, n), a.reshape(P, -1), s.reshape(P, -1)
    cq, ca, cs = _check_reduce(oracle, tfp8, q, a, s, B, what="qwen2.5-7b reduce P=8")
    check_decompress(oracle, tfp8, cq, ca, cs, B, what="qwen2.5-7b decompress of the reduced tensor")


def test_qwen7b_end_to_end_chain(oracle, tfp8):
    # the chain bench.py times: B = 128, P = 8
    _end_to_end_chain(oracle, tfp8, QWEN7B)


def test_gpt6_7b_end_to_end_chain(oracle, tfp8):
    # B = 256 (decompress with its float64 stages) and the P = 4 reduce
    _end_to_end_chain(oracle, tfp8, GPT6_7B)


@pytest.mark.parametrize("flags", [1, 2, 3])
def test_gpt6_7b_end_to_end_chain_variants(oracle, tfp8, flags):
    # the same chain with INT8 codes, without the rotation, and both
    _end_to_end_chain(oracle, tfp8, GPT6_7B, flags)


def _end_to_end_chain(oracle, tfp8, key, flags=0):
    # GPU compress -> GPU reduce (P shards) -> GPU decompress, each stage fed the GPU's own output
    # of the stage before, against the oracle's chain on the same shards.
    #
    # Bound (Q = 448 for E4M3 codes, 127 for INT8; H = I without the rotation).  In the rotated
    # domain shard p contributes c_p = (s_p / alpha_p) dec(q_p) and the reduce requantises
    # r = sum_p c_p: its codes are code(Q r / max|r|) and it reconstructs
    # H (max|r| / Q) dec(q') / sqrt(B).  The GPU's r differs from the oracle's only through
    # compress: an admitted tie moves one code of one shard by one step of the code format
    # (changing r at that element only), and each of s_p, alpha_p may differ by 1e-6 relative.
    # So per element
    #   |r_gpu - r_ref| <= D_i = (1 + e) sum_p f_p |dec(q_gpu,p,i) - dec(q_ref,p,i)|
    #                            + e sum_p f_p |dec(q_ref,p,i)|,      f_p = s_p / alpha_p, e = 2.1e-6,
    # and max|r| moves by at most max_i D_i.  A final code may then differ from the oracle's only
    # where some quotient within (Q / max|r|) (D_i + max D) of the oracle's exact one, widened by
    # the tie window, rounds to it; alpha' within 1e-6 + |D|_2 / |r|_2 and s' within that plus
    # max D / max|r| + 1e-6 relative.  Final code mismatches are held to the tie cap of the flags
    # (1e-4 of the elements; 1e-2 without the rotation).
    from tiecheck import E4M3_VALUES, INT8_VALUES, TIE_ABS, TIE_REL

    int8 = bool(flags & FLAG_INT8)
    VALS, Q = (INT8_VALUES, 127.0) if int8 else (E4M3_VALUES, 448.0)
    wl = WORKLOADS[key]
    B, P, n = wl.block, wl.shards, wl.n
    nb = n // B
    T = 1.0
    xs, (qg, ag, sg), (q, a, s), (qr, ar, sr) = _stacked_compressed(oracle, tfp8, key, flags)

    say("  GPU reduce and decompress of the GPU's own compressed shards")
    cqg, cag, csg = tfp8.reduce_fp8(qg.view(P, n), ag.view(P, nb), sg.view(P, nb), B, T,
                                    flags=flags)
    og = tfp8.decompress(cqg, cag, csg, B, torch.float32, flags=flags)
    torch.cuda.synchronize()
    del qg, ag, sg
    cq, ca, cs, og = cpu(cqg), cpu(cag).astype(np.float64), cpu(csg).astype(np.float64), cpu(og)
    del cqg, cag, csg
    say("  the oracle's chain")
    rq, ra, rs, rt = oracle.reduce_fp8(qr.reshape(P, n), ar.reshape(P, nb), sr.reshape(P, nb), B,
                                       T, with_quot=True, flags=flags)
    orf = oracle.decompress(rq, ra, rs, B, np.float32, flags=flags)
    ra, rs = ra.astype(np.float64), rs.astype(np.float64)

    # D: the bound on |r_gpu - r_ref| per element of the reduced tensor
    e = 2.1e-6
    f = (sr.astype(np.float64) / ar.astype(np.float64)).reshape(P, nb)
    D = np.zeros((nb, B))
    for p in range(P):
        D += np.abs(VALS[qr.reshape(P, n)[p]]).reshape(nb, B) * f[p][:, None]
    D *= e
    ties = np.nonzero(q != qr)[0]
    tp, ti = ties // n, ties % n
    np.add.at(D.reshape(-1), ti, (1 + e) * f[tp, ti // B]
              * np.abs(VALS[q[ties]] - VALS[qr[ties]]))
    del q, qr
    Dmax = D.max(axis=1)
    M = Q * rs / ra  # max|r_ref| per block (s' / alpha' = max|r| / Q, fp32-rounded)
    assert np.all(rs > 0), "a reduced block is zero: these shards never cancel exactly"

    # final codes
    mis = np.nonzero(cq != rq)[0]
    if mis.size:
        k = mis // B
        t = rt[mis]
        w = (Q / (M[k] * (1 - 1e-6))) * (D.reshape(-1)[mis] + Dmax[k]) \
            + TIE_REL * np.abs(t) + TIE_ABS
        lo, hi = rounding_interval(VALS[cq[mis]], int8=int8)
        ok = (lo <= t + w) & (hi >= t - w)
        assert ok.all(), (f"end-to-end: {int((~ok).sum())} final code mismatches of {mis.size} "
                          f"outside the bound; first at {mis[np.argmax(~ok)]}")
    assert mis.size <= tie_cap(flags) * n, f"end-to-end: {mis.size} final code mismatches of {n}"

    # final scales
    Dl2 = np.sqrt((D * D).sum(axis=1))
    tol_a = 1e-6 + 1.001 * Dl2 * ra / np.sqrt(T * B)
    tol_s = tol_a + 1.001 * Dmax / M + 1e-6
    err_a = np.abs(ca - ra) / ra
    err_s = np.abs(cs - rs) / rs
    assert np.all(err_a <= tol_a), f"end-to-end alpha: worst block {int(np.argmax(err_a - tol_a))}"
    assert np.all(err_s <= tol_s), f"end-to-end scale: worst block {int(np.argmax(err_s - tol_s))}"

    # reconstructions: against each other, and both against the exact sum of the inputs
    og64, or64 = og.astype(np.float64), orf.astype(np.float64)
    diff = np.abs(og64 - or64)
    normal = np.abs(or64) >= 2.0 ** -126
    rel = diff[normal] / np.abs(or64[normal])
    z = np.zeros(n)
    for p in range(P):
        z += bf16_bits_to_f32(xs[p]).astype(np.float64)
    zn = np.sqrt(np.dot(z, z))
    e_gpu = np.sqrt(np.dot(og64 - z, og64 - z)) / zn
    e_ref = np.sqrt(np.dot(or64 - z, or64 - z)) / zn
    d_l2 = np.sqrt(np.dot(diff, diff)) / zn
    say(f"  {key} flags={flags} end to end: {ties.size} compress ties ({ties.size / (P * n):.2e}); {mis.size} final code "
        f"mismatches ({mis.size / n:.2e}); scale rel err max alpha {err_a.max():.2e} s "
        f"{err_s.max():.2e}; reconstruction vs the oracle's: max rel {rel.max():.3e}, mean rel "
        f"{rel.mean():.3e}, rel L2 {d_l2:.3e}; rel L2 error vs the exact sum: GPU chain "
        f"{e_gpu:.6e}, oracle chain {e_ref:.6e}")
    # the GPU chain is as accurate as the oracle's: with at most 1e-4 of the codes one step apart,
    # the L2 error can move by a few 1e-4 of itself at most
    assert e_gpu <= e_ref * (1 + 1e-3), (e_gpu, e_ref)


# ----------------------------------------------------------------------------- edge cases

def _special_blocks(B, rng):
    """Blocks that exercise every branch: zero, -0, constant, one-hot, Hadamard-like sign
    patterns, bfloat16-subnormal, large (2^90), small normal (2^-120), mixed magnitudes."""
    blocks = []
    blocks.append(np.zeros(B))
    blocks.append(-np.zeros(B))
    blocks.append(np.full(B, 0.75))
    oh = np.zeros(B); oh[B // 3] = -5.5; blocks.append(oh)
    blocks.append(np.where(rng.random(B) < 0.5, 1.0, -1.0) * 0.125)
    blocks.append(rng.integers(-64, 65, B) * 2.0 ** -133)       # bfloat16 subnormal block
    sub = np.zeros(B); sub[7] = 2.0 ** -133; blocks.append(sub)  # smallest bfloat16 value
    blocks.append(rng.laplace(0, 1, B) * 2.0 ** 90)
    blocks.append(rng.laplace(0, 1, B) * 2.0 ** -120)
    mixed = rng.laplace(0, 1e-3, B); mixed[0] = 3.0e4; blocks.append(mixed)
    blocks.append(rng.laplace(0, 0.02, B))
    return np.concatenate(blocks)


@pytest.mark.parametrize("B", [64, 128, 256, 512])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_edge_blocks_and_ragged_tails(oracle, tfp8, B, dtype):
    rng = np.random.default_rng(B)
    v = _special_blocks(B, rng)
    for extra in (0, 1, 5, 13):  # ragged tile tails: block counts not a multiple of 8
        vv = np.concatenate([v, rng.laplace(0, 0.05, extra * B)])
        if dtype == "bf16":
            x = f32_to_bf16_bits(vv.astype(np.float32))
            x[B:2 * B] = 0x8000  # the second block is all -0
        else:
            x = vv.astype(np.float32)
            x[B:2 * B] = -0.0
        q, a, s = check_compress(oracle, tfp8, x, B, what=f"edge B={B} {dtype} +{extra}")
        check_decompress(oracle, tfp8, q, a, s, B, what=f"edge B={B} {dtype} +{extra}")


@pytest.mark.parametrize("nblocks", [1, 2, 7, 8, 9, 1000, 4097])
def test_block_counts(oracle, tfp8, nblocks):
    x = random_bf16_bits(nblocks * 128, seed=nblocks, scale=0.01)
    q, a, s = check_compress(oracle, tfp8, x, 128, what=f"{nblocks} blocks")
    check_decompress(oracle, tfp8, q, a, s, 128, what=f"{nblocks} blocks")


@pytest.mark.parametrize("T", [2.0 ** -64, 2.0 ** -10, 37.5, 2.0 ** 20, 2.0 ** 64])
def test_target_values(oracle, tfp8, T):
    # the contract's bounds 2^-64 and 2^64 included; compress, reduce and accumulate
    x = make_shard(TINY).reshape(-1)
    q, a, s = check_compress(oracle, tfp8, x, 128, T=T, what=f"tiny T={T}")
    xr = np.stack([make_shard(TINY, p).reshape(-1) for p in range(3)])
    enc = [oracle.compress(v, 128, T) for v in xr]
    check_reduce(oracle, tfp8, np.stack([e[0] for e in enc]), np.stack([e[1] for e in enc]),
                 np.stack([e[2] for e in enc]), 128, T, what=f"reduce T={T}")
    _check_accumulate(oracle, tfp8, q, a, s, xr[1], 128, f"accumulate T={T}", T=T)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("flags", [0, 1, 2, 3])
def test_alpha_exactly_on_the_clamp_bounds(oracle, tfp8, dtype, flags):
    # Blocks whose exact alpha = sqrt(T B / sum(x^2)) is exactly 2^126, or exactly 2^-126, with
    # T B not a perfect square: the kernel's rounded sqrt(T B) and reciprocal square root may
    # put alpha one float inside the clamp range where the oracle stores the bound itself.  The
    # bar holds it to 1e-6, inside the range.  (A random sweep met such a block: float32
    # subnormals whose alpha was exactly 2^126.)
    B = 128

    def blocks(parts):  # one block per (count, magnitude, first position), alternating signs
        x = np.zeros((len(parts), B), np.float32)
        for i, (count, mag, first) in enumerate(parts):
            x[i, first:first + count] = mag * np.where(np.arange(count) % 2 == 0, 1.0, -1.0)
        return x.reshape(-1)

    cases = [
        # T B = 12; sum(x^2) = 12 * 2^-252: alpha = 2^126
        (3.0 / 32, 2.0 ** 126, [(3, 2.0 ** -125, 0), (3, 2.0 ** -125, 61), (12, 2.0 ** -126, 5),
                                (48, 2.0 ** -127, 80)]),
        # T B = 3 * 2^-53; sum(x^2) = 3 * 2^199: alpha = 2^-126
        (3.0 * 2.0 ** -60, 2.0 ** -126, [(6, 2.0 ** 99, 0), (6, 2.0 ** 99, 122),
                                         (24, 2.0 ** 98, 17)]),
    ]
    for T, bound, parts in cases:
        x = blocks(parts)
        if dtype == "bf16":
            x = f32_to_bf16_bits(x)
            assert np.array_equal(bf16_bits_to_f32(x), blocks(parts))  # exact in bfloat16
        what = f"alpha on {bound:.3e}, {dtype} flags={flags}"
        # these sparse power-of-two blocks put many rotated values exactly on code midpoints, so
        # only admissibility is checked (a ledger lifts the per-call tie cap)
        q, a, s = check_compress(oracle, tfp8, x, B, T=T, what=what, flags=flags, tie_ledger=[])
        assert np.all(a == np.float32(bound)), (what, a)  # the construction reaches the bound
        check_decompress(oracle, tfp8, q, a, s, B, what=what, flags=flags)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("flags", [0, 1, 2, 3])
@pytest.mark.parametrize("B", [64, 128, 256, 512])
def test_fast_path_bounds(oracle, tfp8, B, flags, dtype):
    # Compress takes its fast path for blocks whose peak max|w| (w = H x unnormalised, or x
    # without the rotation) lies in [2^-40, 2^60], accumulate for sums whose peak lies in
    # [2^-40, 2^56]; other blocks are brought into range by a power of two first, and
    # accumulate's exact scale path rescales again outside [2^-100, 2^100].  Random blocks
    # scaled by the powers of two that put their peak just below or just above each bound
    # (scaling by 2^k leaves the codes unchanged), and one-hot blocks whose peak is the bound
    # itself, must agree with the oracle on either side.  Accumulate adds them as the local
    # gradient to an all-zero compressed main gradient.  Peaks around 2^100 need the rotation
    # (which gathers a block's energy) to keep every input below the contract's 2^100.
    from scipy.linalg import hadamard

    rng = np.random.default_rng(4040 + B + 7 * flags + (dtype == "f32"))
    rot = not flags & FLAG_NO_ROTATION
    H = hadamard(B).astype(np.float64) if rot else np.eye(B)
    blocks = []
    for bound in (2.0 ** -100, 2.0 ** -40, 2.0 ** 56, 2.0 ** 60) + ((2.0 ** 100,) if rot else ()):
        for _ in range(8):
            v = rng.laplace(0.0, 1.0, B)
            v = bf16_bits_to_f32(f32_to_bf16_bits(v.astype(np.float32))).astype(np.float64)
            k = np.floor(np.log2(bound / np.abs(H @ v).max()))  # peak * 2^k in (bound / 2, bound]
            blocks += [v * 2.0 ** k, v * 2.0 ** (k + 1)]        # just below, just above
        if bound < 2.0 ** 100:
            one = np.zeros(B)
            one[rng.integers(0, B)] = bound * rng.choice([-1.0, 1.0])
            blocks.append(one)  # peak exactly the bound, with and without the rotation
    x = np.concatenate(blocks).astype(np.float32)
    assert np.abs(x).max() < 2.0 ** 100
    if dtype == "bf16":
        xb = f32_to_bf16_bits(x)
        assert np.array_equal(bf16_bits_to_f32(xb), x)  # every value exact in bfloat16
        x = xb
    what = f"fast-path bounds B={B} flags={flags} {dtype}"
    # admissibility only: one tie would exceed 1e-4 of these few blocks
    q, a, s = check_compress(oracle, tfp8, x, B, what=what, flags=flags, tie_ledger=[])
    check_decompress(oracle, tfp8, q, a, s, B, what=what, flags=flags)
    nb = x.size // B
    zq = np.zeros(x.size, np.uint8)
    _check_accumulate(oracle, tfp8, zq, np.ones(nb, np.float32), np.zeros(nb, np.float32), x, B,
                      what + " accumulate", flags=flags, tie_ledger=[])


@pytest.mark.parametrize("flags", [0, 1, 2, 3])
@pytest.mark.parametrize("B", [64, 128, 256, 512])
def test_reduce_range_bounds(oracle, tfp8, B, flags):
    # The reduce rescales sums whose peak max|r| lies outside [2^-100, 2^100] by a power of two
    # before requantising them.  Contributions whose sums straddle both bounds: random blocks
    # scaled so that one contribution's peak (max|H x| / sqrt(B) with the rotation, max|x|
    # without) lies just below or just above 2^-100, and constant blocks c 1 whose peak
    # (sqrt(B) |c| with the rotation, |c| without) lies around 2^100 with |c| < 2^100, reduced
    # as P = 1, 2 and 3 copies (the sum's peak P times one contribution's).
    from scipy.linalg import hadamard

    rot = not flags & FLAG_NO_ROTATION
    H = hadamard(B).astype(np.float64) / np.sqrt(B) if rot else np.eye(B)
    rng = np.random.default_rng(5050 + B + 7 * flags)
    blocks = []
    for _ in range(8):
        v = rng.laplace(0.0, 1.0, B)
        v = bf16_bits_to_f32(f32_to_bf16_bits(v.astype(np.float32))).astype(np.float64)
        k = np.floor(np.log2(2.0 ** -100 / np.abs(H @ v).max()))
        blocks += [v * 2.0 ** k, v * 2.0 ** (k + 1)]
    for c in (2.0 ** 94, 2.0 ** 95, 2.0 ** 96, 1.5 * 2.0 ** 96, 2.0 ** 97, 1.5 * 2.0 ** 98,
              1.5 * 2.0 ** 99):
        blocks.append(np.full(B, c * rng.choice([-1.0, 1.0])))
    x = np.concatenate(blocks).astype(np.float32)
    assert np.abs(x).max() < 2.0 ** 100
    xb = f32_to_bf16_bits(x)
    assert np.array_equal(bf16_bits_to_f32(xb), x)
    q, a, s = oracle.compress(xb, B, 1.0, flags=flags)
    for P in (1, 2, 3):
        check_reduce(oracle, tfp8, np.stack([q] * P), np.stack([a] * P), np.stack([s] * P), B,
                     what=f"reduce range bounds B={B} flags={flags} P={P}", flags=flags,
                     tie_ledger=[])


@pytest.mark.parametrize("flags", [0, 1, 2, 3])
@pytest.mark.parametrize("B", [64, 128, 256, 512])
def test_accumulate_negligible_main_bound(oracle, tfp8, B, flags):
    # Accumulate leaves a main-gradient term out when its peak is below about 2^-60 of the local
    # gradient's transformed peak (it could then move alpha by 2^-60 relative at most, and a code
    # only at a near-exact tie).  Main-gradient blocks scaled so that their peak relative to the
    # local gradient's steps across that threshold, from 2^-68 to 2^-52, must agree with the
    # oracle, which adds every term.
    from scipy.linalg import hadamard

    H = hadamard(B).astype(np.float64) if not flags & FLAG_NO_ROTATION else np.eye(B)
    rng = np.random.default_rng(6060 + B + 7 * flags)
    steps = np.arange(-68, -51)
    g = rng.laplace(0.0, 1.0, (steps.size, B))
    g = bf16_bits_to_f32(f32_to_bf16_bits(g.astype(np.float32))).astype(np.float64)
    m = rng.laplace(0.0, 1.0, (steps.size, B))
    m = bf16_bits_to_f32(f32_to_bf16_bits(m.astype(np.float32))).astype(np.float64)
    ratio = np.abs(m @ H.T).max(axis=1) / np.abs(g @ H.T).max(axis=1)
    m *= 2.0 ** (steps - np.floor(np.log2(ratio)))[:, None]  # peak ratio in [2^step, 2^(step+1))
    xm = f32_to_bf16_bits(m.astype(np.float32).reshape(-1))
    assert np.array_equal(bf16_bits_to_f32(xm), m.reshape(-1))
    q, a, s = oracle.compress(xm, B, 1.0, flags=flags)
    _check_accumulate(oracle, tfp8, q, a, s, f32_to_bf16_bits(g.astype(np.float32).reshape(-1)), B,
                      f"negligible main B={B} flags={flags}", flags=flags, tie_ledger=[])


@pytest.mark.parametrize("gdtype", ["bf16", "f32"])
@pytest.mark.parametrize("flags", [0, 1, 2, 3])
@pytest.mark.parametrize("B", [64, 128, 256, 512])
def test_accumulate_fix_pass_bound(oracle, tfp8, B, flags, gdtype):
    # Accumulate sets a block aside for its exact pass when the sum's peak is under half the
    # larger of its two terms' peaks.  With the local gradient g = -lambda xhat (xhat the main
    # gradient's reconstruction) the sum is (1 - lambda) xhat, so blocks with lambda just below
    # and just above 1/2 take the two paths; both must agree with the oracle.
    rng = np.random.default_rng(7070 + B + 7 * flags + (gdtype == "f32"))
    lam = np.linspace(0.40, 0.60, 41)
    nb = lam.size
    xm = f32_to_bf16_bits(rng.laplace(0.0, 1.0, nb * B).astype(np.float32))
    q, a, s = oracle.compress(xm, B, 1.0, flags=flags)
    xhat = oracle.decompress_f64(q, a, s, B, flags=flags).reshape(nb, B)
    g = (-lam[:, None] * xhat).reshape(-1).astype(np.float32)
    g = g if gdtype == "f32" else f32_to_bf16_bits(g)
    _check_accumulate(oracle, tfp8, q, a, s, g, B, f"fix-pass bound B={B} flags={flags} {gdtype}",
                      flags=flags, tie_ledger=[])


def _every_value_blocks(dtype, qmax, low, B):
    """Every float32 (or bfloat16) value with magnitude in [low, qmax], both signs, 511 per block
    of B = 512 after a leading qmax; the tail is padded with 1.0."""
    lo, hi = np.float32(low).view(np.uint32), np.float32(qmax).view(np.uint32)
    step = 1 if dtype == "f32" else 1 << 16
    pos = np.arange(lo, hi + 1, step, dtype=np.uint32).view(np.float32)
    vals = np.concatenate([pos, -pos])
    nb = -(-vals.size // (B - 1))
    x = np.ones((nb, B), np.float32)
    x[:, 0] = qmax
    body = x[:, 1:].reshape(-1)
    body[:vals.size] = vals
    x[:, 1:] = body.reshape(nb, B - 1)
    return x.reshape(-1), nb


@pytest.mark.parametrize("dtype,flags", [("f32", 2), ("bf16", 2), ("f32", 3)])
def test_hardware_conversion_every_fp32_value(oracle, tfp8, dtype, flags):
    # The kernels' code conversion, checked exhaustively through compress: without the rotation
    # a block whose largest magnitude is exactly Q_max has code multiplier Q_max / Q_max = 1, so
    # every other element's code is the conversion of that exact input value (the oracle's
    # quotient y / s is the same value exactly).  E4M3 (flags 2): every float32 bit pattern with
    # magnitude in [2^-12, 448], both signs, 511 per block of 512 after a leading 448 -- round to
    # nearest even at every midpoint, the subnormal grid, rounding to +-0 and the top of the
    # range; with bfloat16 input, every bfloat16 value in that range (the widening path).  INT8
    # (flags 3): every float32 in [2^-3, 127] after a leading 127 -- the rounding to integers,
    # ties to even, and the byte packing.  No tie allowance: the codes must be identical.
    B = 512
    qmax, low = (127.0, 2.0 ** -3) if flags & 1 else (448.0, 2.0 ** -12)
    x, nb = _every_value_blocks(dtype, qmax, low, B)
    say(f"  every {dtype} value in [{low}, {qmax}], both signs, flags {flags}: {x.size} elements, "
        f"{nb} blocks")
    xin = x if dtype == "f32" else f32_to_bf16_bits(x)  # exact: every value is a bfloat16
    q, a, s = tfp8.compress(f32_to_gpu(x) if dtype == "f32" else bits_to_gpu(xin), B, 1.0,
                            flags=flags)
    torch.cuda.synchronize()
    q, a, s = cpu(q), cpu(a), cpu(s)
    qr, ar, sr = oracle.compress(xin, B, 1.0, flags=flags)
    bad = np.nonzero(q != qr)[0]
    assert bad.size == 0, (f"{bad.size} codes differ; first at value {x[bad[0]]!r}: "
                           f"got {q[bad[0]]:#04x}, oracle {qr[bad[0]]:#04x}")
    assert_scales(a, s, ar, sr, what="every-value blocks")
    assert np.all(q.reshape(nb, B)[:, 0] == (0x7F if flags & 1 else 0x7E))


def test_accumulate_every_fp32_value_onto_zero_main(oracle, tfp8):
    # The every-float32 blocks (magnitudes in [2^-12, 448], 64 similar values per lane at
    # B = 512) as the local gradient added to an all-zero compressed main gradient, without the
    # rotation: the accumulate's own sum of squares and scales on blocks where a sequential
    # float32 sum misses the alpha bar.  Codes identical to the oracle's (the quotients are the
    # inputs exactly), alpha and s within 1e-6.
    B = 512
    g, nb = _every_value_blocks("f32", 448.0, 2.0 ** -12, B)
    n = g.size
    q0 = np.zeros(n, np.uint8)
    a0 = np.ones(nb, np.float32)
    s0 = np.zeros(nb, np.float32)
    say(f"  accumulate onto zero: {n} elements, {nb} blocks")
    q, a, s = tfp8.accumulate(u8_to_gpu(q0), f32_to_gpu(a0), f32_to_gpu(s0), f32_to_gpu(g), B, 1.0,
                              flags=2)
    torch.cuda.synchronize()
    q, a, s = cpu(q), cpu(a), cpu(s)
    qr, ar, sr = oracle.accumulate(q0, a0, s0, g, B, 1.0, flags=2)
    bad = np.nonzero(q != qr)[0]
    assert bad.size == 0, (f"{bad.size} codes differ; first at value {g[bad[0]]!r}: "
                           f"got {q[bad[0]]:#04x}, oracle {qr[bad[0]]:#04x}")
    assert_scales(a, s, ar, sr, what="accumulate every-value blocks")


def test_decompress_bf16_at_a_double_rounding_tie(oracle, tfp8):
    # alpha = float32(256/257), s = 1 and the code of +-1.0 without the rotation reconstruct to
    # +-1/alpha, 2.3e-10 beyond the bfloat16 midpoint 1 + 2^-8.  The oracle rounds that once, to
    # 1 + 2^-7; the kernel multiplies in float32, which lands on the midpoint, then rounds to
    # even.  The float32 output is exact there, and the bfloat16 output is one of the two
    # neighbours, a mismatch the comparison admits only because the exact value sits at the tie.
    B = 64
    one = int(np.flatnonzero(E4M3_VALUES == 1.0)[0])
    q = np.full(2 * B, one, np.uint8)
    q[B:] |= 0x80
    a = np.full(2, np.float32(256 / 257), np.float32)
    s = np.ones(2, np.float32)
    o32 = check_decompress(oracle, tfp8, q, a, s, B, what="double-rounding tie",
                           flags=FLAG_NO_ROTATION)
    assert np.all(cpu(o32)[:B] == np.float32(1 + 2.0 ** -8))
    o16 = gpu_bf16_bits(tfp8.decompress(u8_to_gpu(q), f32_to_gpu(a), f32_to_gpu(s), B,
                                        torch.bfloat16, flags=FLAG_NO_ROTATION))
    assert set(o16[:B].tolist()) <= {0x3F80, 0x3F81} and set(o16[B:].tolist()) <= {0xBF80, 0xBF81}


@pytest.mark.parametrize("B", [128, 256, 512])
def test_decompress_cancelling_partial_sums(oracle, tfp8, B):
    # Codes of +-448 along a Hadamard row make the inverse transform of a block one spike of
    # 448 B, its partial sums passing 2^15 from the seventh stage on.  In 4 pairs of positions
    # whose row signs differ, the codes are set to +t and -t (t = m 2^-9, a subnormal code): the
    # two changes cancel exactly in half of the outputs, which are then exactly 0, while the
    # partial sums carry 2^-9 bits at magnitudes where float32 keeps only 2^-8.  A float32
    # rounding in any stage but the last leaves a residue in those zeros (at B >= 256 it did,
    # before the last stages ran in float64).  Alpha = s = 1; float32 and bfloat16 outputs
    # against the oracle.
    rng = np.random.default_rng(B)
    nb = 257
    r = np.arange(B)
    sign = np.array([[(-1) ** bin(i & j).count("1") for j in r] for i in r], np.int8)
    q = np.empty((nb, B), np.uint8)
    for b in range(nb):
        row = sign[rng.integers(1, B)]  # row 0 is all +1: no pair of opposite signs
        q[b] = np.where(row > 0, 0x7E, 0xFE)  # +-448 along the row
        free = np.ones(B, bool)
        for _ in range(4):
            j1 = int(rng.choice(np.nonzero(free)[0]))
            j2 = int(rng.choice(np.nonzero(free & (row != row[j1]))[0]))
            m = int(rng.integers(1, 8))
            q[b, j1], q[b, j2] = m, 0x80 | m  # +m 2^-9 and -m 2^-9
            free[[j1, j2]] = False
    q = q.reshape(-1)
    a = np.ones(nb, np.float32)
    s = np.ones(nb, np.float32)
    check_decompress(oracle, tfp8, q, a, s, B, what=f"cancelling partial sums B={B}")


@pytest.mark.parametrize("flags", [2, 3])
def test_hardware_decode_every_code(oracle, tfp8, flags):
    # The kernels' code decoding, checked exhaustively through decompress: without the rotation
    # and with alpha = s = 1 the output is the code's value itself.  Every E4M3 code but the two
    # NaNs (flags 2), or every INT8 code (flags 3), at every position of a block, in float32 and
    # bfloat16 (every code value is a bfloat16), identical to the oracle's.
    B = 256
    codes = np.arange(256, dtype=np.uint8)
    if not flags & 1:
        codes = codes[(codes & 0x7F) != 0x7F]  # 0x7F and 0xFF are NaN
    nb = B  # block k holds the codes rotated by k, so each code meets every position
    q = np.stack([np.roll(np.resize(codes, B), k) for k in range(nb)]).reshape(-1)
    a = np.ones(nb, np.float32)
    s = np.ones(nb, np.float32)
    qg, ag, sg = u8_to_gpu(q), f32_to_gpu(a), f32_to_gpu(s)
    o32 = cpu(tfp8.decompress(qg, ag, sg, B, torch.float32, flags=flags))
    o16 = gpu_bf16_bits(tfp8.decompress(qg, ag, sg, B, torch.bfloat16, flags=flags))
    r32 = oracle.decompress(q, a, s, B, np.float32, flags=flags)
    r16 = oracle.decompress(q, a, s, B, np.uint16, flags=flags)
    # values identical; the bit patterns may differ only in the sign of a zero (code 0x80 is -0,
    # and the bar compares values, where +0 == -0)
    for got, ref in ((o32, r32), (bf16_bits_to_f32(o16), bf16_bits_to_f32(r16))):
        assert np.array_equal(got, ref)
        diff = np.nonzero(got.view(np.uint32) != ref.view(np.uint32))[0]
        assert np.all(ref[diff] == 0), ref[diff][:8]
        say(f"  decode flags {flags}: {got.size} values identical, {diff.size} zeros of the "
            f"other sign")


def test_constructed_exact_ties(oracle, tfp8):
    """Rotated values placed exactly on E4M3 rounding midpoints (float32 input, B = 256):
    x = H z / 16 with z_0 = 448 and every other z_i a midpoint between two E4M3 values in
    [1, 16), target = float32(mean(x^2)) so the oracle's alpha is exactly 1, y = z and s = 1.
    Every partial sum of either side's transform is a multiple of 2^-8 below 2^21 (exact in
    float32 and float64), so both sides see the exact midpoints and must round each one to
    the even code."""
    from scipy.linalg import hadamard

    B = 256
    grid = 1.0 + np.arange(8) / 8.0                      # 1, 1.125, ..., 1.875
    mids = 0.5 * (grid[:-1] + grid[1:])                  # 1.0625, ..., 1.8125
    mids = np.concatenate([mids, [0.5 * (1.875 + 2.0)]])  # 1.9375: between 1.875 and 2
    rng = np.random.default_rng(9)
    Z = (rng.choice(mids, (48, B)) * rng.choice([-1.0, 1.0], (48, B))
         * 2.0 ** rng.integers(0, 4, (48, B)))
    Z[:, 0] = 448.0
    X = Z @ hadamard(B).astype(np.float64) / 16.0        # rows are H z / 16 (H symmetric)
    x32 = X.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), X), "construction must be exact in float32"
    for k in range(Z.shape[0]):
        T = float(np.float32(np.mean(X[k] * X[k])))
        q, a, s = check_compress(oracle, tfp8, x32[k], B, T=T, what=f"exact ties block {k}",
                                 gpu=True)
        qr, ar, sr, tr = oracle.compress(x32[k], B, T, with_quot=True)
        assert ar[0] == 1.0 and sr[0] == 1.0 and np.array_equal(tr, Z[k])
        assert np.array_equal(q, qr), f"block {k}: tie rounding differs"


# ----------------------------------------------------------------------------- reduce cases

@pytest.mark.parametrize("P", [1, 2, 3, 8, 16, 33, 64])
@pytest.mark.parametrize("B", [64, 128, 256, 512])
def test_reduce_general(oracle, tfp8, P, B):
    rng = np.random.default_rng(100 * P + B)
    nb = 37
    xs = [f32_to_bf16_bits((rng.laplace(0, 0.02, nb * B) * (1 + p)).astype(np.float32))
          for p in range(P)]
    # block 3 zero everywhere, block 5 zero in contribution 0, block 6 bfloat16-subnormal
    for p in range(P):
        xs[p][3 * B:4 * B] = 0
        xs[p][6 * B:7 * B] = f32_to_bf16_bits(
            (rng.integers(-64, 65, B) * 2.0 ** -133).astype(np.float32))
    xs[0][5 * B:6 * B] = 0
    enc = [oracle.compress(x, B, 1.0) for x in xs]
    q = np.stack([e[0] for e in enc]); a = np.stack([e[1] for e in enc]); s = np.stack([e[2] for e in enc])
    _check_reduce(oracle, tfp8, q, a, s, B, what=f"reduce P={P} B={B}")


def _messages(parts, n, nb, pad):
    """One receive buffer holding a [codes | alpha | scale] message per contribution (the
    oracle's compressed shards), `pad` bytes apart; returns the buffer and [P, ...] row views."""
    P = len(parts)
    M = (n + 8 * nb + pad + 15) // 16 * 16
    host = np.zeros((P, M), np.uint8)
    for p, (q, a, s) in enumerate(parts):
        host[p, :n] = q
        host[p, n:n + 4 * nb] = np.asarray(a, np.float32).view(np.uint8)
        host[p, n + 4 * nb:n + 8 * nb] = np.asarray(s, np.float32).view(np.uint8)
    buf = u8_to_gpu(host)
    return buf, buf[:, :n], buf[:, n:n + 4 * nb].view(torch.float32), \
        buf[:, n + 4 * nb:n + 8 * nb].view(torch.float32)


@pytest.mark.parametrize("B,P,pad,flags", [(128, 8, 0, 0), (64, 3, 65536 + 1024, 0),
                                           (256, 5, 16, 1), (512, 2, 4096, 0), (128, 1, 0, 0)])
def test_reduce_strided_packed_messages(oracle, tfp8, B, P, pad, flags):
    # the P contributions read where one all-to-all would leave them: a [codes | alpha | scale]
    # message per peer in one buffer (alpha and scale inside the codes' span); against the
    # oracle's reduce of the same contributions, and bit for bit against the contiguous call
    nb = 4097 if B < 512 else 1025  # several tiles and a ragged tail
    n = nb * B
    parts = [oracle.compress(random_bf16_bits(n, 100 + p, 0.02 * (p + 1)), B, 1.0, flags=flags)
             for p in range(P)]
    buf, qv, av, sv = _messages(parts, n, nb, pad)
    assert not qv.is_contiguous() or P == 1
    got = tfp8.reduce_fp8(qv, av, sv, B, 1.0, flags=flags)
    ref_gpu = tfp8.reduce_fp8(u8_to_gpu(np.stack([p[0] for p in parts])),
                              f32_to_gpu(np.stack([p[1] for p in parts])),
                              f32_to_gpu(np.stack([p[2] for p in parts])), B, 1.0, flags=flags)
    torch.cuda.synchronize()
    for u, v in zip(got, ref_gpu):
        assert torch.equal(u, v)
    rq, ra, rs, rt = oracle.reduce_fp8(np.stack([p[0] for p in parts]),
                                       np.stack([p[1] for p in parts]),
                                       np.stack([p[2] for p in parts]), B, 1.0, with_quot=True,
                                       flags=flags)
    nmis = assert_codes_match(cpu(got[0]), rq, rt, what="strided reduce codes",
                              int8=bool(flags & 1))
    assert_scales(cpu(got[1]), cpu(got[2]), ra, rs, what="strided reduce")
    say(f"  strided reduce B={B} P={P} pad={pad} flags={flags}: tie mismatches {nmis}")


def test_reduce_strided_random_layouts(tfp8, monkeypatch):
    # 300 seeded layouts with the three row strides drawn apart: P in 1..64, every B and flag
    # set, 3-3000 blocks, the codes' rows n plus up to 1 MiB apart (a multiple of 16 bytes), the
    # alpha and scale rows nb plus up to 4096 floats apart.  The padding between rows holds
    # random bytes (codes) and NaN (scales), so a read outside the rows would show.  The strided
    # call must equal the contiguous call bit for bit (that one is held to the oracle above),
    # through the full library and through the capped build, whose wavefronts loop over tiles.
    capped = _capped()
    rng = np.random.default_rng(9100)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(9100)
    total = 0
    for case in range(300):
        B = int(rng.choice([64, 128, 256, 512]))
        flags = int(rng.integers(0, 4))
        P = min(64, int(np.exp(rng.uniform(0, np.log(65)))))
        nb = int(np.exp(rng.uniform(np.log(3), np.log(3000))))
        n = nb * B
        cst = n + 16 * int(rng.integers(0, 1 << 16))
        ast, sst = nb + int(rng.integers(0, 4097)), nb + int(rng.integers(0, 4097))
        q, a, s = _random_codes(rng, P, n, B, flags)
        what = f"strided layout case {case}: B={B} flags={flags} P={P} nb={nb} strides {cst} {ast} {sst}"
        total += P * n
        qbuf = torch.randint(0, 256, (P * cst,), dtype=torch.uint8, device=DEV, generator=gen)
        abuf = torch.full((P * ast,), float("nan"), dtype=torch.float32, device=DEV)
        sbuf = torch.full((P * sst,), float("nan"), dtype=torch.float32, device=DEV)
        qv = qbuf.as_strided((P, n), (cst, 1))
        av = abuf.as_strided((P, nb), (ast, 1))
        sv = sbuf.as_strided((P, nb), (sst, 1))
        qv.copy_(u8_to_gpu(q))
        av.copy_(f32_to_gpu(a))
        sv.copy_(f32_to_gpu(s))
        ref = tfp8.reduce_fp8(u8_to_gpu(q), f32_to_gpu(a), f32_to_gpu(s), B, 1.0, flags=flags)
        got = tfp8.reduce_fp8(qv, av, sv, B, 1.0, flags=flags)
        with monkeypatch.context() as m:
            m.setattr(tfp8, "_lib", capped)
            got_capped = tfp8.reduce_fp8(qv, av, sv, B, 1.0, flags=flags)
        torch.cuda.synchronize()
        for u, v, w in zip(ref, got, got_capped):
            assert _same_bits(cpu(u), cpu(v)), what
            assert _same_bits(cpu(u), cpu(w)), what + " (capped build)"
    say(f"  300 strided layouts ({total} codes in all) equal the contiguous reduce bit for bit")


def test_sharded_two_shot_dataflow_equals_whole_reduce(oracle, tfp8):
    # The data flow of a two-shot compressed all-reduce over P ranks, on one GPU: each rank's
    # chunk (a block-aligned 1/P of every contribution) is reduced where it lies, through the
    # strided call at row stride n, into its slice of one gathered output.  Blocks are
    # independent, so the gathered result must equal the whole-tensor reduce bit for bit, and
    # the whole-tensor reduce matches the oracle.
    P, B = 8, 128
    n = WORKLOADS[TINY].n
    nb, c = n // B, n // P
    cb = c // B
    xs = np.stack([make_shard(TINY, p).reshape(-1) for p in range(P)])
    enc = [oracle.compress(x, B, 1.0) for x in xs]
    q = u8_to_gpu(np.stack([e[0] for e in enc]))
    a = f32_to_gpu(np.stack([e[1] for e in enc]))
    s = f32_to_gpu(np.stack([e[2] for e in enc]))
    whole = tfp8.reduce_fp8(q, a, s, B, 1.0)
    gq = torch.empty(n, dtype=torch.uint8, device=DEV)
    ga = torch.empty(nb, dtype=torch.float32, device=DEV)
    gs = torch.empty(nb, dtype=torch.float32, device=DEV)
    for r in range(P):
        tfp8.reduce_fp8(q[:, r * c:(r + 1) * c], a[:, r * cb:(r + 1) * cb], s[:, r * cb:(r + 1) * cb],
                        B, 1.0, out=(gq[r * c:(r + 1) * c], ga[r * cb:(r + 1) * cb],
                                     gs[r * cb:(r + 1) * cb]))
    torch.cuda.synchronize()
    for u, v in zip((gq, ga, gs), whole):
        assert torch.equal(u, v)
    rq, ra, rs, rt = oracle.reduce_fp8(np.stack([e[0] for e in enc]), np.stack([e[1] for e in enc]),
                                       np.stack([e[2] for e in enc]), B, 1.0, with_quot=True)
    assert_codes_match(cpu(gq), rq, rt, what="sharded reduce codes")
    assert_scales(cpu(ga), cpu(gs), ra, rs, what="sharded reduce")


def test_reduce_strided_wrapper_checks(tfp8):
    buf = torch.zeros(4, 4096, dtype=torch.uint8, device=DEV)
    a = torch.ones(4, 64, dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError, match="rows"):  # rows not contiguous
        tfp8.reduce_fp8(buf[:, ::2], a[:, :16], a[:, 16:32], 128)
    with pytest.raises(ValueError, match=r"\[4, 16\]"):  # scales of the wrong length
        tfp8.reduce_fp8(buf[:, :2048], a[:, :8], a[:, 16:32], 128)
    with pytest.raises(tfp8.TFP8Error, match="TFP8_E_ARG"):  # rows that overlap (stride < row)
        tfp8.reduce_fp8(buf.view(-1)[:8192].as_strided((4, 2048), (1024, 1)), a[:, :16],
                        a[:, 16:32], 128)


def test_reduce_identities(oracle, tfp8):
    B = 128
    x = make_shard(TINY).reshape(-1)
    q, a, s = oracle.compress(x, B, 1.0)
    # a contribution and its negation cancel: every block becomes a zero block
    q2, a2, s2 = np.stack([q, q ^ 0x80]), np.stack([a, a]), np.stack([s, s])
    cq, ca, cs = tfp8.reduce_fp8(u8_to_gpu(q2), f32_to_gpu(a2), f32_to_gpu(s2), B, 1.0)
    torch.cuda.synchronize()
    assert np.all(cpu(cq) == 0) and np.all(cpu(ca) == 1.0) and np.all(cpu(cs) == 0.0)
    # a single contribution is left as it is (codes up to ties, s/alpha within 1e-6)
    cq, ca, cs = tfp8.reduce_fp8(u8_to_gpu(q[None]), f32_to_gpu(a[None]), f32_to_gpu(s[None]), B, 1.0)
    torch.cuda.synchronize()
    # equal codes, except that a -0 code may come back as +0 (its value is zero either way)
    assert np.array_equal(cpu(cq), np.where(q == 0x80, 0, q))
    nz = s > 0
    assert_rel_close(cpu(cs)[nz] / cpu(ca)[nz], s[nz].astype(np.float64) / a[nz], 1e-6,
                     what="s/alpha under P=1")
    # summed in the order p = 0, 1, 2: a large contribution and its exact negation cancel before
    # a contribution 2^40 times smaller is added, so [x, -x, y] reduces to exactly what [y] alone
    # does (the products g_p dec(q_p) are exact, and so is each partial sum here), through the
    # general any-P form and a fixed-P form (a zero contribution appended)
    y = oracle.compress(make_shard(TINY, 1).reshape(-1), B, 1.0)
    big = s * np.float32(2.0 ** 20)
    one = tfp8.reduce_fp8(u8_to_gpu(y[0][None]), f32_to_gpu(y[1][None]),
                          f32_to_gpu((y[2] * np.float32(2.0 ** -20))[None]), B, 1.0)
    for P in (3, 4):
        qs = [q, q ^ 0x80, y[0], np.zeros_like(q)][:P]
        as_ = [a, a, y[1], np.ones_like(a)][:P]
        ss = [big, big, y[2] * np.float32(2.0 ** -20), np.zeros_like(s)][:P]
        got = tfp8.reduce_fp8(u8_to_gpu(np.stack(qs)), f32_to_gpu(np.stack(as_)),
                              f32_to_gpu(np.stack(ss)), B, 1.0)
        torch.cuda.synchronize()
        for u, v in zip(got, one):
            assert torch.equal(u.view(torch.uint8), v.view(torch.uint8)), f"[x, -x, y] P={P}"


@pytest.mark.parametrize("flags", [0, 1])
def test_reduce_ill_conditioned_blocks(oracle, tfp8, flags):
    # Blocks whose contributions cancel far below float64's resolution of their peaks:
    # contribution 0 of the even blocks is 2^90 times the others and contribution 3 its exact
    # negation, with two ordinary contributions between them.  Summed in that order in float64
    # the small terms are rounded away against contribution 0 wherever it is nonzero, and the
    # oracle (original domain) and the kernel (rotated domain) keep different parts of them.
    # Codes and scales of such blocks that fail the tie rule are admitted within the bound both
    # float64 sums satisfy (tiecheck.reduce_sum_bound); the odd blocks, with the same pattern at
    # ordinary scale, have a bound far inside the tie window.
    from tiecheck import TIE_ABS, reduce_quotient_slack, reduce_sum_bound

    B, nb = 128, 64
    rng = np.random.default_rng(9090)
    big = rng.laplace(0.0, 1.0, (nb, B)) * np.where(np.arange(nb) % 2 == 0, 2.0 ** 90, 1.0)[:, None]
    xs = [big, rng.laplace(0.0, 1.0, (nb, B)), rng.laplace(0.0, 1.0, (nb, B)), -big]
    enc = [oracle.compress(f32_to_bf16_bits(v.astype(np.float32).reshape(-1)), B, 1.0,
                           flags=flags) for v in xs]
    q, a, s = (np.stack([e[i] for e in enc]) for i in range(3))
    # the construction reaches the case: the even blocks' bound dwarfs the tie window, the odd
    # blocks' does not
    Q = 127.0 if flags & FLAG_INT8 else 448.0
    _, ra, rs = oracle.reduce_fp8(q, a, s, B, 1.0, flags=flags)
    w, _ = reduce_quotient_slack(reduce_sum_bound(a, s, Q), ra, rs, Q)
    ill = w > TIE_ABS / 8
    assert ill[0::2].all() and not ill[1::2].any(), ill
    check_reduce(oracle, tfp8, q, a, s, B, what=f"ill-conditioned reduce flags={flags}",
                 flags=flags, tie_ledger=[])


# ----------------------------------------------------------------------------- robustness

def test_guard_bytes_untouched(tfp8):
    B, nb = 128, 29
    n = nb * B
    x = bits_to_gpu(random_bf16_bits(n, seed=3))
    pad = 4096
    codes = torch.full((n + 2 * pad,), 0xA5, dtype=torch.uint8, device=DEV)
    alpha = torch.full((nb + 2 * 64,), 7.0, dtype=torch.float32, device=DEV)
    scale = torch.full((nb + 2 * 64,), 9.0, dtype=torch.float32, device=DEV)
    out = (codes[pad:pad + n], alpha[64:64 + nb], scale[64:64 + nb])
    tfp8.compress(x, B, 1.0, out=out)
    dec = torch.full((n + 2 * pad,), -3.0, dtype=torch.float32, device=DEV)
    tfp8.decompress(*out, B, torch.float32, out=dec[pad:pad + n])
    torch.cuda.synchronize()
    c, a, s, d = cpu(codes), cpu(alpha), cpu(scale), cpu(dec)
    assert np.all(c[:pad] == 0xA5) and np.all(c[pad + n:] == 0xA5)
    assert np.all(a[:64] == 7.0) and np.all(a[64 + nb:] == 7.0)
    assert np.all(s[:64] == 9.0) and np.all(s[64 + nb:] == 9.0)
    assert np.all(d[:pad] == -3.0) and np.all(d[pad + n:] == -3.0)


def test_wrappers_check_buffers_before_launch(tfp8):
    # the C ABI takes bare pointers; the tensor wrappers check dtypes and element counts of every
    # buffer first, so a wrong one raises instead of being read or written past its end
    B, nb = 128, 4
    n = nb * B
    x = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    u8 = lambda k: torch.zeros(k, dtype=torch.uint8, device=DEV)
    f32 = lambda k: torch.zeros(k, dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError, match="block"):
        tfp8.compress(x, 96)
    with pytest.raises(ValueError, match="multiple"):
        tfp8.compress(x[:n - 2], B)
    with pytest.raises(ValueError, match="alpha"):
        tfp8.compress(x, B, out=(u8(n), f32(nb - 1), f32(nb)))
    with pytest.raises(ValueError, match="codes"):
        tfp8.compress(x, B, out=(f32(n), f32(nb), f32(nb)))
    with pytest.raises(ValueError, match="scale"):
        tfp8.decompress(u8(n), f32(nb), f32(nb - 1), B)
    with pytest.raises(ValueError, match="out"):
        tfp8.decompress(u8(n), f32(nb), f32(nb), B, torch.float32, out=f32(n - 1))
    with pytest.raises(ValueError, match="out"):
        tfp8.decompress(u8(n), f32(nb), f32(nb), B, torch.float32,
                        out=torch.zeros(n, dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="stacked"):
        tfp8.reduce_fp8(u8(n), f32(nb), f32(nb), B)
    with pytest.raises(ValueError, match="alpha"):
        tfp8.reduce_fp8(u8(2 * n).view(2, n), f32(nb), f32(2 * nb), B)
    with pytest.raises(ValueError, match="codes_out"):
        tfp8.reduce_fp8(u8(2 * n).view(2, n), f32(2 * nb), f32(2 * nb), B,
                        out=(u8(n + 16), f32(nb), f32(nb)))
    with pytest.raises(ValueError, match="same number"):
        tfp8.accumulate(u8(n), f32(nb), f32(nb), x[:n - B], B)
    with pytest.raises(ValueError, match="scale_out"):
        tfp8.accumulate(u8(n), f32(nb), f32(nb), x, B, out=(u8(n), f32(nb), f32(nb + 1)))
    with pytest.raises(ValueError, match="contiguous"):
        tfp8.decompress(u8(2 * n)[::2], f32(nb), f32(nb), B)
    with pytest.raises(ValueError, match="not both"):
        tfp8.accumulate(u8(n), f32(nb), f32(nb), x, B, out=(u8(n), f32(nb), f32(nb)),
                        inplace=True)
    torch.cuda.synchronize()


def test_graph_capture_replays_match_eager(tfp8):
    # The calls allocate nothing and never synchronize, so a stream can capture them in a graph.
    # compress -> reduce_fp8 -> decompress and an accumulate are captured once, then replayed
    # three times with eager work in between (outputs overwritten, a new input copied in); each
    # replay must equal the eager calls on the same input bit for bit.
    B, P, n = 128, 4, 1 << 18
    nb = n // B
    inputs = [bits_to_gpu(np.concatenate([random_bf16_bits(n, seed=40 * k + p, scale=0.05)
                                          for p in range(P)])) for k in range(3)]
    grads = [bits_to_gpu(random_bf16_bits(n, seed=900 + k, scale=0.02)) for k in range(3)]

    def eager(x, g):
        q, a, s = tfp8.compress(x, B, 1.0)
        rq, ra, rs = tfp8.reduce_fp8(q.view(P, n), a.view(P, nb), s.view(P, nb), B, 1.0)
        d = tfp8.decompress(rq, ra, rs, B, torch.bfloat16)
        aq, aa, as_ = tfp8.accumulate(rq, ra, rs, g, B, 1.0)
        return [q, a, s, rq, ra, rs, d, aq, aa, as_]

    x_in = torch.empty_like(inputs[0])
    g_in = torch.empty_like(grads[0])
    outs = [torch.empty(P * n, dtype=torch.uint8, device=DEV), torch.empty(P * nb, device=DEV),
            torch.empty(P * nb, device=DEV), torch.empty(n, dtype=torch.uint8, device=DEV),
            torch.empty(nb, device=DEV), torch.empty(nb, device=DEV),
            torch.empty(n, dtype=torch.bfloat16, device=DEV),
            torch.empty(n, dtype=torch.uint8, device=DEV), torch.empty(nb, device=DEV),
            torch.empty(nb, device=DEV)]

    def pipeline():
        q, a, s, rq, ra, rs, d, aq, aa, as_ = outs
        tfp8.compress(x_in, B, 1.0, out=(q, a, s))
        tfp8.reduce_fp8(q.view(P, n), a.view(P, nb), s.view(P, nb), B, 1.0, out=(rq, ra, rs))
        tfp8.decompress(rq, ra, rs, B, torch.bfloat16, out=d)
        tfp8.accumulate(rq, ra, rs, g_in, B, 1.0, out=(aq, aa, as_))

    x_in.copy_(inputs[0])
    g_in.copy_(grads[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pipeline()  # one eager run on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pipeline()
    torch.cuda.synchronize()
    for k in range(3):
        for t in outs:
            t.view(torch.uint8).fill_(0xA5)
        x_in.copy_(inputs[k])
        g_in.copy_(grads[k])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = eager(inputs[k], grads[k])
        torch.cuda.synchronize()
        for i, (got, ref) in enumerate(zip(outs, want)):
            assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), (k, i)
    say("  graph: 3 replays equal the eager calls")


def test_bitwise_deterministic_and_stream_safe(tfp8):
    x = bits_to_gpu(make_shard(GPT2_7B).reshape(-1))
    r1 = tfp8.compress(x, 128, 1.0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        r2 = tfp8.compress(x, 128, 1.0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for u, v in zip(r1, r2):
        assert torch.equal(u, v)


def test_concurrent_host_threads(tfp8):
    # The header allows calls from several host threads at once (the library keeps no state
    # beyond a per-device CU count).  Four threads each run compress -> reduce_fp8 (P = 2) ->
    # decompress 25 times on their own stream and buffers, concurrently (ctypes releases the
    # GIL during the calls); every result must equal the same pipeline run alone.
    import threading

    B, n, T = 128, WORKLOADS[GPT2_7B].n, 1.0
    nb = n // B
    jobs = []
    for t in range(4):
        x = bits_to_gpu(np.stack([make_shard(GPT2_7B, 2 * t + k).reshape(-1) for k in range(2)]))
        bufs = dict(x=x.reshape(-1), q=torch.empty(2 * n, dtype=torch.uint8, device=DEV),
                    a=torch.empty(2 * nb, dtype=torch.float32, device=DEV),
                    s=torch.empty(2 * nb, dtype=torch.float32, device=DEV),
                    rq=torch.empty(n, dtype=torch.uint8, device=DEV),
                    ra=torch.empty(nb, dtype=torch.float32, device=DEV),
                    rs=torch.empty(nb, dtype=torch.float32, device=DEV),
                    out=torch.empty(n, dtype=torch.bfloat16, device=DEV))
        jobs.append(bufs)

    def pipeline(b, stream):
        assert tfp8.compress_raw(b["x"].data_ptr(), tfp8.BF16, 2 * n, B, T, b["q"].data_ptr(),
                                 b["a"].data_ptr(), b["s"].data_ptr(), stream) == 0
        assert tfp8.reduce_fp8_raw(b["q"].data_ptr(), b["a"].data_ptr(), b["s"].data_ptr(), 2, n,
                                   B, T, b["rq"].data_ptr(), b["ra"].data_ptr(),
                                   b["rs"].data_ptr(), stream) == 0
        assert tfp8.decompress_raw(b["rq"].data_ptr(), b["ra"].data_ptr(), b["rs"].data_ptr(), n,
                                   B, b["out"].data_ptr(), tfp8.BF16, stream) == 0

    alone = []
    for b in jobs:
        pipeline(b, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        alone.append({k: v.clone() for k, v in b.items() if k != "x"})
        for k in ("q", "rq", "out"):
            b[k].zero_()
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream() for _ in jobs]
    errors = []

    def worker(b, st):
        try:
            for _ in range(25):
                pipeline(b, st.cuda_stream)
        except Exception as e:  # reported after join
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(b, st)) for b, st in zip(jobs, streams)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for b, ref in zip(jobs, alone):
        for k, v in ref.items():
            assert torch.equal(b[k].view(torch.uint8) if b[k].dtype == torch.bfloat16 else b[k],
                               v.view(torch.uint8) if v.dtype == torch.bfloat16 else v), k


def _view_at(numel, byte_offset, dtype):
    """A contiguous GPU view of `numel` elements starting `byte_offset` bytes past the start of a
    fresh (256-byte aligned) allocation."""
    esz = torch.empty(0, dtype=dtype).element_size()
    assert byte_offset % esz == 0
    big = torch.empty(numel + 256 // esz, dtype=dtype, device=DEV)
    v = big[byte_offset // esz:byte_offset // esz + numel]
    assert v.data_ptr() % 256 == byte_offset
    return v


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B", [64, 128, 256, 512])
def test_buffers_at_minimal_alignment(oracle, tfp8, B, dtype):
    # Every buffer at the smallest alignment the header allows, as views into larger
    # allocations: inputs 48 bytes past a 256-byte boundary (so not 32-byte aligned either),
    # codes and reconstructions 16 bytes past one, alpha and s 4 bytes past one.  Every result
    # must equal that of the same call on fresh, 256-byte aligned buffers bit for bit; compress
    # is also held to the oracle.
    nb, P = 77, 3  # 77 blocks: a ragged last tile at every B
    n = nb * B
    rng = np.random.default_rng(4242 + B)
    v = rng.laplace(0.0, 0.02, (P, n))
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    if dtype == "f32":
        host = v.astype(np.float32)
        xs = torch.from_numpy(host).to(DEV)
    else:
        host = f32_to_bf16_bits(v.astype(np.float32))
        xs = torch.from_numpy(host.view(np.int16)).to(DEV).view(torch.bfloat16)

    def odd_x(t):
        xv = _view_at(t.numel(), 48, tdt)
        xv.copy_(t.reshape(-1))
        return xv

    def odd_codes(count, p=1):
        return (_view_at(p * count, 16, torch.uint8).view(p, count) if p > 1 else
                _view_at(count, 16, torch.uint8))

    def odd_scales(count, p=1):
        t = _view_at(p * count, 4, torch.float32)
        return t.view(p, count) if p > 1 else t

    # compress of each contribution, on aligned and on offset buffers
    stacks = [odd_codes(n, P), odd_scales(nb, P), odd_scales(nb, P)]
    for p in range(P):
        ref = tfp8.compress(xs[p], B, 1.0)
        got = tfp8.compress(odd_x(xs[p]), B, 1.0,
                            out=(stacks[0][p], stacks[1][p], stacks[2][p]))
        torch.cuda.synchronize()
        for g, r in zip(got, ref):
            assert torch.equal(g.view(-1), r.view(-1)), f"compress B={B} {dtype} shard {p}"
    qr, ar, sr, tr = oracle.compress(host[0], B, 1.0, with_quot=True)
    # admissibility only: one tie would exceed 1e-4 of these 77 blocks
    assert_codes_match(cpu(stacks[0][0]), qr, tr, max_frac=1.0, what=f"offset compress B={B}")
    assert_scales(cpu(stacks[1][0]), cpu(stacks[2][0]), ar, sr, what=f"offset compress B={B}")

    # decompress, both output dtypes
    for odt in (torch.float32, torch.bfloat16):
        ref = tfp8.decompress(stacks[0][0].clone(), stacks[1][0].clone(), stacks[2][0].clone(),
                              B, odt)
        out = _view_at(n, 16, odt)
        tfp8.decompress(stacks[0][0], stacks[1][0], stacks[2][0], B, odt, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16 if odt == torch.bfloat16 else torch.int32),
                           ref.view(torch.int16 if odt == torch.bfloat16 else torch.int32)), \
            f"decompress B={B} {odt}"

    # reduce of the three, contiguous stacks at offsets, outputs at offsets
    ref = tfp8.reduce_fp8(stacks[0].clone(), stacks[1].clone(), stacks[2].clone(), B, 1.0)
    outs = (odd_codes(n), odd_scales(nb), odd_scales(nb))
    tfp8.reduce_fp8(stacks[0], stacks[1], stacks[2], B, 1.0, out=outs)
    torch.cuda.synchronize()
    for g, r in zip(outs, ref):
        assert torch.equal(g, r), f"reduce B={B} {dtype}"

    # accumulate in place on the offset buffers, against out of place on aligned ones
    grad = odd_x(xs[1])
    ref = tfp8.accumulate(outs[0].clone(), outs[1].clone(), outs[2].clone(), xs[1].clone(), B, 1.0)
    tfp8.accumulate(outs[0], outs[1], outs[2], grad, B, 1.0, inplace=True)
    torch.cuda.synchronize()
    for g, r in zip(outs, ref):
        assert torch.equal(g, r), f"accumulate B={B} {dtype}"


def test_zero_length_is_noop(tfp8):
    x = torch.empty(0, dtype=torch.bfloat16, device=DEV)
    q, a, s = tfp8.compress(x, 128, 1.0)
    assert q.numel() == 0 and a.numel() == 0


# ----------------------------------------------------------------------------- variants

VARIANTS = [1, 2, 3]  # INT8 codes, no rotation, both


@pytest.mark.parametrize("flags", VARIANTS)
@pytest.mark.parametrize("key", [TINY, GPT2_7B])
def test_variant_workloads(oracle, tfp8, key, flags):
    wl = WORKLOADS[key]
    x = make_shard(key).reshape(-1)
    q, a, s = check_compress(oracle, tfp8, x, wl.block, what=f"{key} compress", flags=flags)
    check_decompress(oracle, tfp8, q, a, s, wl.block, what=f"{key} decompress", flags=flags)


@pytest.mark.parametrize("flags", VARIANTS)
@pytest.mark.parametrize("B", [64, 128, 256, 512])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_variant_edge_blocks(oracle, tfp8, B, dtype, flags):
    rng = np.random.default_rng(B + 7)
    v = np.concatenate([_special_blocks(B, rng), rng.laplace(0, 0.05, 5 * B)])
    x = f32_to_bf16_bits(v.astype(np.float32)) if dtype == "bf16" else v.astype(np.float32)
    q, a, s = check_compress(oracle, tfp8, x, B, what=f"edge B={B} {dtype}", flags=flags)
    check_decompress(oracle, tfp8, q, a, s, B, what=f"edge B={B} {dtype}", flags=flags)


@pytest.mark.parametrize("flags", VARIANTS)
@pytest.mark.parametrize("P,B", [(1, 128), (3, 64), (8, 128), (4, 256), (5, 512)])
def test_variant_reduce(oracle, tfp8, P, B, flags):
    rng = np.random.default_rng(100 * P + B + flags)
    nb = 29
    xs = [f32_to_bf16_bits((rng.laplace(0, 0.02, nb * B) * (1 + p)).astype(np.float32))
          for p in range(P)]
    for p in range(P):
        xs[p][3 * B:4 * B] = 0
        xs[p][6 * B:7 * B] = f32_to_bf16_bits(
            (rng.integers(-64, 65, B) * 2.0 ** -133).astype(np.float32))
    enc = [oracle.compress(x, B, 1.0, flags=flags) for x in xs]
    q = np.stack([e[0] for e in enc]); a = np.stack([e[1] for e in enc]); s = np.stack([e[2] for e in enc])
    cq, ca, cs = check_reduce(oracle, tfp8, q, a, s, B, what=f"reduce P={P} B={B}", flags=flags)
    check_decompress(oracle, tfp8, cq, ca, cs, B, what=f"reduced P={P} B={B}", flags=flags)


# ----------------------------------------------------------------------------- accumulate

def _check_accumulate(oracle, tfp8, q, a, s, g, B, what, flags=0, inplace=False, T=1.0,
                      tie_ledger=None, block_mask=None, mask_ledger=None):
    from gpu_helpers import _count_in_blocks
    from tiecheck import FLAG_INT8, tie_cap

    gg = bits_to_gpu(g) if g.dtype == np.uint16 else f32_to_gpu(g)
    qg, ag, sg = u8_to_gpu(q), f32_to_gpu(a), f32_to_gpu(s)
    cq, ca, cs = tfp8.accumulate(qg, ag, sg, gg, B, T, flags=flags, inplace=inplace)
    torch.cuda.synchronize()
    if inplace:
        assert cq.data_ptr() == qg.data_ptr()
    cq, ca, cs = cpu(cq), cpu(ca), cpu(cs)
    rq, ra, rs, rt = oracle.accumulate(q, a, s, g, B, T, with_quot=True, flags=flags)
    nmis = assert_codes_match(cq, rq, rt, max_frac=tie_cap(flags) if tie_ledger is None else 1.0,
                              what=what + " codes", int8=bool(flags & FLAG_INT8))
    if tie_ledger is not None:
        tie_ledger.append((flags, nmis, cq.size))
    _count_in_blocks(cq, rq, B, block_mask, flags, mask_ledger)
    ea, es = assert_scales(ca, cs, ra, rs, what=what)
    say(f"  {what}: n={q.size} B={B} flags={flags} inplace={inplace}: code tie mismatches {nmis} "
        f"({nmis / q.size:.2e}), max rel err alpha {ea:.2e} scale {es:.2e}")
    return cq, ca, cs


def test_accumulate_gradient_workload(oracle, tfp8):
    # the GPT-13B-shaped gradient workload: main gradient = shard 0 compressed, local = shard 1
    wl = WORKLOADS[GPT13B_GRAD]
    B = wl.block
    x0, x1 = make_shard(GPT13B_GRAD, 0).reshape(-1), make_shard(GPT13B_GRAD, 1).reshape(-1)
    q, a, s = oracle.compress(x0, B, 1.0)
    _check_accumulate(oracle, tfp8, q, a, s, x1, B, "gpt13b-grad accumulate")
    _check_accumulate(oracle, tfp8, q, a, s, x1, B, "gpt13b-grad accumulate in place", inplace=True)


@pytest.mark.parametrize("flags", [0, 1])
def test_accumulate_micro_batch_chain(oracle, tfp8, flags):
    # Gradient accumulation over K = 6 micro-batches as AGoQ uses it: the first GPT-13B-shaped
    # gradient compressed, each later one added in place to the compressed main gradient, then the
    # result decompressed; on the GPU with its own outputs throughout, and in the oracle.  The two
    # chains separate only where a step admitted a rounding tie (a tie moves one code by one step,
    # and the next step carries it on), so the final codes must agree but for a small fraction,
    # and both reconstructions must be equally close to the exact sum of the K gradients.
    wl = WORKLOADS[GPT13B_GRAD]
    B, K, T = wl.block, 6, 1.0
    gs = make_shards(GPT13B_GRAD, count=K).reshape(K, -1)
    n = gs.shape[1]
    say(f"{GPT13B_GRAD}: {K} micro-batch gradients of {n} elements, block {B}, flags {flags}")
    q, a, sc = tfp8.compress(bits_to_gpu(gs[0]), B, T, flags=flags)
    for k in range(1, K):
        tfp8.accumulate(q, a, sc, bits_to_gpu(gs[k]), B, T, inplace=True, flags=flags)
    out = tfp8.decompress(q, a, sc, B, torch.float32, flags=flags)
    torch.cuda.synchronize()
    q, a, sc, out = cpu(q), cpu(a), cpu(sc), cpu(out).astype(np.float64)
    qr, ar, sr = oracle.compress(gs[0], B, T, flags=flags)
    for k in range(1, K):
        qr, ar, sr = oracle.accumulate(qr, ar, sr, gs[k], B, T, flags=flags)
    ref = oracle.decompress(qr, ar, sr, B, np.float32, flags=flags).astype(np.float64)
    z = np.zeros(n)
    for k in range(K):
        z += bf16_bits_to_f32(gs[k]).astype(np.float64)
    zn = np.sqrt(np.dot(z, z))
    e_gpu = np.sqrt(np.dot(out - z, out - z)) / zn
    e_ref = np.sqrt(np.dot(ref - z, ref - z)) / zn
    d = np.sqrt(np.dot(out - ref, out - ref)) / zn
    frac = float((q != qr).mean())
    ra_err = float(np.max(np.abs(a.astype(np.float64) - ar) / ar))
    say(f"  micro-batch chain: final codes differing {frac:.2e}, max rel diff alpha {ra_err:.2e}; "
        f"rel L2 error vs the exact sum: GPU chain {e_gpu:.6e}, oracle chain {e_ref:.6e}; "
        f"rel L2 difference between the chains {d:.2e}")
    # K - 1 steps, each admitting ties on at most 1e-4 of the elements, carried forward
    assert frac <= K * 1e-4, frac
    assert abs(e_gpu - e_ref) <= 1e-3 * e_ref, (e_gpu, e_ref)


@pytest.mark.parametrize("flags", [0, 1, 2, 3])
@pytest.mark.parametrize("B", [64, 128, 256, 512])
@pytest.mark.parametrize("gdtype", ["bf16", "f32"])
def test_accumulate_edges(oracle, tfp8, B, gdtype, flags):
    rng = np.random.default_rng(B + flags)
    main = np.concatenate([_special_blocks(B, rng), rng.laplace(0, 0.05, 3 * B)])
    local = rng.laplace(0, 0.03, main.size)
    local[:B] = 0                               # zero local gradient on a zero main block
    local[2 * B:3 * B] = 0                      # zero local gradient on a nonzero block
    local[5 * B:6 * B] *= 2.0 ** -130           # tiny local gradient on the subnormal block
    xm = f32_to_bf16_bits(main.astype(np.float32))
    q, a, s = oracle.compress(xm, B, 1.0, flags=flags)
    g = f32_to_bf16_bits(local.astype(np.float32)) if gdtype == "bf16" else local.astype(np.float32)
    _check_accumulate(oracle, tfp8, q, a, s, g, B, f"accumulate B={B} {gdtype}", flags=flags)


@pytest.mark.parametrize("flags", [0, 1, 2, 3])
@pytest.mark.parametrize("B", [64, 128, 256, 512])
def test_accumulate_exact_cancellation(oracle, tfp8, B, flags):
    # Main gradients whose reconstruction is exact in float32 (codes 0 or +-Q, alpha = Q' 2^e
    # with Q' the odd part of Q, s a power of two; exact at every B without the rotation and at
    # B = 64, 256 with it, where sqrt(B) is a power of two), and local gradients that are exactly
    # their negatives: the sum is exactly zero, so the result is a zero block.  Half of the
    # blocks get one small extra term, so that their sum is a one-hot block far below either
    # term.  A kernel that forms the main term with any error of its own leaves a residue of
    # that size instead, which the codes of the sum magnify to full scale.  At B = 128, 512 with
    # the rotation the float32 negative differs from the reconstruction by its rounding error,
    # which then is the whole sum.
    from tiecheck import FLAG_INT8
    rng = np.random.default_rng(9000 + B + flags)
    nb = 96
    int8 = bool(flags & FLAG_INT8)
    qmax, odd = (127, 127) if int8 else (448, 7)
    pos, neg = (0x7F, 0x81) if int8 else (0x7E, 0xFE)
    pick = rng.choice(3, size=(nb, B), p=[0.6, 0.2, 0.2])
    q = np.where(pick == 1, pos, np.where(pick == 2, neg, 0)).astype(np.uint8)
    q[np.arange(nb), rng.integers(0, B, nb)] = pos           # every block reaches Q
    a = (odd * 2.0 ** rng.integers(-10, 11, nb)).astype(np.float32)
    s = (2.0 ** rng.integers(-10, 11, nb)).astype(np.float32)
    main = oracle.decompress_f64(q.reshape(-1), a, s, B, flags=flags).reshape(nb, B)
    g = -main.astype(np.float32)
    bump = np.arange(nb) % 2 == 1
    k = rng.integers(0, B, nb)
    g[bump, k[bump]] += (np.abs(main[bump]).max(axis=1) * 2.0 ** -20).astype(np.float32)
    exact = (flags & 2) or B in (64, 256)
    if exact:
        assert np.array_equal(g[~bump].astype(np.float64), -main[~bump])
    # where the sum is the rounding error of the negative, its codes fall on midpoints more often
    # than the tie cap (made for the workloads) allows: there only admissibility is checked
    cq, ca, cs = _check_accumulate(oracle, tfp8, q.reshape(-1), a, s, g.reshape(-1), B,
                                   f"exact cancellation B={B} flags={flags}", flags=flags,
                                   tie_ledger=None if exact else [])
    if exact:
        assert np.all(cs[~bump] == 0) and np.all(cq.reshape(nb, B)[~bump] == 0)
        bumped = cq.reshape(nb, B)[bump]
        if flags & 2:   # a one-hot sum keeps one code
            assert np.all(np.count_nonzero(bumped, axis=1) == 1)
        else:           # and rotates to a Hadamard row: every code is +-Q
            assert np.all(np.isin(bumped, [pos, neg]))


def test_accumulate_activation_shards_with_shared_outliers(oracle, tfp8):
    # the Qwen2.5-7B-shaped activation shards 0 and 1 as main and local gradient: their shared
    # outlier channels have random signs, so about 15% of the blocks cancel and take the exact
    # split path; full size, every element compared
    wl = WORKLOADS[QWEN7B]
    xs = make_shards(QWEN7B, count=2).reshape(2, -1)
    q, a, s = oracle.compress(xs[0], wl.block, 1.0)
    _check_accumulate(oracle, tfp8, q, a, s, xs[1], wl.block, "qwen shards accumulate")


@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("flags", [0, 1])
@pytest.mark.parametrize("B,gdtype", [(128, "bf16"), (256, "f32"), (64, "bf16")])
def test_accumulate_cancelling_blocks(oracle, tfp8, B, gdtype, flags, inplace):
    # local gradient ~ minus the main gradient on most blocks, so that the sum is about the main
    # gradient's quantisation error: those blocks take the float64 path, many per 64-block scan
    # tile (more than eight, so the tile is worked through in several rounds), over several
    # tiles and a ragged last one (nb = 3 * 64 + 11)
    rng = np.random.default_rng(1000 + B + 7 * flags + inplace)
    nb = 3 * 64 + 11
    main = rng.laplace(0, 0.05, nb * B)
    main[5 * B + 3] = 40.0                                   # one outlier block
    xm = f32_to_bf16_bits(main.astype(np.float32))
    q, a, s = oracle.compress(xm, B, 1.0, flags=flags)
    local = -bf16_bits_to_f32(xm).astype(np.float64) + rng.normal(0, 1e-4, nb * B)
    keep = rng.random(nb) < 0.25                             # blocks that do not cancel
    keep[64:64 + 20] = False                                 # a tile with 20+ cancelling blocks
    local.reshape(nb, B)[keep] = rng.laplace(0, 0.03, (int(keep.sum()), B))
    g = f32_to_bf16_bits(local.astype(np.float32)) if gdtype == "bf16" else local.astype(np.float32)
    _check_accumulate(oracle, tfp8, q, a, s, g, B, f"cancelling B={B} {gdtype}", flags=flags,
                      inplace=inplace)


@pytest.mark.parametrize("B", [64, 128, 256, 512])
def test_accumulate_each_output_in_place_or_not(oracle, tfp8, B):
    # Each of codes_out, alpha_out and scale_out may be its input or a separate buffer.  The exact
    # pass reads the codes, s and the set-aside marks (-alpha in alpha_out) back, so every one of
    # the 8 combinations is run on blocks that cancel (most of them take that pass) and must equal
    # the out-of-place call bit for bit.
    rng = np.random.default_rng(8080 + B)
    nb = 2 * 64 + 5
    xm = f32_to_bf16_bits(rng.laplace(0, 0.05, nb * B).astype(np.float32))
    q, a, s = oracle.compress(xm, B, 1.0)
    local = -bf16_bits_to_f32(xm).astype(np.float64) + rng.normal(0, 1e-4, nb * B)
    keep = rng.random(nb) < 0.3
    local.reshape(nb, B)[keep] = rng.laplace(0, 0.03, (int(keep.sum()), B))
    gg = bits_to_gpu(f32_to_bf16_bits(local.astype(np.float32)))
    ref = tfp8.accumulate(u8_to_gpu(q), f32_to_gpu(a), f32_to_gpu(s), gg, B, 1.0)
    torch.cuda.synchronize()
    ref = [cpu(t) for t in ref]
    for combo in range(8):
        ins = [u8_to_gpu(q), f32_to_gpu(a), f32_to_gpu(s)]
        outs = [ins[i] if combo >> i & 1 else torch.empty_like(ins[i]) for i in range(3)]
        st = tfp8.accumulate_raw(ins[0].data_ptr(), ins[1].data_ptr(), ins[2].data_ptr(),
                                 gg.data_ptr(), tfp8.BF16, q.size, B, 1.0, outs[0].data_ptr(),
                                 outs[1].data_ptr(), outs[2].data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
        assert st == 0, tfp8.status_string(st)
        torch.cuda.synchronize()
        for o, r, name in zip(outs, ref, ("codes", "alpha", "scale")):
            assert np.array_equal(cpu(o), r), f"B={B} in-place mask {combo:03b}: {name} differ"
    # and the out-of-place result against the oracle
    _check_accumulate(oracle, tfp8, q, a, s, f32_to_bf16_bits(local.astype(np.float32)), B,
                      f"in-place combinations B={B}")


def test_accumulate_zero_main_gradient_equals_compress(oracle, tfp8):
    B, nb = 128, 77
    g = random_bf16_bits(nb * B, seed=12, scale=0.2)
    q = np.zeros(nb * B, np.uint8); a = np.ones(nb, np.float32); s = np.zeros(nb, np.float32)
    cq, ca, cs = _check_accumulate(oracle, tfp8, q, a, s, g, B, "accumulate onto zero")
    # the oracle's compress of the same gradient is the expected value as well
    rq, ra, rs, rt = oracle.compress(g, B, 1.0, with_quot=True)
    assert_codes_match(cq, rq, rt, what="accumulate onto zero vs compress")
    assert_scales(ca, cs, ra, rs, what="accumulate onto zero vs compress")
    check_compress(oracle, tfp8, g, B, what="compress of the same gradient")


def _seven_parts(tile, seed, dtype="bf16"):
    """Seven independent random tiles of `tile` elements, part w scaled by 2^(w - 3), as
    bfloat16 bits or float32.  A block read from another tile differs in its codes as well as
    in alpha: a power-of-two scaling of one tile would change alpha alone and leave the codes
    identical."""
    parts = []
    for w in range(7):
        if dtype == "f32":
            rng = np.random.default_rng(seed + w)
            parts.append((rng.standard_normal(tile) * (0.05 * 2.0 ** (w - 3))).astype(np.float32))
        else:
            v = bf16_bits_to_f32(random_bf16_bits(tile, seed=seed + w, scale=0.05))
            parts.append(f32_to_bf16_bits(v * np.float32(2.0 ** (w - 3))))
    return parts


def _tiled_input(scaled, n, tile):
    """Tile t of the input is scaled[t mod 7] (the last one cut to what is left of n)."""
    x = np.empty(n, scaled[0].dtype)
    for t in range(-(-n // tile)):
        seg = x[t * tile:(t + 1) * tile]
        seg[:] = scaled[t % 7][:seg.size]
    return x


def _check_tiled_compress_every_block(oracle, q, a, s, scaled, n, tile, B, flags, what):
    """Compress output of a _tiled_input checked on every block: block k lies in tile
    kB // tile, which is scaled[tile mod 7], so its expected codes, scales and quotients are those
    of the oracle's compress of the seven scaled tiles, gathered by index (no arithmetic)."""
    from tiecheck import FLAG_INT8, tie_cap

    nb, bpt = n // B, tile // B
    refs = [oracle.compress(v, B, 1.0, with_quot=True, flags=flags) for v in scaled]
    rq = np.stack([r[0] for r in refs]).reshape(7 * bpt, B)
    ra = np.concatenate([r[1] for r in refs])
    rs = np.concatenate([r[2] for r in refs])
    rt = np.stack([r[3] for r in refs]).reshape(7 * bpt, B)
    k = np.arange(nb, dtype=np.int64)
    src = (k // bpt % 7) * bpt + k % bpt  # row of the seven tiles' outputs that block k equals
    nmis = assert_codes_match_every_block(
        cpu(q).reshape(nb, B), rq[src], B, lambda idx: rt[src[idx]], max_frac=tie_cap(flags),
        what=what, int8=bool(flags & FLAG_INT8))
    assert_scales(cpu(a), cpu(s), ra[src], rs[src], what=what)
    return nmis


@pytest.mark.parametrize("dtype,B,extra_blocks", [("bf16", 128, -3), ("bf16", 128, 13),
                                                  ("f32", 128, 5), ("bf16", 64, -3),
                                                  ("bf16", 64, 13), ("f32", 64, 5)])
def test_compress_both_launch_shapes(oracle, tfp8, dtype, B, extra_blocks):
    # Compress picks its launch shape by input size: below 1.5 GiB four wavefronts per
    # workgroup in dispatch order, from 1.5 GiB one wavefront per workgroup with each XCD on a
    # contiguous eighth of the tiles (grid rounded up to a multiple of 8).  Inputs just below
    # and above the switch, each with a ragged last tile (block count not a multiple of 8).  The
    # input repeats seven random tiles of 2^20 elements, so a block read from the wrong place
    # shows; every block is checked.  At B = 64 a tile is 16 blocks, a pair per lane group, and
    # an odd block count leaves the last pair with one block.
    tile = 1 << 20
    esize = 2 if dtype == "bf16" else 4
    nb = (3 << 29) // esize // B + extra_blocks
    n = nb * B
    scaled = _seven_parts(tile, 1536, dtype)
    x = _tiled_input(scaled, n, tile)
    say(f"  launch shapes: {dtype}, {n * esize / 2**30:.4f} GiB of input, nb = {nb}, every block")
    xg = (bits_to_gpu(x) if dtype == "bf16" else f32_to_gpu(x))
    del x
    q, a, s = tfp8.compress(xg, B, 1.0)
    torch.cuda.synchronize()
    del xg
    what = f"launch shapes {dtype} B={B} {nb} blocks"
    nmis = _check_tiled_compress_every_block(oracle, q, a, s, scaled, n, tile, B, 0, what)
    say(f"  {what}: tie mismatches {nmis} ({nmis / n:.2e})")


def test_compress_large_input_every_block_size_and_variant(oracle, tfp8):
    # Inputs of 1.5 GiB or more take the remapped launch at every block size.  One 1.6 GB bf16
    # input, prefixes of it for every block size (each with a ragged last tile), and every flag
    # set at B = 128 and B = 64; every block checked.
    tile = 1 << 20
    n_all = ((3 << 29) // 2 // 128 + 13) * 128
    scaled = _seven_parts(tile, 1537)
    xg = bits_to_gpu(_tiled_input(scaled, n_all, tile))
    cases = [(64, 0), (256, 0), (512, 0), (128, 1), (128, 2), (128, 3), (64, 2), (64, 1)]
    for B, flags in cases:
        nb = n_all // B
        n = nb * B
        assert n * 2 >= 3 << 29 and nb % (64 // (4 if B == 64 else 8)) != 0
        q, a, s = tfp8.compress(xg[:n], B, 1.0, flags=flags)
        torch.cuda.synchronize()
        what = f"large input B={B} flags={flags}"
        nmis = _check_tiled_compress_every_block(oracle, q, a, s, scaled, n, tile, B, flags, what)
        say(f"  {what}: every block ({nb}), tie mismatches {nmis} ({nmis / n:.2e})")
        del q, a, s


# (block, input dtype, tiles of 2^22 elements).  At 513 tiles (2^31 + 2^22 - 37 B elements)
# element indexes pass 2^31, bfloat16 byte offsets 2^32, float32 ones 2^33 and code byte offsets
# 2^31, in the launches with a wavefront for every tile.  The larger cases pass the size at
# which the launches are capped at 2^30 work-items and their wavefronts loop over tiles,
# loading the next tile before working on the current one: 2^34 elements at B = 64 and 128
# (2^33 for decompress at B = 64), and 2^35 for compress, decompress and accumulate at B = 256.
# The reduce's tiles hold 1024 elements at every B, so it loops past 2^34 at B = 256 and 512
# too; at B = 512 the other three still launch a wavefront per tile there.
_LARGE_CASES = [(128, "bf16", 513), (64, "bf16", 513), (512, "bf16", 513), (128, "f32", 513),
                (128, "bf16", 4097), (64, "bf16", 4097), (128, "f32", 4097), (512, "bf16", 4097),
                (256, "bf16", 8193)]


def _large_input_every_block(oracle, tfp8, B, dtype, ntiles, flags=0, f32_out=True, reduce=True,
                             tile=1 << 22, seed=None, cancel=()):
    # n = ntiles * tile - 37 B elements (4.3-137 GB of input at tiles of 2^22, a ragged last
    # tile), built on the GPU from seven random tiles (tile t is part t mod 7), so that a read at
    # an offset cut to 32 bits (1024 tiles away for codes, 512 for bfloat16, 256 for float32)
    # or any other wrong place shows.  Compress, decompress to bfloat16 and (f32_out) float32,
    # the reduce (reduce) and accumulate each run on the whole tensor with the given variant
    # flags; every output block is checked against the oracle's output for its part.  The
    # accumulation's local gradient is the input with the parts in `cancel` negated: there it
    # cancels the main gradient down to its quantisation error, and the blocks go to the second
    # kernel.  No expected value comes from the GPU.
    T = 1.0
    n = ntiles * tile - 37 * B
    nb, bpt = n // B, tile // B
    f32 = dtype == "f32"
    # device memory at the largest step (input and codes; codes and a reconstruction; two rows
    # of codes, their sum and the codes), with a tenth to spare
    esize = 4 if f32 else 2
    peak = 1.1 * n * max(esize + 1, 1 + (4 if f32_out else 2), 4 if reduce else 0)
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info(DEV)
    if free < peak:
        pytest.skip(f"needs {peak / 1e9:.0f} GB of free device memory, {free / 1e9:.0f} GB free")
    variants = _seven_parts(tile, 2034 + 8 * B if seed is None else seed, dtype)
    enc = [oracle.compress(v, B, T, with_quot=True, flags=flags) for v in variants]
    say(f"  large input B={B} {dtype} flags={flags}: n = {n} ({n * (4 if f32 else 2) / 1e9:.1f} GB of "
        f"input), every block")

    def input_on_gpu(parts=variants):
        if f32:
            return fill_periodic(torch.empty(n, dtype=torch.float32, device=DEV), parts, tile)
        return fill_periodic(torch.empty(n, dtype=torch.int16, device=DEV),
                             [v.view(np.int16) for v in parts], tile).view(torch.bfloat16)

    def codes_on_gpu(parts):
        # the oracle's codes, alpha and s of the seven tiles, tiled like the input
        q = torch.empty(n, dtype=torch.uint8, device=DEV)
        a, s = (torch.empty(nb, dtype=torch.float32, device=DEV) for _ in range(2))
        return (fill_periodic(q, [e[0] for e in parts], tile),
                fill_periodic(a, [e[1] for e in parts], bpt),
                fill_periodic(s, [e[2] for e in parts], bpt))

    # compress
    x = input_on_gpu()
    q, a, s = tfp8.compress(x, B, T, flags=flags)
    torch.cuda.synchronize()
    del x
    torch.cuda.empty_cache()
    nmis, ea, es = assert_periodic_codes(q, a, s, enc, n, tile, B, what="large compress",
                                         flags=flags)
    del q, a, s
    torch.cuda.empty_cache()
    say(f"  large compress: tie mismatches {nmis}, max rel err alpha {ea:.2e} s {es:.2e}")

    # decompress of the oracle's codes, bfloat16 and float32
    qg, ag, sg = codes_on_gpu(enc)
    dec = [(e[0], e[1], e[2]) for e in enc]
    r64 = [oracle.decompress_f64(*d, B, flags=flags) for d in dec]
    outs = ((torch.bfloat16, np.uint16), (torch.float32, np.float32)) if f32_out else \
        ((torch.bfloat16, np.uint16),)
    for odt, ndt in outs:
        out = tfp8.decompress(qg, ag, sg, B, odt, flags=flags)
        torch.cuda.synchronize()
        refs = [(oracle.decompress(*d, B, ndt, flags=flags), r) for d, r in zip(dec, r64)]
        nt = assert_periodic_decompress(out, refs, n, tile, B, what=f"large decompress {odt}")
        del out
        torch.cuda.empty_cache()
        say(f"  large decompress {odt}: " + (f"bf16 tie mismatches {nt}" if nt or ndt == np.uint16
                                             else "every output within 1e-6"))
    del r64

    # reduce, P = 2: row 0 the tiled codes, row 1 the same tiles three parts on
    if reduce:
        sq = torch.empty((2, n), dtype=torch.uint8, device=DEV)
        sa = torch.empty((2, nb), dtype=torch.float32, device=DEV)
        ss = torch.empty((2, nb), dtype=torch.float32, device=DEV)
        sq[0], sa[0], ss[0] = qg, ag, sg
        other = [enc[(w + 3) % 7] for w in range(7)]
        fill_periodic(sq[1], [e[0] for e in other], tile)
        fill_periodic(sa[1], [e[1] for e in other], bpt)
        fill_periodic(ss[1], [e[2] for e in other], bpt)
        cq, ca, cs = tfp8.reduce_fp8(sq, sa, ss, B, T, flags=flags)
        torch.cuda.synchronize()
        del sq, sa, ss
        torch.cuda.empty_cache()
        refs = [oracle.reduce_fp8(np.stack([e[0], o[0]]), np.stack([e[1], o[1]]),
                                  np.stack([e[2], o[2]]), B, T, with_quot=True, flags=flags)
                for e, o in zip(enc, other)]
        nmis, ea, es = assert_periodic_codes(cq, ca, cs, refs, n, tile, B, what="large reduce",
                                             flags=flags)
        del cq, ca, cs
        torch.cuda.empty_cache()
        say(f"  large reduce: tie mismatches {nmis}, max rel err alpha {ea:.2e} s {es:.2e}")

    # accumulate in place: main gradient = the tiled codes, local gradient = the input, with the
    # parts in `cancel` negated (the sign bit flipped: exact in both types)
    local = [(v ^ np.uint16(0x8000) if v.dtype == np.uint16 else -v) if w in cancel else v
             for w, v in enumerate(variants)]
    x = input_on_gpu(local)
    tfp8.accumulate(qg, ag, sg, x, B, T, inplace=True, flags=flags)
    torch.cuda.synchronize()
    del x
    refs = [oracle.accumulate(e[0], e[1], e[2], v, B, T, with_quot=True, flags=flags)
            for e, v in zip(enc, local)]
    nmis, ea, es = assert_periodic_codes(qg, ag, sg, refs, n, tile, B,
                                         what="large accumulate", flags=flags)
    del qg, ag, sg
    torch.cuda.empty_cache()
    say(f"  large accumulate: tie mismatches {nmis}, max rel err alpha {ea:.2e} s {es:.2e}")


@pytest.mark.parametrize("B,dtype,ntiles", _LARGE_CASES)
def test_large_offsets_and_grid_stride_loops_every_block(oracle, tfp8, B, dtype, ntiles):
    _large_input_every_block(oracle, tfp8, B, dtype, ntiles)


# The looping forms of the variants (INT8 codes, the rotation left out, both) at B = 128, of both
# together at B = 64, 256 and 512, and of float32 input at B = 64 and 256 (past 2^34, 2^35 and
# 2^36 elements).
@pytest.mark.parametrize("B,dtype,ntiles,flags", [(128, "bf16", 4097, 1), (128, "bf16", 4097, 2),
                                                  (128, "bf16", 4097, 3), (64, "bf16", 4097, 3),
                                                  (256, "bf16", 8193, 3), (512, "bf16", 16385, 3),
                                                  (64, "f32", 4097, 0), (256, "f32", 8193, 0)])
def test_grid_stride_loops_variants_and_fp32_every_block(oracle, tfp8, B, dtype, ntiles, flags):
    big = ntiles > 8193  # 137 GB of input: no float32 reconstruction, no reduce (as at flags 0)
    _large_input_every_block(oracle, tfp8, B, dtype, ntiles, flags=flags, f32_out=not big,
                             reduce=not big)


def test_grid_stride_loops_at_block_512_every_block(oracle, tfp8):
    # At B = 512 the launches of compress, decompress and accumulate loop over tiles from 2^36
    # elements on: n = 16385 * 2^22 - 37 * 512 (137 GB of bfloat16).  Compress holds 206 GB at its
    # peak (input and codes), decompress to bfloat16 and accumulate as much; the float32
    # decompress (275 GB) and the reduce (its loop at B = 512 starts at 2^34 and is checked
    # above) are left out.  Like every case here it skips on a device without the memory.
    _large_input_every_block(oracle, tfp8, 512, "bf16", 16385, f32_out=False, reduce=False)


# The looping forms again, through a second build of the library with every launch capped at one
# workgroup per compute unit (tests/capped_build; the kernels compile to the same instructions,
# checked by tests/test_codegen_hazards.py).  At 2^24 - 37 B elements each wavefront works through
# 4-32 tiles in turn (compress at B = 512: 4092 tiles over 1024 wavefronts), against one or two in
# the cases above, at every block size, input type and flag set.  Parts 1 and 4 of the
# accumulation's local gradient cancel the main gradient, so its second kernel, grid-striding too,
# redoes two sevenths of the blocks.  The last cases pass the 1.5 GiB at which compress switches to
# one wavefront per workgroup with each XCD on a contiguous eighth of the tiles: its 256
# wavefronts then loop 388-3088 times, and the other kernels 97-1544 times.  Among them is float32
# input at B = 512, whose looping form the full build reaches only past 2^36 elements (275 GB).
_CAPPED_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "capped_build",
                           "libtfp8_capped.so")
_capped_cdll = []


def _capped():
    """The capped build, opened once and declared like the package's library."""
    import ctypes

    import fp8_compression_tensor_amd as m

    assert os.path.exists(_CAPPED_LIB), (f"{_CAPPED_LIB} is not built; run "
                                         "tests/capped_build/build.py (or __graft_entry__.build())")
    if not _capped_cdll:
        _capped_cdll.append(m._declare(ctypes.CDLL(_CAPPED_LIB)))
    return _capped_cdll[0]


@pytest.fixture
def capped(tfp8, monkeypatch):
    """The package, its calls routed through the capped build for the test's duration."""
    monkeypatch.setattr(tfp8, "_lib", _capped())
    yield tfp8


@pytest.mark.parametrize("B,dtype,flags", [(B, "bf16", f) for B in (64, 128, 256, 512)
                                           for f in (0, 1, 2, 3)] +
                                          [(B, "f32", f) for B in (64, 128, 256, 512)
                                           for f in (0, 3)])
def test_capped_launches_loop_every_block(oracle, capped, B, dtype, flags):
    _large_input_every_block(oracle, capped, B, dtype, 64, flags=flags, tile=1 << 18,
                             seed=3034 + 8 * B + flags, cancel=(1, 4))


def _random_codes(rng, P, n, B, flags):
    """Codes, alpha and s of P contributions drawn directly (any codes are valid reduce inputs):
    uniform codes without the E4M3 NaN patterns (INT8: without -128), alpha log-uniform in
    [2^-8, 2^8], s in [2^-10, 2^2]; block 1 of every contribution is a zero block and block 2 of
    contribution 0 is the exact negation of contribution 1's."""
    nb = n // B
    q = rng.integers(0, 256, (P, n), dtype=np.uint8)
    if flags & FLAG_INT8:
        q[q == 0x80] = 0x81
    else:
        q[(q & 0x7F) == 0x7F] = 0x7E
    a = (2.0 ** rng.uniform(-8, 8, (P, nb))).astype(np.float32)
    sc = (2.0 ** rng.uniform(-10, 2, (P, nb))).astype(np.float32)
    q[:, B:2 * B] = 0
    a[:, 1], sc[:, 1] = 1.0, 0.0
    if P > 1:
        neg = (-q[1, 2 * B:3 * B].astype(np.int8)).view(np.uint8) if flags & FLAG_INT8 else \
            q[1, 2 * B:3 * B] ^ 0x80
        q[0, 2 * B:3 * B] = neg
        a[0, 2], sc[0, 2] = a[1, 2], sc[1, 2]
    return q, a, sc


@pytest.mark.parametrize("B,P,flags", [(64, 3, 0), (128, 13, 1), (256, 13, 0), (512, 3, 1),
                                       (64, 64, 1), (256, 64, 0), (512, 64, 0)])
def test_capped_launches_reduce_any_P(oracle, tfp8, monkeypatch, B, P, flags):
    # The reduce's general form (any P, in chunks of 8) and its fixed-P forms through the capped
    # build: n = 2^22 - 37 B elements (2^21 at P = 64) make each of the 1024 wavefronts loop over
    # 2-4 tiles of 1024 elements.  Every output against the oracle, and bit for bit against the
    # full library (the grid only changes which wavefront takes which tile).
    rng = np.random.default_rng(7000 + 10 * B + P + flags)
    n = (1 << (21 if P == 64 else 22)) - 37 * B
    q, a, sc = _random_codes(rng, P, n, B, flags)
    full = tfp8.reduce_fp8(u8_to_gpu(q), f32_to_gpu(a), f32_to_gpu(sc), B, 1.0, flags=flags)
    with monkeypatch.context() as m:
        m.setattr(tfp8, "_lib", _capped())
        got = check_reduce(oracle, tfp8, q, a, sc, B, flags=flags, gpu=True,
                           what="capped reduce")
    torch.cuda.synchronize()
    for u, v in zip(got, full):
        assert np.array_equal(u, cpu(v)), "capped and full launches differ"


@pytest.mark.parametrize("B,P,pad,flags", [(128, 8, 0, 0), (64, 5, 65536 + 1024, 1),
                                           (512, 13, 16, 0)])
def test_capped_launches_reduce_strided_messages(oracle, tfp8, monkeypatch, B, P, pad, flags):
    # the strided reduce from one receive buffer of [codes | alpha | scale] messages, looping
    # over tiles in the capped build; bit for bit against the full library's contiguous call
    rng = np.random.default_rng(7500 + B + P)
    n = (1 << 22) - 37 * B
    nb = n // B
    q, a, sc = _random_codes(rng, P, n, B, flags)
    buf, qv, av, sv = _messages(list(zip(q, a, sc)), n, nb, pad)
    full = tfp8.reduce_fp8(u8_to_gpu(q), f32_to_gpu(a), f32_to_gpu(sc), B, 1.0, flags=flags)
    with monkeypatch.context() as m:
        m.setattr(tfp8, "_lib", _capped())
        got = tfp8.reduce_fp8(qv, av, sv, B, 1.0, flags=flags)
    torch.cuda.synchronize()
    for u, v in zip(got, full):
        assert torch.equal(u, v), "capped strided and full contiguous reduces differ"
    rq, ra, rs, rt = oracle.reduce_fp8(q, a, sc, B, 1.0, with_quot=True, flags=flags)
    nmis, nfb, ea, es = assert_reduce_matches(cpu(got[0]), cpu(got[1]), cpu(got[2]), rq, rt, ra,
                                              rs, a, sc, B, flags, tie_cap(flags),
                                              "capped strided reduce")
    say(f"  capped strided reduce B={B} P={P} pad={pad} flags={flags}: tie mismatches {nmis}"
        + (f", {nfb} in float64 noise" if nfb else ""))


@pytest.mark.parametrize("B,dtype,ntiles,flags", [(512, "f32", 97, 0), (512, "f32", 97, 3),
                                                  (64, "bf16", 193, 0), (256, "bf16", 193, 1)])
def test_capped_launches_remapped_loop_every_block(oracle, capped, B, dtype, ntiles, flags):
    n = ntiles * (1 << 22) - 37 * B
    assert n * (4 if dtype == "f32" else 2) >= 3 << 29  # compress's remapped launch shape
    _large_input_every_block(oracle, capped, B, dtype, ntiles, flags=flags,
                             seed=4034 + 8 * B + flags, cancel=(1, 4))


# The capped launches at the boundary of their loops.  A capped launch has W = 4 x (compute
# units) wavefronts.  Each kernel runs at three tile counts: W (one tile per wavefront, the last
# one short by a block: compress and decompress take their one-tile forms), W + 1 (wavefront 0
# takes a second tile holding a single block, loaded while it works on its first) and 2 W + 1
# (a third, ragged tile for wavefront 0).  The accumulation's second kernel scans 128 blocks per
# wavefront and iteration; at B = 64 and 128 it also runs at W + 1 scans, with set-aside blocks in
# wavefront 0's first and second scans, in the last scan of wavefront W - 1 and in the last
# block.  Every output against the oracle, and bit for bit against the full library, whose
# launches take one tile per wavefront.
def _capped_waves():
    return 4 * torch.cuda.get_device_properties(DEV).multi_processor_count


def _boundary_counts(W, bpt):
    """Block counts for W tiles of bpt blocks (the last one short by a block), W + 1 tiles (the
    last holding one block) and 2 W + 1 tiles (the last holding about half)."""
    return (W * bpt - 1, W * bpt + 1, 2 * W * bpt + max(1, bpt // 2 - 1))


def _boundary_input(rng, nb, B, dense=()):
    """float32 values of nb blocks: Laplace bodies at scales 2^-30..2^30 with zero,
    bfloat16-subnormal and outlier blocks; the blocks in `dense` are plain Laplace blocks."""
    v = rng.laplace(0, 1, (nb, B)) * 2.0 ** rng.integers(-30, 30, (nb, 1))
    kind = rng.integers(0, 16, nb)
    kind[list(dense)] = 15
    v[kind == 0] = 0.0
    v[kind == 1] = rng.integers(-64, 65, (int((kind == 1).sum()), B)) * 2.0 ** -133
    v[kind == 2, :3] *= 1e3
    return v.reshape(-1).astype(np.float32)


def _same_bits(u, v):
    u, v = np.ascontiguousarray(u), np.ascontiguousarray(v)
    return u.shape == v.shape and np.array_equal(u.view(np.uint8), v.view(np.uint8))


@pytest.mark.parametrize("B,flags", [(64, 0), (128, 1), (256, 2), (512, 3)])
def test_capped_launches_at_the_loop_boundary(oracle, tfp8, monkeypatch, B, flags):
    W = _capped_waves()
    capped = _capped()
    rng = np.random.default_rng(8100 + B + flags)

    def both(fn):
        # fn() through the full library, then through the capped build
        full = fn()
        torch.cuda.synchronize()
        with monkeypatch.context() as m:
            m.setattr(tfp8, "_lib", capped)
            got = fn()
            torch.cuda.synchronize()
        return full, got

    # compress, bfloat16 and float32 input
    for f32 in (False, True):
        for nb in _boundary_counts(W, 16 if B == 64 else 8):
            v = _boundary_input(rng, nb, B)
            x = v if f32 else f32_to_bf16_bits(v)
            what = f"capped compress B={B} flags={flags} {'f32' if f32 else 'bf16'} nb={nb}"
            say(what)
            full, got = both(lambda: check_compress(oracle, tfp8, x, B, what=what, flags=flags,
                                                    gpu=True))
            for u, w in zip(got, full):
                assert _same_bits(u, w), what + ": capped and full launches differ"

    # decompress of the oracle's codes, float32 and bfloat16 output
    for nb in _boundary_counts(W, 8):
        q, a, s = oracle.compress(f32_to_bf16_bits(_boundary_input(rng, nb, B)), B, 1.0,
                                  flags=flags)
        what = f"capped decompress B={B} flags={flags} nb={nb}"
        say(what)
        qg, ag, sg = u8_to_gpu(q), f32_to_gpu(a), f32_to_gpu(s)
        full, got = both(lambda: [cpu(tfp8.decompress(qg, ag, sg, B, torch.float32, flags=flags)),
                                  gpu_bf16_bits(tfp8.decompress(qg, ag, sg, B, torch.bfloat16,
                                                                flags=flags))])
        for u, w in zip(got, full):
            assert _same_bits(u, w), what + ": capped and full launches differ"
        with monkeypatch.context() as m:
            m.setattr(tfp8, "_lib", capped)
            check_decompress(oracle, tfp8, q, a, s, B, what=what, flags=flags)

    # the reduce: its fixed-P forms (P = 2, 8) and its general form (P = 3), on contributions
    # compressed by the oracle, the first three blocks of contribution 1 the negation of
    # contribution 0's
    for P, nb in zip((2, 3, 8), _boundary_counts(W, 1024 // B)):
        xs = [_boundary_input(rng, nb, B) for _ in range(P)]
        xs[1].reshape(nb, B)[:3] = -xs[0].reshape(nb, B)[:3]
        enc = [oracle.compress(f32_to_bf16_bits(v), B, 1.0, flags=flags) for v in xs]
        q, a, s = (np.stack([e[k] for e in enc]) for k in range(3))
        what = f"capped reduce B={B} flags={flags} P={P} nb={nb}"
        say(what)
        full, got = both(lambda: check_reduce(oracle, tfp8, q, a, s, B, what=what, flags=flags,
                                              gpu=True))
        for u, w in zip(got, full):
            assert _same_bits(u, w), what + ": capped and full launches differ"

    # the accumulation: the streaming kernel at the boundary of its loop, and at B <= 128 the
    # second kernel at the boundary of its own (W + 1 scans of 128 blocks)
    counts = list(_boundary_counts(W, 16 if B == 64 else 8))
    if B <= 128:
        counts.append(W * 128 + 3)
    for i, nb in enumerate(counts):
        cancel = sorted({0, 5, min(W * 128 - 2, nb - 2), min(W * 128 + 1, nb - 1), nb - 1})
        v = _boundary_input(rng, nb, B, dense=cancel)
        x = f32_to_bf16_bits(v)
        q, a, s = oracle.compress(x, B, 1.0, flags=flags)
        g = _boundary_input(rng, nb, B)
        g.reshape(nb, B)[cancel] = -bf16_bits_to_f32(x).reshape(nb, B)[cancel]
        f32 = i % 2 == 1
        gl = g if f32 else f32_to_bf16_bits(g)
        inplace = i == 2
        what = (f"capped accumulate B={B} flags={flags} {'f32' if f32 else 'bf16'} nb={nb} "
                f"inplace={inplace}")
        say(what)
        full, got = both(lambda: _check_accumulate(oracle, tfp8, q, a, s, gl, B, what,
                                                   flags=flags, inplace=inplace))
        for u, w in zip(got, full):
            assert _same_bits(u, w), what + ": capped and full launches differ"


def _sweep_input(rng, nb, B):
    """A mixture of block kinds: Laplace bodies at random scales, outlier blocks, zero blocks,
    bfloat16-subnormal blocks and huge blocks."""
    blocks = []
    for _ in range(nb):
        kind = rng.integers(0, 10)
        scale = 2.0 ** rng.integers(-30, 30)
        if kind == 0:
            v = np.zeros(B)
        elif kind == 1:
            v = rng.integers(-64, 65, B) * 2.0 ** -133
        elif kind == 2:
            v = rng.laplace(0, 1, B) * 2.0 ** 90
        elif kind <= 4:
            v = rng.laplace(0, 1, B) * scale
            v[rng.integers(0, B, 3)] *= 1e3
        else:
            v = rng.laplace(0, 1, B) * scale
        blocks.append(v)
    return np.concatenate(blocks)


def test_random_sweep(oracle, tfp8):
    # 1000 seeded random cases over block size, variant flags, dtype, block count, target and
    # block kinds, through all four operations (later stages take the oracle's outputs).  Every
    # code mismatch must be an admissible tie; the tie counts are held to the caps over the
    # whole sweep, per flag set, since one tie in a 64-element case would exceed 1e-4 of it.
    from tiecheck import tie_cap

    ledger = []
    for case in range(1000):
        rng = np.random.default_rng(7000 + case)
        B = int(rng.choice([64, 128, 256, 512]))
        flags = int(rng.integers(0, 4))
        f32 = bool(rng.integers(0, 2))
        nb = int(rng.integers(1, 70))
        T = float(2.0 ** rng.integers(-20, 21) * rng.choice([1.0, 0.75, 1.5]))
        v = _sweep_input(rng, nb, B)
        x = v.astype(np.float32) if f32 else f32_to_bf16_bits(v.astype(np.float32))
        what = f"sweep {case}: B={B} flags={flags} {'f32' if f32 else 'bf16'} nb={nb} T={T}"
        q, a, s = check_compress(oracle, tfp8, x, B, T=T, what=what, flags=flags,
                                 tie_ledger=ledger)
        check_decompress(oracle, tfp8, q, a, s, B, what=what, flags=flags)
        P = int(rng.integers(1, 6))
        enc = [(q, a, s)] + [oracle.compress(
            f32_to_bf16_bits((_sweep_input(rng, nb, B) * rng.choice([-1.0, 1.0])).astype(np.float32)),
            B, T, flags=flags) for _ in range(P - 1)]
        check_reduce(oracle, tfp8, np.stack([e[0] for e in enc]), np.stack([e[1] for e in enc]),
                     np.stack([e[2] for e in enc]), B, T, what=what + f" P={P}", flags=flags,
                     tie_ledger=ledger)
        # local gradient: minus the input on some blocks (cancellation), fresh values elsewhere
        g = -(bf16_bits_to_f32(x) if not f32 else x).astype(np.float64)
        g = g + rng.normal(0, 1e-3, g.size) * np.abs(g)
        fresh = rng.random(nb) < 0.5
        if fresh.any():
            g.reshape(nb, B)[fresh] = _sweep_input(rng, int(fresh.sum()), B).reshape(-1, B)
        gl = g.astype(np.float32) if rng.integers(0, 2) else f32_to_bf16_bits(g.astype(np.float32))
        _check_accumulate(oracle, tfp8, q, a, s, gl, B, what + " accumulate", flags=flags,
                          inplace=bool(rng.integers(0, 2)), T=T, tie_ledger=ledger)
    for fl in range(4):
        mis = sum(m for f, m, _ in ledger if f == fl)
        n = sum(k for f, _, k in ledger if f == fl)
        say(f"  sweep flags={fl}: {mis} tie mismatches in {n} codes")
        assert mis <= tie_cap(fl) * max(n, 1), (fl, mis, n)


def _struct_input(rng, nb, B, with_mask=False):
    """Blocks built to stress exactness: Hadamard rows with a few perturbed entries, one-hot
    blocks with tiny noise, constant and alternating blocks, each at a random power-of-two scale,
    mixed with the random sweep's kinds.  Their rotated values and sums often land exactly on
    code midpoints or cancel exactly.  With with_mask, also return which blocks are of the random
    kinds (not built to land on midpoints)."""
    idx = np.arange(B)
    out = []
    rand = np.zeros(nb, bool)
    for bi in range(nb):
        kind = rng.integers(0, 6)
        rand[bi] = kind >= 4
        scale = 2.0 ** rng.integers(-40, 40)
        if kind == 0:
            r = rng.integers(0, B)
            v = np.array([(-1.0) ** bin(r & j).count("1") for j in idx])
            k = rng.integers(0, 6)
            v[rng.integers(0, B, k)] *= rng.choice([0.5, 1.5, 1e-3, -1.0], k)
        elif kind == 1:
            v = np.zeros(B)
            v[rng.integers(0, B)] = rng.choice([-1.0, 1.0])
            v[rng.integers(0, B, 3)] += rng.normal(0, 1e-4, 3)
        elif kind == 2:
            v = np.full(B, rng.choice([-1.0, 1.0])) + rng.normal(0, 1e-3, B) * (rng.random(B) < 0.1)
        elif kind == 3:
            v = np.where(idx % 2 == 0, 1.0, -1.0) * (1 + rng.integers(0, 3, B) / 8)
        else:
            v = _sweep_input(rng, 1, B)
            scale = 1.0
        out.append(v * scale)
    return (np.concatenate(out), rand) if with_mask else np.concatenate(out)


def test_structured_sweep(oracle, tfp8):
    # 1000 seeded cases like the random sweep, on structured blocks, with local gradients that are
    # the input's negative up to bf16-sized noise (so many blocks cancel exactly or nearly).  By
    # construction many codes sit exactly on midpoints, so over all blocks only admissibility is
    # checked; the tie counts are held to the caps over the blocks of the random kinds, whose
    # outputs come only from such blocks (every contribution of a reduced block, and for the
    # accumulation both the main block and a fresh local-gradient block).
    from tiecheck import tie_cap

    ledger, rand_ledger = [], []
    for case in range(1000):
        rng = np.random.default_rng(10000 + case)
        B = int(rng.choice([64, 128, 256, 512]))
        flags = int(rng.integers(0, 4))
        f32 = bool(rng.integers(0, 2))
        nb = int(rng.choice([1, 7, 63, 257]))
        T = float(2.0 ** rng.integers(-20, 21) * rng.choice([1.0, 0.75, 1.5]))
        v, rand_x = _struct_input(rng, nb, B, with_mask=True)
        x = v.astype(np.float32) if f32 else f32_to_bf16_bits(v.astype(np.float32))
        what = f"structured {case}: B={B} flags={flags} {'f32' if f32 else 'bf16'} nb={nb} T={T}"
        q, a, s = check_compress(oracle, tfp8, x, B, T=T, what=what, flags=flags,
                                 tie_ledger=ledger, block_mask=rand_x, mask_ledger=rand_ledger)
        check_decompress(oracle, tfp8, q, a, s, B, what=what, flags=flags)
        P = int(rng.choice([1, 2, 3, 8, 16]))
        enc = [(q, a, s)]
        rand_r = rand_x.copy()
        for _ in range(P - 1):
            vp, rp = _struct_input(rng, nb, B, with_mask=True)
            enc.append(oracle.compress(
                f32_to_bf16_bits((vp * rng.choice([-1.0, 1.0])).astype(np.float32)), B, T,
                flags=flags))
            rand_r &= rp
        check_reduce(oracle, tfp8, np.stack([e[0] for e in enc]), np.stack([e[1] for e in enc]),
                     np.stack([e[2] for e in enc]), B, T, what=what + f" P={P}", flags=flags,
                     tie_ledger=ledger, block_mask=rand_r, mask_ledger=rand_ledger)
        g = -(bf16_bits_to_f32(x) if not f32 else x).astype(np.float64)
        g = g + rng.normal(0, 1e-3, g.size) * np.abs(g)
        fresh = rng.random(nb) < 0.3
        rand_g = np.zeros(nb, bool)
        if fresh.any():
            vg, rg = _struct_input(rng, int(fresh.sum()), B, with_mask=True)
            g.reshape(nb, B)[fresh] = vg.reshape(-1, B)
            rand_g[fresh] = rg
        gl = g.astype(np.float32) if rng.integers(0, 2) else f32_to_bf16_bits(g.astype(np.float32))
        _check_accumulate(oracle, tfp8, q, a, s, gl, B, what + " accumulate", flags=flags,
                          inplace=bool(rng.integers(0, 2)), T=T, tie_ledger=ledger,
                          block_mask=rand_x & rand_g, mask_ledger=rand_ledger)
    for fl in range(4):
        mis = sum(m for f, m, _ in rand_ledger if f == fl)
        n = sum(k for f, _, k in rand_ledger if f == fl)
        say(f"  structured sweep flags={fl}, random-kind blocks: {mis} tie mismatches in {n} codes")
        assert mis <= tie_cap(fl) * max(n, 1), (fl, mis, n)
    for fl in range(4):
        mis = sum(m for f, m, _ in ledger if f == fl)
        n = sum(k for f, _, k in ledger if f == fl)
        say(f"  structured sweep flags={fl}: {mis} tie mismatches in {n} codes")


def test_wide_sweep(oracle, tfp8):
    # 300 seeded cases over wider ranges than the sweeps above: up to 600 blocks, T anywhere in
    # the contract's [2^-64, 2^64], random and structured blocks mixed within a case, P up to 64
    # with some contributions the exact negation of the first (sums that cancel below float64's
    # resolution of their peaks are held to the bound both float64 sums satisfy), and local
    # gradients at 2^-80 to 2^80 of the main gradient's peak or its negation.  Only admissibility
    # is checked: the structured blocks land on code midpoints by construction.
    for case in range(300):
        rng = np.random.default_rng(20000 + case)
        B = int(rng.choice([64, 128, 256, 512]))
        flags = int(rng.integers(0, 4))
        f32 = bool(rng.integers(0, 2))
        nb = max(1, int(np.exp(rng.uniform(0, np.log(600)))))
        T = min(max(float(np.float32(2.0 ** rng.uniform(-64, 64))), 2.0 ** -64), 2.0 ** 64)
        pick = rng.random(nb) < rng.uniform(0, 1)
        v = np.where(pick[:, None], _struct_input(rng, nb, B).reshape(nb, B),
                     _sweep_input(rng, nb, B).reshape(nb, B)).reshape(-1)
        x = v.astype(np.float32) if f32 else f32_to_bf16_bits(v.astype(np.float32))
        xf = (x if f32 else bf16_bits_to_f32(x)).astype(np.float64)
        what = f"wide {case}: B={B} flags={flags} {'f32' if f32 else 'bf16'} nb={nb} T={T:.3e}"
        q, a, s = check_compress(oracle, tfp8, x, B, T=T, what=what, flags=flags, tie_ledger=[])
        check_decompress(oracle, tfp8, q, a, s, B, what=what, flags=flags)
        P = max(1, int(np.exp(rng.uniform(0, np.log(65)))))
        enc = [(q, a, s)]
        for _ in range(P - 1):
            xp = -xf if rng.integers(0, 4) == 0 else _sweep_input(rng, nb, B) * rng.choice([-1.0, 1.0])
            enc.append(oracle.compress(f32_to_bf16_bits(xp.astype(np.float32)), B, T, flags=flags))
        check_reduce(oracle, tfp8, np.stack([e[0] for e in enc]), np.stack([e[1] for e in enc]),
                     np.stack([e[2] for e in enc]), B, T, what=what + f" P={P}", flags=flags,
                     tie_ledger=[])
        # each fresh local-gradient block brought to 2^U(-80, 80) of the main block's peak
        peaks = np.abs(xf.reshape(nb, B)).max(axis=1)
        fresh = _sweep_input(rng, nb, B).reshape(nb, B)
        fpk = np.abs(fresh).max(axis=1)
        target = np.where(peaks > 0, peaks, 1.0) * 2.0 ** rng.uniform(-80, 80, nb)
        fresh *= np.where(fpk > 0, target / np.where(fpk > 0, fpk, 1.0), 0.0)[:, None]
        g = np.where((rng.random(nb) < 0.5)[:, None], -xf.reshape(nb, B), fresh)
        g = np.clip(g, -2.0 ** 99, 2.0 ** 99).reshape(-1)
        assert np.all(np.isfinite(g))
        gl = g.astype(np.float32) if rng.integers(0, 2) else f32_to_bf16_bits(g.astype(np.float32))
        _check_accumulate(oracle, tfp8, q, a, s, gl, B, what + " accumulate", flags=flags,
                          inplace=bool(rng.integers(0, 2)), T=T, tie_ledger=[])
