"""Helpers for the GPU parity tests: move inputs to the device, run the library through its
C ABI (via the thin binding), and compare with the oracle to the stated bar."""
from __future__ import annotations

import sys

import numpy as np
import torch

from tiecheck import FLAG_INT8, assert_codes_match, assert_rel_close, tie_cap

DEV = torch.device("cuda:0")


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def bits_to_gpu(bits: np.ndarray) -> torch.Tensor:
    """bfloat16 bit patterns (uint16) -> bfloat16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def f32_to_gpu(v: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(DEV)


def u8_to_gpu(v: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(v, np.uint8)).to(DEV)


def cpu(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def gpu_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_scales(alpha, scale, ref_alpha, ref_scale, what="scales"):
    """Per block: alpha and s within 1e-6 relative; zero blocks exactly (alpha 1, s 0);
    a clamped alpha exactly."""
    alpha = np.asarray(alpha, np.float32).reshape(-1)
    scale = np.asarray(scale, np.float32).reshape(-1)
    ref_alpha = np.asarray(ref_alpha, np.float32).reshape(-1)
    ref_scale = np.asarray(ref_scale, np.float32).reshape(-1)
    zero = ref_scale == 0
    assert np.all(scale[zero] == 0) and np.all(alpha[zero] == 1), f"{what}: zero blocks differ"
    clamped = (ref_alpha == np.float32(2.0 ** 126)) | (ref_alpha == np.float32(2.0 ** -126))
    assert np.array_equal(alpha[clamped], ref_alpha[clamped]), f"{what}: clamped alpha differs"
    ea = assert_rel_close(alpha, ref_alpha, 1e-6, what=what + " alpha")
    es = assert_rel_close(scale, ref_scale, 1e-6, what=what + " scale")
    return ea, es


def assert_bf16_match(got_bits, ref_bits, ref_f64, rel=2.0 ** -20, what="bf16 output"):
    """bfloat16 outputs identical except adjacent values where the exact result is within
    `rel` of the midpoint between them (double rounding through float32)."""
    got = np.asarray(got_bits, np.uint16).reshape(-1)
    ref = np.asarray(ref_bits, np.uint16).reshape(-1)
    x = np.asarray(ref_f64, np.float64).reshape(-1)
    gv = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rv = (ref.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    bad = np.nonzero(gv != rv)[0]  # +0 and -0 compare equal as values
    if bad.size == 0:
        return 0
    g, r = got[bad].astype(np.int64), ref[bad].astype(np.int64)
    same_sign = (g >> 15) == (r >> 15)
    adjacent = same_sign & (np.abs((g & 0x7FFF) - (r & 0x7FFF)) == 1)
    mid = 0.5 * (gv[bad] + rv[bad])
    near = np.abs(x[bad] - mid) <= rel * np.abs(mid) + 2.0 ** -150
    ok = adjacent & near
    assert ok.all(), (f"{what}: {int((~ok).sum())} bf16 mismatches not at a rounding tie; first at "
                      f"{bad[np.argmax(~ok)]}: got {gv[bad][np.argmax(~ok)]!r} ref "
                      f"{rv[bad][np.argmax(~ok)]!r} exact {x[bad][np.argmax(~ok)]!r}")
    return int(bad.size)


def assert_codes_match_every_block(got, ref, B: int, quot_of_blocks, max_frac: float,
                                   what="codes", int8: bool = False):
    """Whole-tensor code check for tensors too large to carry the oracle's quotients for every
    element: codes are compared on every element, the exact quotients are fetched only for the
    blocks that hold a mismatch (``quot_of_blocks(block_indices)`` returns them flattened, in the
    order given), every mismatch must be an admissible tie, and the tie count is held to
    ``max_frac`` of the WHOLE tensor.  Returns the number of mismatches."""
    got = np.asarray(got, np.uint8).reshape(-1, B)
    ref = np.asarray(ref, np.uint8).reshape(-1, B)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    nbt = got.shape[0]
    chunk = 1 << 20  # blocks per pass, to bound the temporary mask
    blocks = [np.nonzero((got[i:i + chunk] != ref[i:i + chunk]).any(axis=1))[0] + i
              for i in range(0, nbt, chunk)]
    blocks = np.concatenate(blocks) if blocks else np.zeros(0, np.int64)
    if blocks.size == 0:
        return 0
    t = np.asarray(quot_of_blocks(blocks), np.float64).reshape(-1)
    assert t.size == blocks.size * B, (t.size, blocks.size)
    nmis = assert_codes_match(got[blocks], ref[blocks], t, max_frac=1.0, what=what, int8=int8)
    assert nmis <= max_frac * got.size, (f"{what}: {nmis} tie mismatches of {got.size} exceed "
                                         f"{max_frac} of the tensor")
    return nmis


def _count_in_blocks(got, ref, B, block_mask, flags, mask_ledger):
    """Append (flags, mismatches, elements) over the blocks selected by block_mask to the ledger."""
    if block_mask is None:
        return
    m = np.asarray(block_mask, bool).reshape(-1)
    g = np.asarray(got, np.uint8).reshape(-1, B)[m]
    r = np.asarray(ref, np.uint8).reshape(-1, B)[m]
    mask_ledger.append((flags, int((g != r).sum()), int(g.size)))


def _tie_cap(flags, ledger):
    """Per-call tie cap, or none when the caller keeps a ledger of (flags, mismatches, elements)
    and holds the total to the cap itself (many small calls: one tie would exceed 1e-4 of 64)."""
    return 1.0 if ledger is not None else tie_cap(flags)


def check_compress(oracle, tfp8, x: np.ndarray, B: int, T: float = 1.0, what="compress",
                   flags: int = 0, gpu: bool = False, tie_ledger=None, block_mask=None,
                   mask_ledger=None):
    """GPU compress of host input x (uint16 bfloat16 bits or float32) vs the oracle.
    Returns the oracle's (codes, alpha, scale), the input of any later stage (no oracle input
    ever comes from the GPU), or with gpu=True the GPU's, as numpy arrays."""
    xg = bits_to_gpu(x) if x.dtype == np.uint16 else f32_to_gpu(x)
    q, a, s = tfp8.compress(xg.reshape(-1), B, T, flags=flags)
    torch.cuda.synchronize()
    q, a, s = cpu(q), cpu(a), cpu(s)
    qr, ar, sr, tr = oracle.compress(x.reshape(-1), B, T, with_quot=True, flags=flags)
    nmis = assert_codes_match(q, qr, tr, max_frac=_tie_cap(flags, tie_ledger),
                              what=what + " codes", int8=bool(flags & FLAG_INT8))
    if tie_ledger is not None:
        tie_ledger.append((flags, nmis, q.size))
    _count_in_blocks(q, qr, B, block_mask, flags, mask_ledger)
    ea, es = assert_scales(a, s, ar, sr, what=what)
    say(f"  {what}: n={x.size} B={B} T={T} flags={flags}: code tie mismatches {nmis} "
        f"({nmis / max(x.size, 1):.2e}), max rel err alpha {ea:.2e} scale {es:.2e}")
    return (q, a, s) if gpu else (qr, ar, sr)


def check_decompress(oracle, tfp8, q, a, s, B: int, what="decompress", flags: int = 0):
    """GPU decompress of the given codes and scales vs the oracle, float32 and bfloat16."""
    qg, ag, sg = u8_to_gpu(q.reshape(-1)), f32_to_gpu(a), f32_to_gpu(s)
    o32 = tfp8.decompress(qg, ag, sg, B, torch.float32, flags=flags)
    o16 = tfp8.decompress(qg, ag, sg, B, torch.bfloat16, flags=flags)
    torch.cuda.synchronize()
    r64 = oracle.decompress_f64(q, a, s, B, flags=flags)
    r32 = oracle.decompress(q, a, s, B, np.float32, flags=flags)
    r16 = oracle.decompress(q, a, s, B, np.uint16, flags=flags)
    e32 = assert_rel_close(cpu(o32), r32, 1e-6, 2.0 ** -149, what=what + " f32")
    n16 = assert_bf16_match(gpu_bf16_bits(o16), r16, r64, what=what + " bf16")
    normal = np.abs(r32) >= 2.0 ** -126
    e32n = float((np.abs(cpu(o32)[normal] - r32[normal]) / np.abs(r32[normal])).max()) if normal.any() else 0.0
    say(f"  {what}: n={q.size} B={B} flags={flags}: max rel err f32 (normal results) {e32n:.2e}, "
        f"bf16 tie mismatches {n16}")
    return o32


def check_reduce(oracle, tfp8, q, a, s, B, T=1.0, what="reduce", flags: int = 0,
                 gpu: bool = False, tie_ledger=None, block_mask=None, mask_ledger=None):
    """GPU reduce of stacked codes/scales [P, ...] vs the oracle's reduce by definition.
    Returns the oracle's (codes, alpha, scale), or with gpu=True the GPU's."""
    P, n = q.shape
    qg, ag, sg = u8_to_gpu(q), f32_to_gpu(a), f32_to_gpu(s)
    cq, ca, cs = tfp8.reduce_fp8(qg, ag, sg, B, T, flags=flags)
    torch.cuda.synchronize()
    cq, ca, cs = cpu(cq), cpu(ca), cpu(cs)
    rq, ra, rs, rt = oracle.reduce_fp8(q, a, s, B, T, with_quot=True, flags=flags)
    nmis = assert_codes_match(cq, rq, rt, max_frac=_tie_cap(flags, tie_ledger),
                              what=what + " codes", int8=bool(flags & FLAG_INT8))
    if tie_ledger is not None:
        tie_ledger.append((flags, nmis, cq.size))
    _count_in_blocks(cq, rq, B, block_mask, flags, mask_ledger)
    ea, es = assert_scales(ca, cs, ra, rs, what=what)
    say(f"  {what}: P={P} n={n} B={B} flags={flags}: code tie mismatches {nmis} ({nmis / n:.2e}), "
        f"max rel err alpha {ea:.2e} scale {es:.2e}")
    return (cq, ca, cs) if gpu else (rq, ra, rs)
