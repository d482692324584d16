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


ALPHA_MIN, ALPHA_MAX = 2.0 ** -126, 2.0 ** 126


def assert_scales(alpha, scale, ref_alpha, ref_scale, what="scales"):
    """Per block: alpha and s within 1e-6 relative; zero blocks exactly (alpha 1, s 0); every
    alpha inside the clamp range [2^-126, 2^126].  A clamped alpha is held to the same bar, so
    it is the bound or a value inside the range within 1e-6 of it, not the bound exactly: a block
    whose exact alpha is the bound itself (or within the kernel's few-ulp alpha error of it) is
    clamped by the oracle and may land one float inside the range on the GPU."""
    alpha = np.asarray(alpha, np.float32).reshape(-1)
    scale = np.asarray(scale, np.float32).reshape(-1)
    ref_alpha = np.asarray(ref_alpha, np.float32).reshape(-1)
    ref_scale = np.asarray(ref_scale, np.float32).reshape(-1)
    zero = ref_scale == 0
    assert np.all(scale[zero] == 0) and np.all(alpha[zero] == 1), f"{what}: zero blocks differ"
    inside = (alpha >= ALPHA_MIN) & (alpha <= ALPHA_MAX)
    assert inside.all(), f"{what}: {int((~inside).sum())} alpha outside the clamp range"
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
    """GPU reduce of stacked codes/scales [P, ...] vs the oracle's reduce by definition, to the
    tie rule; a code or scale that fails it is admitted only within the bound both float64 sums
    satisfy (assert_reduce_matches).  Returns the oracle's (codes, alpha, scale), or with
    gpu=True the GPU's."""
    P, n = q.shape
    qg, ag, sg = u8_to_gpu(q), f32_to_gpu(a), f32_to_gpu(s)
    cq, ca, cs = tfp8.reduce_fp8(qg, ag, sg, B, T, flags=flags)
    torch.cuda.synchronize()
    cq, ca, cs = cpu(cq), cpu(ca), cpu(cs)
    rq, ra, rs, rt = oracle.reduce_fp8(q, a, s, B, T, with_quot=True, flags=flags)
    nmis, nfb, ea, es = assert_reduce_matches(cq, ca, cs, rq, rt, ra, rs, a.reshape(P, -1),
                                              s.reshape(P, -1), B, flags,
                                              _tie_cap(flags, tie_ledger), what)
    if tie_ledger is not None:
        tie_ledger.append((flags, nmis, cq.size))
    _count_in_blocks(cq, rq, B, block_mask, flags, mask_ledger)
    say(f"  {what}: P={P} n={n} B={B} flags={flags}: code tie mismatches {nmis} ({nmis / n:.2e}), "
        f"max rel err alpha {ea:.2e} scale {es:.2e}"
        + (f"; {nfb} codes or blocks in float64 noise at the tie window's scale" if nfb else ""))
    return (cq, ca, cs) if gpu else (rq, ra, rs)


def assert_reduce_matches(cq, ca, cs, rq, rt, ra, rs, alpha_in, scale_in, B: int, flags: int,
                          max_frac: float, what: str):
    """A reduce's codes and scales against the oracle's.

    Blocks whose float64 noise stays far inside the tie window (slack w of tiecheck's
    reduce_quotient_slack under an eighth of its absolute term: every block whose contributions
    do not cancel by a large factor) are held to the tie rule, their ties capped at max_frac of
    the elements, and to the 1e-6 scale bar with zero blocks exact.  In the other blocks a code
    that is not an admissible tie must be the rounding of some quotient within w of the
    oracle's, alpha' and s' must lie within 1e-6 or the relative error that the bound D allows,
    and where the reference peak M lies inside the noise (M <= 2 D) the GPU's peak must be at
    most M + D; their mismatches are counted apart from the ties and kept out of the tie
    statistics.  Every alpha must lie inside the clamp range.  Returns (ties, codes and blocks
    counted apart, max rel err alpha, s over the blocks within 1e-6)."""
    from tiecheck import (TIE_ABS, assert_codes_match, assert_codes_within, code_mismatches,
                          reduce_quotient_slack, reduce_sum_bound)

    int8 = bool(flags & FLAG_INT8)
    Q = 127.0 if int8 else 448.0
    D = reduce_sum_bound(alpha_in, scale_in, Q)
    w, M = reduce_quotient_slack(D, ra, rs, Q)
    noisy_blk = w > TIE_ABS / 8
    noisy = np.repeat(noisy_blk, B)
    # codes of the ordinary blocks: the tie rule, the cap over the whole tensor
    nties = assert_codes_match(cq[~noisy], rq[~noisy], rt[~noisy], max_frac=1.0,
                               what=what + " codes", int8=int8)
    assert nties <= max_frac * max(cq.size, 1), (f"{what}: {nties} tie mismatches of {cq.size} "
                                                f"exceed {max_frac}")
    # codes of the noisy blocks: the tie rule, else the float64 sums' bound
    nm_n, bad_n = code_mismatches(cq[noisy], rq[noisy], rt[noisy], int8=int8, return_bad=True,
                                  record=False)
    bad = np.arange(cq.size)[noisy][bad_n]
    blk = bad // B
    fin = np.isfinite(w[blk])
    if fin.any():
        assert_codes_within(cq[bad[fin]], rt[bad[fin]], w[blk[fin]], int8,
                            what=what + " codes (float64 sums' bound)")
    noise_blocks = set(blk[~fin].tolist())
    # scales
    inside = (ca >= ALPHA_MIN) & (ca <= ALPHA_MAX)
    assert inside.all(), f"{what}: {int((~inside).sum())} alpha outside the clamp range"
    a64, s64 = ca.astype(np.float64), cs.astype(np.float64)
    ra64, rs64 = ra.astype(np.float64), rs.astype(np.float64)
    zero = rs64 == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        ea = np.where(zero, np.where(a64 == 1, 0.0, np.inf), np.abs(a64 / ra64 - 1))
        es = np.where(zero, np.where(s64 == 0, 0.0, np.inf), np.abs(s64 / rs64 - 1))
    std = (ea <= 1e-6) & (es <= 1e-6)
    off = np.nonzero(~std)[0]
    for k in off:
        assert noisy_blk[k], (f"{what}: block {k} alpha {a64[k]!r} s {s64[k]!r} against "
                              f"{ra64[k]!r}, {rs64[k]!r}: beyond 1e-6 (zero blocks exactly)")
        if np.isfinite(w[k]):
            rel_a = 1e-6 + 2 * np.sqrt(B) * D[k] / M[k]
            rel_s = rel_a + 2 * D[k] / M[k] + 1e-6
            assert ea[k] <= rel_a and es[k] <= rel_s, (
                f"{what}: block {k} alpha {a64[k]!r} s {s64[k]!r} against {ra64[k]!r}, {rs64[k]!r}")
        else:
            noise_blocks.add(int(k))
    for k in noise_blocks:  # a block inside its noise: only its peak is bounded
        assert s64[k] * Q / a64[k] <= M[k] + D[k], f"{what}: block {k} peak beyond its noise"
    return nties, nm_n + len(off), float(ea[std].max(initial=0.0)), \
        float(es[std].max(initial=0.0))


# ---- inputs that repeat every seven tiles, checked on every block on the GPU ----------------
#
# A tensor of tens of gigabytes cannot be compared with the oracle element by element on the
# host.  When its input repeats with a period of seven tiles (tile t is parts[t mod 7]), every
# output block equals the oracle's output for the same block of one of the seven parts, so the
# expected values are the oracle's outputs for the seven parts, gathered on the GPU by index.

def fill_periodic(dst: torch.Tensor, parts, per_tile: int) -> torch.Tensor:
    """Fill the flat GPU tensor dst so that tile t (per_tile elements, the last one cut short)
    is parts[t mod len(parts)]: the first period is uploaded, then doubled by copies of whole
    periods.  Returns dst."""
    period = len(parts) * per_tile
    head = torch.from_numpy(np.ascontiguousarray(np.concatenate(parts))).to(DEV)
    assert head.dtype == dst.dtype and head.numel() == period, (head.dtype, head.numel())
    c = min(period, dst.numel())
    dst[:c] = head[:c]
    while c < dst.numel():  # c stays a multiple of the period until the last copy
        k = min(c, dst.numel() - c)
        dst[c:c + k] = dst[:k]
        c += k
    return dst


def _periodic_src(k0: int, k1: int, bpt: int) -> torch.Tensor:
    """Row of the seven parts' stacked outputs that block k of the whole tensor equals."""
    k = torch.arange(k0, k1, device=DEV, dtype=torch.int64)
    return torch.div(k, bpt, rounding_mode="floor") % 7 * bpt + k % bpt


def assert_periodic_codes(q, a, s, refs, n: int, tile: int, B: int, what: str, flags: int = 0,
                          chunk: int = 1 << 20):
    """Codes, alpha and s of a whole periodic tensor against refs[w] = (codes, alpha, scale,
    quotients), the oracle's output for part w.  Codes and scales are compared on the GPU block
    by block; the blocks that hold a code mismatch are fetched, every mismatch must be an
    admissible tie and their count is held to the cap over the whole tensor.  alpha and s follow
    the rule of assert_scales (1e-6 relative; zero blocks alpha 1, s 0; every alpha inside the
    clamp range, a clamped one within 1e-6 of its bound).  Returns (tie mismatches, max rel err
    alpha, max rel err s)."""
    nb, bpt = n // B, tile // B
    hq = np.stack([np.asarray(r[0], np.uint8).reshape(bpt, B) for r in refs])
    ht = np.stack([np.asarray(r[3], np.float64).reshape(bpt, B) for r in refs])
    rq = u8_to_gpu(hq.reshape(-1, B))
    ra = torch.from_numpy(np.concatenate([r[1] for r in refs]).astype(np.float64)).to(DEV)
    rs = torch.from_numpy(np.concatenate([r[2] for r in refs]).astype(np.float64)).to(DEV)
    qv = q.view(nb, B)
    bad, worst = [], torch.zeros(2, dtype=torch.float64, device=DEV)
    nviol = torch.zeros((), dtype=torch.int64, device=DEV)
    for k0 in range(0, nb, chunk):
        k1 = min(nb, k0 + chunk)
        src = _periodic_src(k0, k1, bpt)
        bad.append(torch.nonzero((qv[k0:k1] != rq[src]).any(1)).view(-1) + k0)
        ga, gs, ea, es = a[k0:k1].double(), s[k0:k1].double(), ra[src], rs[src]
        da, ds = (ga - ea).abs(), (gs - es).abs()
        ok = (da <= 1e-6 * ea.abs()) & (ds <= 1e-6 * es.abs())
        ok &= (es != 0) | ((gs == 0) & (ga == 1))
        ok &= (ga >= ALPHA_MIN) & (ga <= ALPHA_MAX)
        nviol += (~ok).sum()
        zero = torch.zeros((), dtype=torch.float64, device=DEV)
        worst = torch.maximum(worst, torch.stack([
            torch.where(ea != 0, da / ea.abs(), zero).max(),
            torch.where(es != 0, ds / es.abs(), zero).max()]))
    assert int(nviol) == 0, f"{what}: {int(nviol)} blocks with alpha or s outside the bar"
    blocks = torch.cat(bad)
    nmis = 0
    if blocks.numel():
        bh = cpu(blocks)
        w, off = bh // bpt % 7, bh % bpt
        nmis = assert_codes_match(cpu(qv[blocks]), hq[w, off], ht[w, off], max_frac=1.0,
                                  what=what + " codes", int8=bool(flags & FLAG_INT8))
    assert nmis <= tie_cap(flags) * n, (f"{what}: {nmis} tie mismatches of {n} exceed "
                                        f"{tie_cap(flags)} of the tensor")
    ea, es = (float(v) for v in cpu(worst))
    return nmis, ea, es


def assert_periodic_decompress(out, refs, n: int, tile: int, B: int, what: str,
                               chunk: int = 1 << 18):
    """A whole periodic decompress output against refs[w] = (values, exact float64) from the
    oracle for part w: float32 outputs within 1e-6 relative (floor 2^-149), bfloat16 outputs
    identical except adjacent values whose exact result lies within 2^-20 of their midpoint
    (the rule of assert_bf16_match), all on the GPU.  Returns the bfloat16 tie count (0 for
    float32)."""
    nb, bpt = n // B, tile // B
    bf16 = out.dtype == torch.bfloat16
    if bf16:
        rv = torch.from_numpy(np.stack([np.asarray(r[0], np.uint16).view(np.int16)
                                        for r in refs]).reshape(-1, B)).to(DEV)
    else:
        rv = torch.from_numpy(np.stack([np.asarray(r[0], np.float32)
                                        for r in refs]).reshape(-1, B)).to(DEV)
    r64 = torch.from_numpy(np.stack([np.asarray(r[1], np.float64)
                                     for r in refs]).reshape(-1, B)).to(DEV)
    ov = out.view(nb, B)
    nmis = torch.zeros((), dtype=torch.int64, device=DEV)
    nviol = torch.zeros((), dtype=torch.int64, device=DEV)
    for k0 in range(0, nb, chunk):
        k1 = min(nb, k0 + chunk)
        src = _periodic_src(k0, k1, bpt)
        if not bf16:
            g, e = ov[k0:k1].double(), rv[src].double()
            nviol += (~((g - e).abs() <= 1e-6 * e.abs() + 2.0 ** -149)).sum()
            continue
        gb, eb = ov[k0:k1].view(torch.int16), rv[src]
        gv, ev = gb.view(torch.bfloat16).double(), eb.view(torch.bfloat16).double()
        mis = gv != ev  # +0 and -0 compare equal as values
        gi, ei = gb[mis].int(), eb[mis].int()
        adjacent = ((gi & 0x8000) == (ei & 0x8000)) & (((gi & 0x7FFF) - (ei & 0x7FFF)).abs() == 1)
        mid = 0.5 * (gv[mis] + ev[mis])
        near = (r64[src][mis] - mid).abs() <= 2.0 ** -20 * mid.abs() + 2.0 ** -150
        nmis += mis.sum()
        nviol += (~(adjacent & near)).sum()
    assert int(nviol) == 0, f"{what}: {int(nviol)} outputs outside the bar"
    return int(nmis)

