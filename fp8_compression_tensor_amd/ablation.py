"""Numerical ablation of the block codecs on tensor-parallel-like tensors.

The TACO page ("TACO: Efficient Communication Compression of Intermediate Tensors for Scalable
Tensor-Parallel LLM Training") argues that uniform INT8 maps distinct small values onto the same
integer and loses the dense near-zero body of TP tensors ("zero collapse", sections 2.A and 3),
that E4M3's exponent keeps those values, and that the scale-Hadamard transform with dual scales
is what makes FP8 usable (sections 2.B.1-2.B.2, ablation in section 4).  This module measures
those claims on a given tensor for four codecs, all run by the GPU library:

  int8            per-block absmax INT8 (Q_max 127), no rotation
  e4m3            per-block absmax E4M3 (Q_max 448), no rotation
  int8+ash+ds     INT8 codes after the adaptive scale-Hadamard transform
  e4m3+ash+ds     the method: E4M3 codes after the adaptive scale-Hadamard transform

For each it reports the round-trip error of x -> codes -> x_hat (float32 output):
  rel_l2          ||x_hat - x|| / ||x||
  zero_collapse   fraction of the nonzero inputs that come back as exactly 0
  sign_flip       fraction of the nonzero inputs that come back nonzero with the other sign
  body_rel_err    median |x_hat - x| / |x| over the nonzero inputs at or below the median |x|
                  (the dense near-zero body)
  block_snr_db    median over nonzero blocks of 10 log10(sum x^2 / sum (x_hat - x)^2)

Usage: python -m fp8_compression_tensor_amd.ablation [--workloads tiny gpt2.7b-act ...]
"""
from __future__ import annotations

import argparse
import json
import math
import sys

import torch

from . import FLAG_INT8, FLAG_NO_ROTATION, compress, decompress

VARIANTS = {
    "int8": FLAG_INT8 | FLAG_NO_ROTATION,
    "e4m3": FLAG_NO_ROTATION,
    "int8+ash+ds": FLAG_INT8,
    "e4m3+ash+ds": 0,
}


def error_metrics(x: torch.Tensor, xh: torch.Tensor, block: int) -> dict:
    """Round-trip error statistics of a reconstruction xh of x (same shape, any device)."""
    x = x.reshape(-1).to(torch.float64)
    xh = xh.reshape(-1).to(torch.float64)
    err = xh - x
    nz = x != 0
    n_nz = int(nz.sum())
    ax = x.abs()
    out = {
        "rel_l2": float(err.norm() / x.norm()) if float(x.norm()) > 0 else 0.0,
        "zero_collapse": float((nz & (xh == 0)).sum()) / max(n_nz, 1),
        "sign_flip": float((nz & (xh != 0) & (torch.sign(xh) != torch.sign(x))).sum()) / max(n_nz, 1),
    }
    if n_nz:
        med = ax[nz].median()
        body = nz & (ax <= med)
        out["body_rel_err"] = float((err[body].abs() / ax[body]).median())
    else:
        out["body_rel_err"] = 0.0
    xb, eb = x.reshape(-1, block), err.reshape(-1, block)
    sig, noise = (xb * xb).sum(1), (eb * eb).sum(1)
    keep = sig > 0
    snr = 10.0 * torch.log10(sig[keep] / noise[keep].clamp_min(1e-300))
    out["block_snr_db"] = float(snr.median()) if int(keep.sum()) else math.inf
    return out


def roundtrip(x: torch.Tensor, block: int, flags: int, target: float = 1.0) -> torch.Tensor:
    """x -> codes -> float32 reconstruction, on the GPU."""
    codes, alpha, scale = compress(x.reshape(-1), block, target, flags=flags)
    return decompress(codes, alpha, scale, block, torch.float32, flags=flags)


def ablate(x: torch.Tensor, block: int, target: float = 1.0) -> dict:
    """Metrics of every variant on the GPU tensor x (bfloat16 or float32)."""
    return {name: error_metrics(x, roundtrip(x, block, flags, target), block)
            for name, flags in VARIANTS.items()}


def _table(rows):
    cols = ["rel_l2", "zero_collapse", "sign_flip", "body_rel_err", "block_snr_db"]
    lines = ["| workload | codec | " + " | ".join(cols) + " |", "|---" * (len(cols) + 2) + "|"]
    for wname, name, m in rows:
        vals = [f"{m[c]:.3e}" if c != "block_snr_db" else f"{m[c]:.1f}" for c in cols]
        lines.append(f"| {wname} | {name} | " + " | ".join(vals) + " |")
    return "\n".join(lines)


def main(argv=None):
    import os

    import numpy as np

    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from workloads import WORKLOADS, make_shard

    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", nargs="*", default=list(WORKLOADS), choices=list(WORKLOADS))
    ap.add_argument("--json", action="store_true")
    args = ap.parse_args(argv)
    rows = []
    for key in args.workloads:
        wl = WORKLOADS[key]
        bits = make_shard(key, 0).reshape(-1)
        x = torch.from_numpy(bits.view(np.int16)).to("cuda:0").view(torch.bfloat16)
        for name, m in ablate(x, wl.block).items():
            rows.append((f"{key} ({wl.label}, B={wl.block})", name, m))
        print(f"{key} done", file=sys.stderr, flush=True)
    if args.json:
        print(json.dumps([{"workload": c, "codec": n, **m} for c, n, m in rows]))
    else:
        print(_table(rows))


if __name__ == "__main__":
    main()
