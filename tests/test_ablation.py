"""The ablation harness: its metric definitions (CPU, hand-computed case) and its GPU numbers
against the same metrics on the oracle's reconstructions."""
import math
import os

import numpy as np
import pytest
import torch

from fp8_compression_tensor_amd.ablation import VARIANTS, ablate, error_metrics
from workloads import TINY, WORKLOADS, bf16_bits_to_f32, make_shard


def test_error_metrics_hand_computed():
    # block 4: x = [1, 2, 0, -4], xh = [1, 0, 0, 4]
    x = torch.tensor([1.0, 2.0, 0.0, -4.0])
    xh = torch.tensor([1.0, 0.0, 0.0, 4.0])
    m = error_metrics(x, xh, 4)
    assert math.isclose(m["rel_l2"], math.sqrt(4 + 64) / math.sqrt(21))
    assert math.isclose(m["zero_collapse"], 1 / 3)   # the 2 came back as 0
    assert math.isclose(m["sign_flip"], 1 / 3)       # the -4 came back as +4
    # body: nonzero |x| <= median(|x| of nonzero) = 2 -> {1, 2}, rel errs {0, 1}; median = 0
    # (torch's median of an even count is the lower middle value)
    assert m["body_rel_err"] == 0.0
    assert math.isclose(m["block_snr_db"], 10 * math.log10(21 / 68))


@pytest.mark.gpu
def test_ablation_matches_oracle(oracle):
    oracle.set_threads(min(16, len(os.sched_getaffinity(0))))
    wl = WORKLOADS[TINY]
    bits = make_shard(TINY).reshape(-1)
    x = torch.from_numpy(bits.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    got = ablate(x, wl.block)
    xv = torch.from_numpy(bf16_bits_to_f32(bits))
    for name, flags in VARIANTS.items():
        q, a, s = oracle.compress(bits, wl.block, 1.0, flags=flags)
        xh = torch.from_numpy(oracle.decompress(q, a, s, wl.block, np.float32, flags=flags))
        ref = error_metrics(xv, xh, wl.block)
        g = got[name]
        print(name, g, flush=True)
        assert math.isclose(g["rel_l2"], ref["rel_l2"], rel_tol=1e-4), (name, g, ref)
        assert abs(g["zero_collapse"] - ref["zero_collapse"]) <= 1e-4, (name, g, ref)
        assert abs(g["sign_flip"] - ref["sign_flip"]) <= 1e-4, (name, g, ref)
        assert math.isclose(g["body_rel_err"], ref["body_rel_err"], rel_tol=1e-3, abs_tol=1e-9)
        assert abs(g["block_snr_db"] - ref["block_snr_db"]) <= 1e-3, (name, g, ref)
