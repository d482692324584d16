"""The C-ABI library loads, exports every symbol include/tfp8.h declares, and rejects bad
arguments before touching the GPU (these calls make no HIP call, so they run without one)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tfp8.h")


@pytest.fixture(scope="module")
def tfp8():
    import fp8_compression_tensor_amd as m

    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tfp8_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_three_operations():
    names = declared_functions()
    for want in ("tfp8_compress", "tfp8_decompress", "tfp8_reduce_fp8", "tfp8_status_string"):
        assert want in names


def test_library_exports_every_declared_symbol(tfp8):
    L = tfp8.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.tfp8_version() >> 16 == 1


def test_capped_test_build_exports_every_declared_symbol(tfp8):
    # the launch-capped build that the GPU tests of the grid-stride loops load
    path = os.path.join(ROOT, "tests", "capped_build", "libtfp8_capped.so")
    assert os.path.exists(path), f"{path} is not built (tests/capped_build/build.py)"
    L = tfp8._declare(ctypes.CDLL(path))
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.tfp8_version() == tfp8.lib().tfp8_version()


def test_status_strings(tfp8):
    for st in range(-7, 1):
        s = tfp8.status_string(st)
        assert s and s != "unknown status"
    assert tfp8.status_string(-99) == "unknown status"


FAKE = 0x7F0000000000  # a 16-byte aligned address that is never dereferenced here


def test_compress_argument_errors(tfp8):
    c = tfp8.compress_raw
    assert c(FAKE, 0, 1024, 96, 1.0, FAKE + 4096, FAKE + 8192, FAKE + 12288) == -3  # block
    assert c(FAKE, 0, 1000, 128, 1.0, FAKE + 4096, FAKE + 8192, FAKE + 12288) == -2  # n % B
    assert c(FAKE, 0, -128, 128, 1.0, FAKE + 4096, FAKE + 8192, FAKE + 12288) == -2
    # above the 2^40 maximum (byte counts of such sizes could overflow)
    big = (1 << 40) + 128
    assert c(FAKE, 0, big, 128, 1.0, FAKE + 4096, FAKE + 8192, FAKE + 12288) == -2
    assert c(FAKE, 1, 1 << 62, 128, 1.0, FAKE + 4096, FAKE + 8192, FAKE + 12288) == -2
    assert tfp8.decompress_raw(FAKE, FAKE + 4096, FAKE + 8192, big, 128, FAKE + 16384, 1) == -2
    assert tfp8.reduce_fp8_raw(FAKE, FAKE + 65536, FAKE + 81920, 4, big, 128, 1.0, FAKE + 131072,
                               FAKE + 196608, FAKE + 200704) == -2
    assert tfp8.accumulate_raw(FAKE, FAKE + 8192, FAKE + 12288, FAKE + 16384, 0, big, 128, 1.0,
                               FAKE + 32768, FAKE + 40960, FAKE + 45056) == -2
    assert c(FAKE, 2, 1024, 128, 1.0, FAKE + 4096, FAKE + 8192, FAKE + 12288) == -4  # dtype
    for t in (0.0, -1.0, float("inf"), float("nan"), 2.0 ** 70, 2.0 ** -70):
        assert c(FAKE, 0, 1024, 128, t, FAKE + 4096, FAKE + 8192, FAKE + 12288) == -6
    assert c(None, 0, 1024, 128, 1.0, FAKE + 4096, FAKE + 8192, FAKE + 12288) == -1
    assert c(FAKE, 0, 1024, 128, 1.0, None, FAKE + 8192, FAKE + 12288) == -1
    assert c(FAKE + 2, 0, 1024, 128, 1.0, FAKE + 4096, FAKE + 8192, FAKE + 12288) == -5
    assert c(FAKE, 0, 1024, 128, 1.0, FAKE + 4104, FAKE + 8192, FAKE + 12288) == -5
    assert c(FAKE, 0, 1024, 128, 1.0, FAKE + 4096, FAKE + 8194, FAKE + 12288) == -5
    # codes overlapping the input, alpha overlapping scale
    assert c(FAKE, 0, 1024, 128, 1.0, FAKE + 1024, FAKE + 8192, FAKE + 12288) == -6
    assert c(FAKE, 0, 1024, 128, 1.0, FAKE + 4096, FAKE + 8192, FAKE + 8192 + 16) == -6
    # n = 0 is a no-op, even with NULL pointers
    assert c(None, 0, 0, 128, 1.0, None, None, None) == 0


def test_unknown_flags_are_rejected(tfp8):
    assert tfp8.compress_raw(FAKE, 0, 1024, 128, 1.0, FAKE + 4096, FAKE + 8192, FAKE + 12288,
                             0, 4) == -6
    assert tfp8.decompress_raw(FAKE, FAKE + 4096, FAKE + 8192, 1024, 128, FAKE + 16384, 1,
                               0, 8) == -6
    assert tfp8.reduce_fp8_raw(FAKE, FAKE + 65536, FAKE + 81920, 4, 1024, 128, 1.0, FAKE + 131072,
                               FAKE + 196608, FAKE + 200704, 0, 16) == -6
    # valid flags pass the checks (then n = 0 returns before any launch)
    assert tfp8.compress_raw(None, 0, 0, 128, 1.0, None, None, None, 0, 3) == 0


def test_decompress_argument_errors(tfp8):
    d = tfp8.decompress_raw
    assert d(FAKE, FAKE + 4096, FAKE + 8192, 1024, 100, FAKE + 16384, 1) == -3
    assert d(FAKE, FAKE + 4096, FAKE + 8192, 1000, 128, FAKE + 16384, 1) == -2
    assert d(FAKE, FAKE + 4096, FAKE + 8192, 1024, 128, FAKE + 16384, 5) == -4
    assert d(FAKE, None, FAKE + 8192, 1024, 128, FAKE + 16384, 1) == -1
    assert d(FAKE, FAKE + 4096, FAKE + 8192, 1024, 128, FAKE + 16388, 1) == -5
    assert d(FAKE, FAKE + 4096, FAKE + 8192, 1024, 128, FAKE + 512, 1) == -6  # out over codes
    assert d(None, None, None, 0, 128, None, 1) == 0


def test_reduce_argument_errors(tfp8):
    r = tfp8.reduce_fp8_raw
    args = (FAKE, FAKE + 65536, FAKE + 81920)
    outs = (FAKE + 131072, FAKE + 196608, FAKE + 200704)
    assert r(*args, 4, 1024, 64 * 3, 1.0, *outs) == -3
    assert r(*args, 4, 1000, 128, 1.0, *outs) == -2
    assert r(*args, 0, 1024, 128, 1.0, *outs) == -6
    assert r(*args, 65, 1024, 128, 1.0, *outs) == -6
    assert r(*args, 4, 1024, 128, 0.0, *outs) == -6
    assert r(FAKE, None, FAKE + 81920, 4, 1024, 128, 1.0, *outs) == -1
    # output codes inside the stacked input codes
    assert r(*args, 4, 1024, 128, 1.0, FAKE + 1024, outs[1], outs[2]) == -6
    assert r(None, None, None, 4, 0, 128, 1.0, None, None, None) == 0


def test_reduce_strided_argument_errors(tfp8):
    r = tfp8.reduce_strided_raw
    n, nb = 1024, 8  # block 128
    M = 1 << 16  # one message per peer in a receive buffer: [codes | alpha | scale], 64 KiB apart
    ins = (FAKE, M, FAKE + n, M // 4, FAKE + n + 4 * nb, M // 4)
    out0 = FAKE + 4 * M  # past the last of 4 messages
    outs = (out0, out0 + 4096, out0 + 8192)
    # stride checks: below the row length, codes stride not a multiple of 16, above 2^40
    assert r(FAKE, n - 16, *ins[2:], 4, n, 128, 1.0, *outs) == -6
    assert r(*ins[:3], nb - 1, *ins[4:], 4, n, 128, 1.0, *outs) == -6
    assert r(*ins[:5], nb - 1, 4, n, 128, 1.0, *outs) == -6
    assert r(FAKE, M + 8, *ins[2:], 4, n, 128, 1.0, *outs) == -5
    assert r(FAKE, (1 << 40) + 16, *ins[2:], 4, n, 128, 1.0, *outs) == -2
    assert r(*ins, 0, n, 128, 1.0, *outs) == -6
    assert r(*ins, 4, n, 96, 1.0, *outs) == -3
    assert r(*ins, 4, n, 128, 1.0, *outs, flags=4) == -6
    assert r(None, M, *ins[2:], 4, n, 128, 1.0, *outs) == -1
    # an output inside the span of the strided inputs, even in a gap between two messages
    assert r(*ins, 4, n, 128, 1.0, FAKE + M - 4096, outs[1], outs[2]) == -6
    assert r(*ins, 4, n, 128, 1.0, outs[0], FAKE + 2 * M + 4096, outs[2]) == -6
    # n = 0 is valid and launches nothing (the GPU tests pass inputs that overlap each other:
    # alpha and scale inside the codes' span)
    assert r(*ins, 4, 0, 128, 1.0, *outs) == 0
    assert r(None, 0, None, 0, None, 0, 4, 0, 128, 1.0, None, None, None) == 0


def test_accumulate_argument_errors(tfp8):
    a = tfp8.accumulate_raw
    ins = (FAKE, FAKE + 8192, FAKE + 12288, FAKE + 16384)
    outs = (FAKE + 32768, FAKE + 40960, FAKE + 45056)
    assert a(*ins, 0, 1024, 96, 1.0, *outs) == -3
    assert a(*ins, 0, 1000, 128, 1.0, *outs) == -2
    assert a(*ins, 7, 1024, 128, 1.0, *outs) == -4
    assert a(*ins, 0, 1024, 128, 0.0, *outs) == -6
    assert a(*ins, 0, 1024, 128, 1.0, *outs, 0, 8) == -6
    assert a(FAKE, FAKE + 8192, FAKE + 12288, None, 0, 1024, 128, 1.0, *outs) == -1
    assert a(FAKE, FAKE + 8192, FAKE + 12288, FAKE + 16386, 0, 1024, 128, 1.0, *outs) == -5
    # output codes over the gradient, or shifted into the input codes: rejected
    assert a(*ins, 0, 1024, 128, 1.0, FAKE + 16384, outs[1], outs[2]) == -6
    assert a(*ins, 0, 1024, 128, 1.0, FAKE + 16, outs[1], outs[2]) == -6
    # exactly in place: accepted (n = 0 makes it a no-op, so nothing is launched)
    assert a(*ins, 0, 0, 128, 1.0, FAKE, FAKE + 8192, FAKE + 12288) == 0


def test_tensor_wrappers_refuse_cpu_tensors(tfp8):
    import torch

    x = torch.zeros(1024, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        tfp8.compress(x, 128)
    with pytest.raises(ValueError, match="GPU"):
        tfp8.decompress(torch.zeros(1024, dtype=torch.uint8), torch.zeros(8), torch.zeros(8), 128)
