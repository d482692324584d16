"""Build tests/capped_build/libtfp8_capped.so: the library from the same source with every
launch capped at one workgroup per compute unit (TFP8_*_WGS_PER_CU = 1), so that inputs of a few
tens of MB run the kernels' grid-stride loops with many tiles per wavefront.  The caps change
only the host's choice of grid; the kernels are the same.  The GPU tests route the package's
calls through this capped library to check the looping forms at every block size, input type
and flag set, at sizes the full library reaches only past 2^34-2^36 elements."""
from __future__ import annotations

import importlib.util
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libtfp8_capped.so")
CAPS = ["-DTFP8_COMPRESS_WGS_PER_CU=1", "-DTFP8_DECOMPRESS_WGS_PER_CU=1",
        "-DTFP8_REDUCE_WGS_PER_CU=1", "-DTFP8_ACCUMULATE_FIX_WGS_PER_CU=1"]


def build(verbose: bool = False) -> str:
    # the package's own build script, loaded by path (importing the package would load the
    # library it builds)
    spec = importlib.util.spec_from_file_location(
        "_tfp8_hip_build", os.path.join(ROOT, "fp8_compression_tensor_amd", "build.py"))
    hip_build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(hip_build)
    return hip_build.build(verbose=verbose, extra=CAPS, out=LIB)


if __name__ == "__main__":
    print(build(verbose=True), file=sys.stderr)
