"""The library driven from plain C99 (tests/c_driver/tfp8_c_driver.c) through include/tfp8.h,
with no Python binding and no torch in the process: the header compiles as C, the program links
against libtfp8.so, argument errors come back as the header documents them, and on the GPU
compress, reduce_fp8 and decompress called this way match the oracle to the parity bar.

Every input of the GPU checks comes from the seeded generators or from the oracle, never from an
earlier GPU result."""
import importlib.util
import os
import subprocess
import tempfile

import numpy as np
import pytest

from tiecheck import assert_codes_match, assert_rel_close
from workloads import TINY, WORKLOADS, make_shard

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER_DIR = os.path.join(HERE, "c_driver")
EXE = os.path.join(DRIVER_DIR, "tfp8_c_driver")


def _build_module():
    spec = importlib.util.spec_from_file_location("_tfp8_c_driver_build",
                                                  os.path.join(DRIVER_DIR, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(*args, timeout=120):
    r = subprocess.run([EXE, *map(str, args)], capture_output=True, text=True, timeout=timeout)
    print(r.stdout, r.stderr, flush=True)
    return r


def test_header_compiles_as_c99_and_errors_match_the_header():
    import fp8_compression_tensor_amd as tfp8

    tfp8.lib()  # the library must be built
    _build_module().build()  # gcc -std=c99 -Werror, links -ltfp8; no GPU needed
    r = _run("errors")
    assert r.returncode == 0 and "errors: ok" in r.stdout


def _files(d, **arrays):
    for name, a in arrays.items():
        np.ascontiguousarray(a).tofile(os.path.join(d, name))


def _load(d, name, dtype):
    return np.fromfile(os.path.join(d, name), dtype=dtype)


@pytest.mark.gpu
def test_c_caller_matches_the_oracle(oracle):
    assert os.path.exists(EXE), f"{EXE} is not built; run __graft_entry__.build()"
    wl = WORKLOADS[TINY]
    B, n, P, T = wl.block, wl.n, 3, 1.0
    xs = [make_shard(TINY, p).reshape(-1) for p in range(P)]
    with tempfile.TemporaryDirectory() as d:
        # compress
        _files(d, **{"x.bf16": xs[0]})
        r = _run("compress", d, n, B, T)
        assert r.returncode == 0, r.stdout
        q, a, s = _load(d, "codes.u8", np.uint8), _load(d, "alpha.f32", np.float32), \
            _load(d, "scale.f32", np.float32)
        qr, ar, sr, tr = oracle.compress(xs[0], B, T, with_quot=True)
        assert_codes_match(q, qr, tr, what="C caller compress codes")
        assert_rel_close(a, ar, 1e-6, what="C caller alpha")
        assert_rel_close(s, sr, 1e-6, what="C caller scale")

        # reduce of the oracle's compressed shards
        enc = [oracle.compress(x, B, T) for x in xs]
        _files(d, **{"in_codes.u8": np.stack([e[0] for e in enc]),
                     "in_alpha.f32": np.stack([e[1] for e in enc]),
                     "in_scale.f32": np.stack([e[2] for e in enc])})
        r = _run("reduce", d, n, B, T, P)
        assert r.returncode == 0, r.stdout
        rq, ra, rs, rt = oracle.reduce_fp8(np.stack([e[0] for e in enc]),
                                           np.stack([e[1] for e in enc]),
                                           np.stack([e[2] for e in enc]), B, T, with_quot=True)
        assert_codes_match(_load(d, "codes.u8", np.uint8), rq, rt, what="C caller reduce codes")
        assert_rel_close(_load(d, "alpha.f32", np.float32), ra, 1e-6, what="C caller reduce alpha")
        assert_rel_close(_load(d, "scale.f32", np.float32), rs, 1e-6, what="C caller reduce scale")

        # decompress of the oracle's compressed shard 0
        _files(d, **{"in_codes.u8": qr, "in_alpha.f32": ar, "in_scale.f32": sr})
        r = _run("decompress", d, n, B)
        assert r.returncode == 0, r.stdout
        assert_rel_close(_load(d, "out.f32", np.float32),
                         oracle.decompress(qr, ar, sr, B, np.float32), 1e-6, 2.0 ** -149,
                         what="C caller decompress")
