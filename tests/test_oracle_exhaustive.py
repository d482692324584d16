"""The oracle's E4M3FN encoder on every float32 bit pattern (2^32 of them, NaNs skipped) against a
brute-force nearest-value search written from the format definition alone
(tests/c_exhaustive/e4m3_all_float32.c).  Runs on the CPU, in parallel over the cores, in about
15 s on 8 of them."""
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_exhaustive", "e4m3_all_float32.c")


def test_e4m3_encoder_on_every_float32(oracle):
    oracle.lib()  # the oracle library (built first if it is missing)
    odir = os.path.join(ROOT, "oracle")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "e4m3_all_float32")
        subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-Wall", "-Wextra", "-Werror",
                        "-I", odir, "-o", exe, SRC, "-L", odir, "-ltfp8_oracle",
                        "-Wl,-rpath," + odir, "-lm"], check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0 and r.stdout.startswith("ok "), r.stdout + r.stderr
    assert int(r.stdout.split()[1]) == (1 << 32) - 2 * ((1 << 23) - 1)  # every non-NaN pattern
