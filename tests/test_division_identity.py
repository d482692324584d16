"""The float64 division by reciprocal plus one FMA correction that the accumulation's exact pass
uses, checked on the host against correctly rounded division (tests/c_division/div_by_reciprocal.c,
2*10^7 cases of the pass's shape, about a second)."""
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "c_division", "div_by_reciprocal.c")


def test_reciprocal_division_is_correctly_rounded():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "div_by_reciprocal")
        # -ffp-contract=off: m * y stays a separately rounded product (libm's fma is exact)
        subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-Wall",
                        "-Wextra", "-Werror", "-o", exe, SRC, "-lm"], check=True)
        r = subprocess.run([exe, "20000000"], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0 and r.stdout.startswith("ok "), r.stdout + r.stderr
