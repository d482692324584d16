"""The generated gfx950 code of every kernel keeps the wait states that the inline asm relies on.

The compiler inserts hardware wait states only around instructions it emits itself; the library's
inline asm (the DPP butterflies and the bfloat16 widening with v_dot2_f32_bf16) has to provide its
own.  This test compiles the kernels to assembly (hipcc, no GPU needed) and checks, in every
kernel, two rules of the CDNA3/CDNA4 instruction set:
  * a VALU result read as the DPP source operand needs 2 wait states;
  * a DOT result (v_dot*) must not be read or overwritten by another VALU instruction for 3 wait
    states.
A wait state is an instruction issued in between, or s_nop n (n + 1 states)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "fp8_compression_tensor_amd", "csrc", "tfp8_kernels.hip")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")


def _kernel_bodies(out, extra=()):
    """Instructions of every kernel in the gfx950 assembly of the library's source, compiled with
    the library's build flags (plus `extra`), by kernel symbol."""
    import importlib.util

    # the library's build flags, loaded under a private name (no sys.path or module clash)
    spec = importlib.util.spec_from_file_location(
        "_tfp8_lib_build", os.path.join(ROOT, "fp8_compression_tensor_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    HIPCC_FLAGS = mod.HIPCC_FLAGS

    flags = [f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    r = subprocess.run(["hipcc", *flags, *extra, "--cuda-device-only", "-S", "-o", out, SRC],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = open(out).read().split("\n")
    bodies, cur, name = {}, None, None
    for line in text:
        m = re.match(r"^(_ZN4tfp8\w*k_\w+):", line)
        if m:
            name, cur = m.group(1), []
            continue
        if cur is not None:
            if "s_endpgm" in line:
                bodies[name] = cur
                cur = None
                continue
            ins = line.split(";")[0].strip()
            if ins and not ins.startswith(".") and not ins.endswith(":"):
                cur.append(ins)
    return bodies


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    return _kernel_bodies(str(tmp_path_factory.mktemp("asm") / "k.s"))


def _regs(tok):
    tok = tok.strip().split(" ")[0].strip("|-")
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _parse(ins):
    op, _, rest = ins.partition(" ")
    ops = [t.strip() for t in rest.split(",")] if rest else []
    return op, ops


def _states(op, ops):
    return int(ops[0], 0) + 1 if op == "s_nop" else 1


def test_kernels_were_found(kernels):
    names = " ".join(kernels)
    for k in ("k_compress", "k_decompress", "k_reduce", "k_accumulate", "k_accumulate_fix"):
        assert k in names


def test_dpp_sources_are_not_written_in_the_two_states_before(kernels):
    bad = []
    for name, body in kernels.items():
        parsed = [_parse(i) for i in body]
        for i, (op, ops) in enumerate(parsed):
            if "_dpp" not in op or len(ops) < 2:
                continue
            src = _regs(ops[1])
            waited = 0
            for pop, pops in reversed(parsed[max(0, i - 4):i]):
                if pop.startswith("v_") and pops and _regs(pops[0]) & src:
                    if waited < 2:
                        bad.append((name, " ".join([pop] + pops), op))
                    break
                waited += _states(pop, pops)
                if waited >= 2:
                    break
    assert not bad, bad[:5]


def test_dot_results_wait_three_states(kernels):
    bad, checked = [], 0
    for name, body in kernels.items():
        parsed = [_parse(i) for i in body]
        for i, (op, ops) in enumerate(parsed):
            if not op.startswith("v_dot"):
                continue
            checked += 1
            dst = _regs(ops[0])
            waited = 0
            for nop, nops in parsed[i + 1:i + 6]:
                if nop.startswith("v_") and not nop.startswith("v_dot"):
                    used = set().union(*[_regs(t) for t in nops]) if nops else set()
                    if used & dst and waited < 3:
                        bad.append((name, op, nop))
                        break
                waited += _states(nop, nops)
                if waited >= 3:
                    break
    assert checked > 0
    assert not bad, bad[:5]


def test_capped_test_build_has_the_same_kernels(kernels, tmp_path):
    # The GPU tests of the grid-stride loops use a second build of the library with every launch
    # capped at one workgroup per compute unit (tests/capped_build).  The caps only change the
    # host's choice of grid: every kernel must compile to the same instructions.
    import importlib.util

    spec = importlib.util.spec_from_file_location(
        "_tfp8_capped_build", os.path.join(ROOT, "tests", "capped_build", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    capped = _kernel_bodies(str(tmp_path / "capped.s"), mod.CAPS)
    assert sorted(capped) == sorted(kernels)
    assert all(capped[k] == kernels[k] for k in kernels)
