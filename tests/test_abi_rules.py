"""The argument rules of the C ABI (include/tfp8.h), as a property: from a valid argument set one
rule is broken at a time and the call must return that rule's status.

Hypothesis draws the block, the size, the data types, flags, target, P and the strides, and then
which rule to break and on which operand: an unsupported block, a bad size, data type, target,
flag bit, P or stride, a NULL pointer, a misaligned pointer or stride, or two operands that the
rules keep apart made to overlap.  The expected status comes from the header's table, not from the
library.  With n = 0 the pointer rules are not examined, so the same pointer-level breaks must
return TFP8_OK there.

Every call breaks exactly one rule, so none of them reaches a launch (a TFP8_E_HIP would show that
one was attempted).  The pointers are fake, so the module skips wherever a GPU is visible."""
import math

import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

OK, E_NULL, E_SIZE, E_BLOCK, E_DTYPE, E_ALIGN, E_ARG, E_HIP = 0, -1, -2, -3, -4, -5, -6, -7
MAX_N = 1 << 40
BASE = 0x7F0000000000  # fake device addresses, 16-byte aligned, never dereferenced
REGION = 1 << 28       # each operand in its own 256 MiB region: the largest span is ~2 MiB


def _no_gpu():
    try:
        import torch

        return torch.cuda.device_count() == 0  # counts devices without initialising HIP
    except Exception:
        return True


pytestmark = pytest.mark.skipif(not _no_gpu(), reason="calls with fake device pointers")


@pytest.fixture(scope="module")
def L():
    import fp8_compression_tensor_amd as m

    return m.lib()


# ----------------------------------------------------------------------------- the operations
# Each operation: its pointer operands with their alignment, their spans in bytes, the pairs of
# operands that may not overlap, the scalar rules it has, and a call that takes the arguments.

def _spans_compress(a):
    n, nb, es = a["n"], a["n"] // a["B"], 4 if a["dtype"] == 1 else 2
    return {"x": n * es, "codes": n, "alpha": 4 * nb, "scale": 4 * nb}


def _spans_decompress(a):
    n, nb, es = a["n"], a["n"] // a["B"], 4 if a["dtype"] == 1 else 2
    return {"codes": n, "alpha": 4 * nb, "scale": 4 * nb, "out": n * es}


def _spans_reduce(a):
    n, nb, P = a["n"], a["n"] // a["B"], a["P"]
    return {"codes": (P - 1) * a["cs"] + n, "alpha": 4 * ((P - 1) * a["as"] + nb),
            "scale": 4 * ((P - 1) * a["ss"] + nb), "codes_out": n, "alpha_out": 4 * nb,
            "scale_out": 4 * nb}


def _spans_accumulate(a):
    n, nb, es = a["n"], a["n"] // a["B"], 4 if a["dtype"] == 1 else 2
    return {"codes": n, "alpha": 4 * nb, "scale": 4 * nb, "grad": n * es, "codes_out": n,
            "alpha_out": 4 * nb, "scale_out": 4 * nb}


OPS = {
    "compress": dict(
        ptrs={"x": 16, "codes": 16, "alpha": 4, "scale": 4},
        spans=_spans_compress,
        # compress: no two of its buffers may overlap
        apart=[("x", "codes"), ("x", "alpha"), ("x", "scale"), ("codes", "alpha"),
               ("codes", "scale"), ("alpha", "scale")],
        scalars=("block", "size", "dtype", "target", "flags"),
        call=lambda L, a, p: L.tfp8_compress_ex(p["x"], a["dtype"], a["n"], a["B"], a["T"],
                                                a["flags"], p["codes"], p["alpha"], p["scale"],
                                                None)),
    "decompress": dict(
        ptrs={"codes": 16, "alpha": 4, "scale": 4, "out": 16},
        spans=_spans_decompress,
        # the output may overlap no input (the inputs are only read)
        apart=[("out", "codes"), ("out", "alpha"), ("out", "scale")],
        scalars=("block", "size", "dtype", "flags"),
        call=lambda L, a, p: L.tfp8_decompress_ex(p["codes"], p["alpha"], p["scale"], a["n"],
                                                  a["B"], a["flags"], p["out"], a["dtype"],
                                                  None)),
    "reduce": dict(
        ptrs={"codes": 16, "alpha": 4, "scale": 4, "codes_out": 16, "alpha_out": 4,
              "scale_out": 4},
        spans=_spans_reduce,
        # no output may overlap an input span or another output
        apart=[(o, i) for o in ("codes_out", "alpha_out", "scale_out")
               for i in ("codes", "alpha", "scale")] +
              [("codes_out", "alpha_out"), ("codes_out", "scale_out"), ("alpha_out", "scale_out")],
        scalars=("block", "size", "target", "flags", "P", "stride_small", "stride_big"),
        call=lambda L, a, p: L.tfp8_reduce_strided(p["codes"], a["cs"], p["alpha"], a["as"],
                                                   p["scale"], a["ss"], a["P"], a["n"], a["B"],
                                                   a["T"], a["flags"], p["codes_out"],
                                                   p["alpha_out"], p["scale_out"], None)),
    "accumulate": dict(
        ptrs={"codes": 16, "alpha": 4, "scale": 4, "grad": 16, "codes_out": 16, "alpha_out": 4,
              "scale_out": 4},
        spans=_spans_accumulate,
        # an output may be exactly its own input and overlap nothing else
        apart=[(o, i) for o in ("codes_out", "alpha_out", "scale_out")
               for i in ("codes", "alpha", "scale", "grad")] +
              [("codes_out", "alpha_out"), ("codes_out", "scale_out"), ("alpha_out", "scale_out")],
        in_place={("codes_out", "codes"), ("alpha_out", "alpha"), ("scale_out", "scale")},
        scalars=("block", "size", "dtype", "target", "flags"),
        call=lambda L, a, p: L.tfp8_accumulate(p["codes"], p["alpha"], p["scale"], p["grad"],
                                               a["dtype"], a["n"], a["B"], a["T"], a["flags"],
                                               p["codes_out"], p["alpha_out"], p["scale_out"],
                                               None)),
}

F32_ABOVE_2_64 = math.ldexp(1 + 2.0 ** -23, 64)    # the float32 just above 2^64
F32_BELOW_2_M64 = math.ldexp(1 - 2.0 ** -24, -64)  # the float32 just below 2^-64


@st.composite
def valid_args(draw, op):
    """A valid argument set for `op`, every pointer in its own region."""
    B = draw(st.sampled_from([64, 128, 256, 512]))
    nb = draw(st.integers(1, 64))
    a = {"B": B, "n": nb * B, "dtype": draw(st.sampled_from([0, 1])),
         "flags": draw(st.integers(0, 3)),
         "T": draw(st.one_of(st.sampled_from([2.0 ** -64, 1.0, 2.0 ** 64]),
                             st.floats(-64, 64).map(lambda e: 2.0 ** e)))}
    if op == "reduce":
        a["P"] = draw(st.integers(1, 64))
        a["cs"] = a["n"] + 16 * draw(st.integers(0, 64))
        a["as"] = nb + draw(st.integers(0, 64))
        a["ss"] = nb + draw(st.integers(0, 64))
    ptrs = {name: BASE + i * REGION for i, name in enumerate(OPS[op]["ptrs"])}
    return a, ptrs


BREAKS = ["block", "size", "dtype", "target", "flags", "P", "stride_small", "stride_big", "null",
          "align", "overlap"]


@st.composite
def one_break(draw, op):
    """(arguments, pointers, expected status, description) with exactly one rule broken."""
    spec = OPS[op]
    a, p = draw(valid_args(op))
    kinds = [k for k in BREAKS if k in spec["scalars"] or k in ("null", "align", "overlap")]
    kind = draw(st.sampled_from(kinds))
    if kind == "block":
        a["B"] = draw(st.sampled_from([0, 1, 32, 96, 100, 192, 1024, -128, 2 ** 31 - 1]))
        return a, p, E_BLOCK, f"block {a['B']}"
    if kind == "size":
        B = a["B"]
        a["n"] = draw(st.sampled_from([-B, a["n"] + draw(st.integers(1, B - 1)),
                                       (MAX_N // B + 1) * B, -1]))
        return a, p, E_SIZE, f"n {a['n']}"
    if kind == "dtype":
        a["dtype"] = draw(st.sampled_from([2, 3, -1, 255]))
        return a, p, E_DTYPE, f"dtype {a['dtype']}"
    if kind == "target":
        a["T"] = draw(st.sampled_from([0.0, -0.0, -1.0, 2.0 ** -65, 2.0 ** 65, F32_ABOVE_2_64,
                                       F32_BELOW_2_M64, math.inf, -math.inf, math.nan]))
        return a, p, E_ARG, f"target {a['T']}"
    if kind == "flags":
        a["flags"] |= draw(st.sampled_from([4, 8, 16, 1 << 31]))
        return a, p, E_ARG, f"flags {a['flags']:#x}"
    if kind == "P":
        a["P"] = draw(st.sampled_from([0, -1, 65, 1000]))
        return a, p, E_ARG, f"P {a['P']}"
    if kind == "stride_small":
        which = draw(st.sampled_from(["cs", "as", "ss"]))
        a[which] = a["n"] - 16 if which == "cs" else a["n"] // a["B"] - 1
        return a, p, E_ARG, f"{which} below the row"
    if kind == "stride_big":
        which = draw(st.sampled_from(["cs", "as", "ss"]))
        a[which] = MAX_N + 16
        return a, p, E_SIZE, f"{which} above 2^40"
    if kind == "null":
        name = draw(st.sampled_from(sorted(p)))
        p[name] = None
        return a, p, E_NULL, f"{name} NULL"
    if kind == "align":
        choices = sorted(p) + (["cs"] if op == "reduce" else [])
        name = draw(st.sampled_from(choices))
        if name == "cs":
            a["cs"] += draw(st.integers(1, 15))
            return a, p, E_ALIGN, "codes stride not a multiple of 16"
        al = spec["ptrs"][name]
        p[name] += draw(st.integers(1, al - 1))
        return a, p, E_ALIGN, f"{name} misaligned"
    # overlap: operand u moved onto the span of v, at an offset that keeps u aligned
    u, v = draw(st.sampled_from(spec["apart"]))
    if draw(st.booleans()):
        u, v = v, u  # either operand of the pair may be the one that moves
    spans = spec["spans"](a)
    al = spec["ptrs"][u]
    lo = -((spans[u] - 1) // al)        # u's end just past v's start
    hi = (spans[v] - 1) // al           # u's start just before v's end
    k = draw(st.integers(lo, hi))
    if (u, v) in spec.get("in_place", ()) or (v, u) in spec.get("in_place", ()):
        if k == 0:                      # exactly in place is allowed: move it off by one step
            k = 1 if hi >= 1 else -1
            if k == -1 and lo > -1:
                return one_break_fallback(a, p)
    p[u] = p[v] + k * al
    return a, p, E_ARG, f"{u} at {k * al:+d} bytes from {v}"


def one_break_fallback(a, p):
    # a one-block case whose in-place pair cannot be shifted: break the block instead
    a["B"] = 96
    return a, p, E_BLOCK, "block 96"


def _check(L, op, case):
    a, p, want, what = case
    got = OPS[op]["call"](L, a, p)
    assert got != E_HIP, f"{op}: {what}: the call reached a launch"
    assert got == want, f"{op}: {what}: status {got}, expected {want} ({a})"
    # with n = 0 the pointer rules are not examined
    if want in (E_NULL, E_ALIGN) or (want == E_ARG and what.split()[0] in p):
        a0 = dict(a, n=0)
        assert OPS[op]["call"](L, a0, p) == OK, f"{op}: {what} with n = 0"


_settings = settings(max_examples=800, deadline=None, derandomize=True)


@_settings
@given(case=one_break("compress"))
def test_compress_rules(L, case):
    _check(L, "compress", case)


@_settings
@given(case=one_break("decompress"))
def test_decompress_rules(L, case):
    _check(L, "decompress", case)


@_settings
@given(case=one_break("reduce"))
def test_reduce_strided_rules(L, case):
    _check(L, "reduce", case)


@_settings
@given(case=one_break("accumulate"))
def test_accumulate_rules(L, case):
    _check(L, "accumulate", case)
