"""The oracle's pins are strong enough to notice plausible mistakes.

Each case plants one mistake in a temporary copy of the oracle's C source (a dropped term,
a wrong sign, a swapped operand, a wrong constant, an off-by-one index), builds it, and runs
the oracle pin suites against the broken build in a fresh process.  Every mutant must fail
at least one pin.  The real oracle is never modified.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "tfp8_oracle.c")

# (name, text to find, replacement, occurrence index to replace: 0 = first)
MUTANTS = [
    ("m2 without /B", "double m2 = sumsq / B;", "double m2 = sumsq;", 0),
    ("alpha from m2/T", "double a = sqrt(T / m2);", "double a = sqrt(m2 / T);", 0),
    ("no alpha clamp", "a = fmin(fmax(a, 0x1p-126), 0x1p126);\n  float alpha", "\n  float alpha", 0),
    ("prescale dropped", "y[i] = (double)alpha * v[i];", "y[i] = v[i];", 0),
    ("butterfly sign", "v[j + h] = a - b;", "v[j + h] = b - a;", 0),
    ("Hadamard entry or", "(i & j)", "(i | j)", 0),
    ("no 1/sqrt(B)", "for (int i = 0; i < B; ++i) y[i] = y[i] / rootB;", "", 0),
    ("Qmax 240", "? 127.0 : 448.0", "? 127.0 : 240.0", 0),
    ("encode half-up", "double k = nearbyint(ldexp(a, 3 - E));",
     "double k = floor(ldexp(a, 3 - E) + 0.5);", 0),
    ("encode subnormal half-up", "nearbyint(a * 512.0)", "floor(a * 512.0 + 0.5)", 0),
    ("encode loses -0", "uint8_t sign = signbit(v) ? 0x80 : 0x00;",
     "uint8_t sign = (v < 0) ? 0x80 : 0x00;", 0),
    ("encode no saturation", "if (!(a <= 448.0)) return sign | 0x7E;", "", 0),
    ("decode subnormal step", "ldexp((double)m, -9)", "ldexp((double)m, -10)", 0),
    ("decode bias", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)", 0),
    ("bf16 round half-up", "double r = nearbyint(a / step) * step;",
     "double r = floor(a / step + 0.5) * step;", 0),
    ("zero block alpha 0", "*alpha_out = 1.0f;", "*alpha_out = 0.0f;", 0),
    ("decompress no 1/alpha", "for (int i = 0; i < B; ++i) out[i] = out[i] / (double)alpha;",
     "", 0),
    ("decompress times alpha", "out[i] = out[i] / (double)alpha;",
     "out[i] = out[i] * (double)alpha;", 0),
    ("decompress no rotation", "  tfp8_ref_fwht(out, B);\n", "\n", 0),
    ("decompress scale dropped", "out[i] = (double)scale * cval[i];", "out[i] = cval[i];", 0),
    ("reduce drops last", "for (int p = 0; p < P; ++p) {\n      const uint8_t *q",
     "for (int p = 0; p < P - 1; ++p) {\n      const uint8_t *q", 0),
    ("reduce wrong scale index", "decompress_block(c, alpha[(int64_t)p * nb + k], scale[(int64_t)p * nb + k]",
     "decompress_block(c, alpha[k], scale[k]", 0),
    ("rotated reduce s/alpha swapped", "double g = (double)s / (double)alpha[(int64_t)p * nb + k];",
     "double g = (double)alpha[(int64_t)p * nb + k] / (double)s;", 0),
    ("rotated reduce no /Qmax", "double Q = code_qmax(flags);", "double Q = 1.0;", 0),
    ("INT8 Qmax 128", "? 127.0 : 448.0", "? 128.0 : 448.0", 0),
    ("INT8 decode unsigned", "return (double)(int8_t)code;", "return (double)code;", 0),
    ("INT8 encode half-up", "double k = nearbyint(v);", "double k = floor(v + 0.5);", 0),
    ("INT8 values decoded as E4M3",
     "return (flags & TFP8_REF_INT8) ? tfp8_ref_int8_decode(code) : tfp8_ref_e4m3_decode(code);",
     "return tfp8_ref_e4m3_decode(code);", 0),
    ("compress ignores no-rotation", "if (!(flags & TFP8_REF_NO_ROTATION)) {\n    tfp8_ref_fwht(y, B);",
     "if (1) {\n    tfp8_ref_fwht(y, B);", 0),
    ("accumulate drops the local gradient",
     "for (int i = 0; i < block; ++i) z[i] += load_elem(grad, grad_dtype, k * block + i);", "", 0),
    ("rotated accumulate drops sqrt(B)", "if (rotate) g *= rootB;", "", 0),
    ("decompress ignores no-rotation",
     "if (!(flags & TFP8_REF_NO_ROTATION)) {\n    tfp8_ref_fwht(out, B);",
     "if (1) {\n    tfp8_ref_fwht(out, B);", 0),
    ("post-scale from the unrotated input", "for (int i = 0; i < B; ++i) my = fmax(my, fabs(y[i]));",
     "for (int i = 0; i < B; ++i) my = fmax(my, fabs(v[i]));", 0),
    ("quotient with the unrounded scale", "double t = y[i] / (double)s;",
     "double t = y[i] * code_qmax(flags) / my;", 0),
    ("reduce averages", "for (int i = 0; i < block; ++i) z[i] += xh[i];",
     "for (int i = 0; i < block; ++i) z[i] += xh[i] / P;", 0),
    ("reduce ignores the target",
     "compress_block(z, block, (double)target, flags, codes_out + k * block, alpha_out + k,",
     "compress_block(z, block, 1.0, flags, codes_out + k * block, alpha_out + k,", 0),
    ("reduce decodes variant codes as E4M3", "for (int i = 0; i < block; ++i) c[i] = code_value(q[i], flags);",
     "for (int i = 0; i < block; ++i) c[i] = code_value(q[i], 0);", 0),
    ("rotated reduce energy without 1/B", "double a = sqrt(T / (sumsq / block));",
     "double a = sqrt(T / sumsq);", 0),
    ("rotated reduce quotient without alpha", "double t = (double)alpha2 * r[i] / (double)s2;",
     "double t = r[i] / (double)s2;", 0),
    ("accumulate ignores the target",
     "compress_block(z, block, (double)target, flags, codes_out + k * block, alpha_out + k,",
     "compress_block(z, block, 1.0, flags, codes_out + k * block, alpha_out + k,", 1),
    ("accumulate subtracts the local gradient",
     "for (int i = 0; i < block; ++i) z[i] += load_elem(grad, grad_dtype, k * block + i);",
     "for (int i = 0; i < block; ++i) z[i] -= load_elem(grad, grad_dtype, k * block + i);", 0),
    ("accumulate reads block 0's scales", "decompress_block(c, alpha[k], scale[k], block, flags, z);",
     "decompress_block(c, alpha[0], scale[0], block, flags, z);", 0),
    ("accumulate decodes variant codes as E4M3",
     "for (int i = 0; i < block; ++i) c[i] = code_value(codes[k * block + i], flags);",
     "for (int i = 0; i < block; ++i) c[i] = code_value(codes[k * block + i], 0);", 0),
    ("rotated accumulate energy without the rotation's 1/B",
     "double m2 = (rotate ? sumsq / block : sumsq) / block;", "double m2 = sumsq / block;", 0),
    ("INT8 saturates at 128", "if (k > 127.0) k = 127.0;", "if (k > 128.0) k = 128.0;", 0),
    ("INT8 no negative saturation", "if (k < -127.0) k = -127.0;", "", 0),
    ("energy from |x|", "for (int i = 0; i < B; ++i) sumsq += v[i] * v[i];",
     "for (int i = 0; i < B; ++i) sumsq += fabs(v[i]);", 0),
    ("FWHT misses its last stage", "for (int64_t h = 1; h < len; h <<= 1)",
     "for (int64_t h = 1; h < len / 2; h <<= 1)", 0),
    ("bf16 widened by 15 bits", "uint32_t u = (uint32_t)((const uint16_t *)x)[i] << 16;",
     "uint32_t u = (uint32_t)((const uint16_t *)x)[i] << 15;", 0),
    ("alpha clamp at 2^-127", "a = fmin(fmax(a, 0x1p-126), 0x1p126);\n  float alpha",
     "a = fmin(fmax(a, 0x1p-127), 0x1p126);\n  float alpha", 0),
    ("prescale with the unrounded alpha", "y[i] = (double)alpha * v[i];", "y[i] = a * v[i];", 0),
    ("zero test on the first element", "for (int i = 0; i < B; ++i) ax = fmax(ax, fabs(v[i]));",
     "ax = fabs(v[0]);", 0),
    ("encode subnormal range ends at 2^-7", "if (a < 0x1p-6) {", "if (a < 0x1p-7) {", 0),
    ("encode exponent carry dropped", "if (k == 16.0) {\n    E += 1;", "if (k == 16.0) {\n    E += 0;", 0),
    ("decode NaN pattern ignored", "if (e == 15 && m == 7) return NAN;", "", 0),
    ("bf16 output truncated", "double r = nearbyint(a / step) * step;",
     "double r = trunc(a / step) * step;", 0),
    ("bf16 subnormal step 2^-134", "double step = (E < -126) ? 0x1p-133 : ldexp(1.0, E - 7);",
     "double step = (E < -126) ? 0x1p-134 : ldexp(1.0, E - 7);", 0),
    ("decompress divides by B", "for (int i = 0; i < B; ++i) out[i] = out[i] / rootB;\n  }\n  for",
     "for (int i = 0; i < B; ++i) out[i] = out[i] / B;\n  }\n  for", 0),
    ("decompress zero block left undefined", "for (int i = 0; i < B; ++i) out[i] = 0.0;\n    return;",
     "return;", 0),
    ("reduce sums in reverse order",
     "    for (int p = 0; p < P; ++p) {\n      const uint8_t *q = codes + (int64_t)p * n + k * block;",
     "    for (int p = P - 1; p >= 0; --p) {\n      const uint8_t *q = codes + (int64_t)p * n + k * block;",
     0),
    ("rotated reduce sums in reverse order", "    for (int p = 0; p < P; ++p) {\n      float s = scale[",
     "    for (int p = P - 1; p >= 0; --p) {\n      float s = scale[", 0),
    ("bf16 subnormal range ends at 2^-127", "double step = (E < -126) ?", "double step = (E < -127) ?", 0),
    ("accumulate reads a float32 gradient as bfloat16",
     "z[i] += load_elem(grad, grad_dtype, k * block + i);",
     "z[i] += load_elem(grad, TFP8_REF_BF16, k * block + i);", 0),
    ("rotated accumulate reads a float32 gradient as bfloat16",
     "w[i] = load_elem(grad, grad_dtype, k * block + i);",
     "w[i] = load_elem(grad, TFP8_REF_BF16, k * block + i);", 0),
    ("rotated accumulate post-scale without 1/sqrt(B)",
     "float s2 = (float)((double)alpha2 * aw / div / Q);",
     "float s2 = (float)((double)alpha2 * aw / Q);", 0),
    ("compress max misses the last element",
     "for (int i = 0; i < B; ++i) my = fmax(my, fabs(y[i]));",
     "for (int i = 0; i < B - 1; ++i) my = fmax(my, fabs(y[i]));", 0),
    ("compress energy misses the last element",
     "for (int i = 0; i < B; ++i) sumsq += v[i] * v[i];",
     "for (int i = 0; i < B - 1; ++i) sumsq += v[i] * v[i];", 0),
    ("rotated reduce quotient with the unrounded alpha",
     "double t = (double)alpha2 * r[i] / (double)s2;", "double t = a * r[i] / (double)s2;", 0),
    ("rotated reduce scale with the unrounded alpha",
     "float s2 = (float)((double)alpha2 * ar / Q);", "float s2 = (float)(a * ar / Q);", 0),
    ("scale rounded twice", "float s = (float)(my / code_qmax(flags));",
     "float s = (float)my / (float)code_qmax(flags);", 0),
    ("INT8 encode half away from zero", "double k = nearbyint(v);", "double k = round(v);", 0),
    ("reduce reconstructs variant codes with the rotation",
     "scale[(int64_t)p * nb + k], block, flags, xh);",
     "scale[(int64_t)p * nb + k], block, flags & TFP8_REF_INT8, xh);", 0),
    ("rotated accumulate quotient with the unrounded alpha",
     "double t = (double)alpha2 * w[i] / div / (double)s2;",
     "double t = a * w[i] / div / (double)s2;", 0),
    ("rotated accumulate scale with the unrounded alpha",
     "float s2 = (float)((double)alpha2 * aw / div / Q);", "float s2 = (float)(a * aw / div / Q);", 0),
    ("decompress to bf16 rounds twice",
     "((uint16_t *)out)[k * block + i] = tfp8_ref_round_bf16(r[i]);",
     "((uint16_t *)out)[k * block + i] = tfp8_ref_round_bf16((double)(float)r[i]);", 0),
    ("compress reads float32 input as bfloat16",
     "v[i] = load_elem(x, x_dtype, k * block + i);\n    compress_block(v, block, (double)target, flags,",
     "v[i] = load_elem(x, TFP8_REF_BF16, k * block + i);\n    compress_block(v, block, (double)target, flags,",
     0),
    ("alpha clamp at 2^127", "a = fmin(fmax(a, 0x1p-126), 0x1p126);",
     "a = fmin(fmax(a, 0x1p-126), 0x1p127);", 0),
    ("rotated reduce alpha clamp at 2^127", "a = fmin(fmax(a, 0x1p-126), 0x1p126);",
     "a = fmin(fmax(a, 0x1p-126), 0x1p127);", 1),
    ("rotated accumulate alpha clamp at 2^127", "a = fmin(fmax(a, 0x1p-126), 0x1p126);",
     "a = fmin(fmax(a, 0x1p-126), 0x1p127);", 2),
    ("target lower bound exclusive", "!(target >= 0x1p-64f)", "!(target > 0x1p-64f)", 0),
    ("target upper bound exclusive", "!(target <= 0x1p64f)", "!(target < 0x1p64f)", 0),
    ("reduce accepts P = 0", "if (P < 1) return TFP8_REF_E_ARG;", "if (P < 0) return TFP8_REF_E_ARG;", 0),
]


def _apply(src, find, repl, occ):
    idx = -1
    for _ in range(occ + 1):
        idx = src.find(find, idx + 1)
        assert idx >= 0, f"mutation anchor not found: {find!r}"
    return src[:idx] + repl + src[idx + len(find):]


def _run_mutant(case, tmpdir):
    name, find, repl, occ = case
    sys.path.insert(0, os.path.join(ROOT, "oracle"))
    import build as oracle_build

    src = open(SRC).read()
    mutated = _apply(src, find, repl, occ)
    assert mutated != src
    d = os.path.join(tmpdir, name.replace(" ", "_").replace("/", "_"))
    os.makedirs(d)
    msrc = os.path.join(d, "tfp8_oracle.c")
    with open(msrc, "w") as f:
        f.write(mutated)
    lib = oracle_build.build(src=msrc, out=os.path.join(d, "libmutant.so"))
    env = dict(os.environ, TFP8_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_oracle_codec.py"),
           os.path.join(ROOT, "tests", "test_oracle_method.py"),
           os.path.join(ROOT, "tests", "test_oracle_variants.py"),
           os.path.join(ROOT, "tests", "test_oracle_accumulate.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    return name, r.returncode, r.stdout[-1500:]


def test_every_mutant_is_caught():
    from concurrent.futures import ThreadPoolExecutor

    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with tempfile.TemporaryDirectory() as tmp, ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda c: _run_mutant(c, tmp), MUTANTS))
    survivors = [(n, out) for n, rc, out in results if rc != 1]
    assert not survivors, "mutants not caught by the oracle pins: " + "; ".join(
        f"{n}: {out}" for n, out in survivors)
