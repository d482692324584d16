"""ctypes front end of the plain FP64 CPU oracle (tfp8_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg import this package; the product path never does, and nothing here imports
the product package.  Arguments are numpy arrays on the host; every function returns new
arrays and raises ``ValueError`` carrying the oracle's status code on bad arguments.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
BF16, F32 = 0, 1
INT8, NO_ROTATION = 1, 2  # variant flags of the *_ex oracle entry points

_lib = None


def lib():
    """Load the compiled oracle, building it first only if it is missing."""
    global _lib
    if _lib is None:
        # TFP8_ORACLE_LIB lets the mutation test load a deliberately broken copy instead.
        path = os.environ.get("TFP8_ORACLE_LIB", _build.LIB)
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        L.tfp8_ref_e4m3_encode.argtypes = [ctypes.c_double]
        L.tfp8_ref_e4m3_encode.restype = ctypes.c_uint8
        L.tfp8_ref_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.tfp8_ref_e4m3_decode.restype = ctypes.c_double
        L.tfp8_ref_round_bf16.argtypes = [ctypes.c_double]
        L.tfp8_ref_round_bf16.restype = ctypes.c_uint16
        L.tfp8_ref_hadamard_entry.argtypes = [i64, i64]
        L.tfp8_ref_hadamard_entry.restype = i32
        L.tfp8_ref_fwht.argtypes = [vp, i64]
        L.tfp8_ref_fwht.restype = None
        L.tfp8_ref_hadamard_dense.argtypes = [vp, i64, vp]
        L.tfp8_ref_hadamard_dense.restype = None
        L.tfp8_ref_compress.argtypes = [vp, i32, i64, i32, f32, vp, vp, vp, vp]
        L.tfp8_ref_compress_unrounded.argtypes = [vp, i32, i64, i32, f32, vp, vp, vp]
        L.tfp8_ref_decompress.argtypes = [vp, vp, vp, i64, i32, vp, i32]
        L.tfp8_ref_decompress_f64.argtypes = [vp, vp, vp, i64, i32, vp]
        L.tfp8_ref_decompress_unrounded.argtypes = [vp, vp, vp, i64, i32, vp]
        L.tfp8_ref_reduce_fp8.argtypes = [vp, vp, vp, i32, i64, i32, f32, vp, vp, vp, vp]
        L.tfp8_ref_reduce_fp8_rotated.argtypes = [vp, vp, vp, i32, i64, i32, f32, vp, vp, vp, vp]
        L.tfp8_ref_int8_encode.argtypes = [ctypes.c_double]
        L.tfp8_ref_int8_encode.restype = ctypes.c_uint8
        L.tfp8_ref_int8_decode.argtypes = [ctypes.c_uint8]
        L.tfp8_ref_int8_decode.restype = ctypes.c_double
        L.tfp8_ref_compress_ex.argtypes = [vp, i32, i64, i32, f32, i32, vp, vp, vp, vp]
        L.tfp8_ref_decompress_ex.argtypes = [vp, vp, vp, i64, i32, i32, vp, i32]
        L.tfp8_ref_decompress_f64_ex.argtypes = [vp, vp, vp, i64, i32, i32, vp]
        L.tfp8_ref_reduce_ex.argtypes = [vp, vp, vp, i32, i64, i32, f32, i32, vp, vp, vp, vp]
        L.tfp8_ref_reduce_rotated_ex.argtypes = [vp, vp, vp, i32, i64, i32, f32, i32, vp, vp, vp, vp]
        L.tfp8_ref_accumulate_ex.argtypes = [vp, vp, vp, vp, i32, i64, i32, f32, i32, vp, vp, vp, vp]
        L.tfp8_ref_accumulate_rotated_ex.argtypes = [vp, vp, vp, vp, i32, i64, i32, f32, i32, vp, vp,
                                                     vp, vp]
        L.tfp8_ref_set_threads.argtypes = [i32]
        L.tfp8_ref_set_threads.restype = i32
        _lib = L
    return _lib


def set_threads(n: int) -> int:
    return lib().tfp8_ref_set_threads(int(n))


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(st):
    if st != 0:
        raise ValueError(f"oracle status {st}")


def _input(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x.reshape(-1), BF16
    if x.dtype == np.float32:
        return x.reshape(-1), F32
    raise TypeError("oracle input must be bfloat16 bits (uint16) or float32")


def e4m3_encode(v: float) -> int:
    return int(lib().tfp8_ref_e4m3_encode(float(v)))


def e4m3_decode(c: int) -> float:
    return float(lib().tfp8_ref_e4m3_decode(int(c)))


def e4m3_decode_table() -> np.ndarray:
    return np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


def int8_encode(v: float) -> int:
    return int(lib().tfp8_ref_int8_encode(float(v)))


def int8_decode(c: int) -> float:
    return float(lib().tfp8_ref_int8_decode(int(c)))


def round_bf16(v: float) -> int:
    return int(lib().tfp8_ref_round_bf16(float(v)))


def hadamard_entry(i: int, j: int) -> int:
    return int(lib().tfp8_ref_hadamard_entry(int(i), int(j)))


def fwht(v: np.ndarray) -> np.ndarray:
    out = np.array(v, dtype=np.float64, copy=True)
    lib().tfp8_ref_fwht(_ptr(out), out.size)
    return out


def hadamard_dense(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty_like(v)
    lib().tfp8_ref_hadamard_dense(_ptr(v), v.size, _ptr(out))
    return out


def compress(x, block: int, target: float = 1.0, with_quot: bool = False, flags: int = 0):
    """-> codes uint8[n], alpha f32[nb], scale f32[nb] (+ quot f64[n] if with_quot)."""
    x, dt = _input(x)
    n = x.size
    nb = n // block if block > 0 else 0
    codes = np.empty(n, np.uint8)
    alpha = np.empty(nb, np.float32)
    scale = np.empty(nb, np.float32)
    quot = np.empty(n, np.float64) if with_quot else None
    _check(lib().tfp8_ref_compress_ex(_ptr(x), dt, n, block, target, flags, _ptr(codes), _ptr(alpha),
                                      _ptr(scale), _ptr(quot)))
    return (codes, alpha, scale, quot) if with_quot else (codes, alpha, scale)


def compress_unrounded(x, block: int, target: float = 1.0):
    x, dt = _input(x)
    n = x.size
    t = np.empty(n, np.float64)
    alpha = np.empty(n // block, np.float32)
    scale = np.empty(n // block, np.float32)
    _check(lib().tfp8_ref_compress_unrounded(_ptr(x), dt, n, block, target, _ptr(t), _ptr(alpha),
                                             _ptr(scale)))
    return t, alpha, scale


def decompress(codes, alpha, scale, block: int, out_dtype=np.float32, flags: int = 0):
    codes = np.ascontiguousarray(codes, np.uint8).reshape(-1)
    alpha = np.ascontiguousarray(alpha, np.float32)
    scale = np.ascontiguousarray(scale, np.float32)
    n = codes.size
    if out_dtype == np.float32:
        out, dt = np.empty(n, np.float32), F32
    else:
        out, dt = np.empty(n, np.uint16), BF16
    _check(lib().tfp8_ref_decompress_ex(_ptr(codes), _ptr(alpha), _ptr(scale), n, block, flags,
                                        _ptr(out), dt))
    return out


def decompress_f64(codes, alpha, scale, block: int, flags: int = 0):
    codes = np.ascontiguousarray(codes, np.uint8).reshape(-1)
    alpha = np.ascontiguousarray(alpha, np.float32)
    scale = np.ascontiguousarray(scale, np.float32)
    out = np.empty(codes.size, np.float64)
    _check(lib().tfp8_ref_decompress_f64_ex(_ptr(codes), _ptr(alpha), _ptr(scale), codes.size,
                                            block, flags, _ptr(out)))
    return out


def decompress_unrounded(t, alpha, scale, block: int):
    t = np.ascontiguousarray(t, np.float64)
    alpha = np.ascontiguousarray(alpha, np.float32)
    scale = np.ascontiguousarray(scale, np.float32)
    out = np.empty(t.size, np.float64)
    _check(lib().tfp8_ref_decompress_unrounded(_ptr(t), _ptr(alpha), _ptr(scale), t.size, block,
                                               _ptr(out)))
    return out


def _reduce(fn, codes, alpha, scale, block, target, with_quot, flags):
    codes = np.ascontiguousarray(codes, np.uint8)
    P = codes.shape[0]
    codes = codes.reshape(P, -1)
    n = codes.shape[1]
    alpha = np.ascontiguousarray(alpha, np.float32).reshape(P, -1)
    scale = np.ascontiguousarray(scale, np.float32).reshape(P, -1)
    qo = np.empty(n, np.uint8)
    ao = np.empty(n // block, np.float32)
    so = np.empty(n // block, np.float32)
    quot = np.empty(n, np.float64) if with_quot else None
    _check(fn(_ptr(codes), _ptr(alpha), _ptr(scale), P, n, block, target, flags, _ptr(qo), _ptr(ao),
              _ptr(so), _ptr(quot)))
    return (qo, ao, so, quot) if with_quot else (qo, ao, so)


def reduce_fp8(codes, alpha, scale, block: int, target: float = 1.0, with_quot: bool = False,
               flags: int = 0):
    """codes [P, n], alpha/scale [P, nb] -> codes [n], alpha [nb], scale [nb] (by definition)."""
    return _reduce(lib().tfp8_ref_reduce_ex, codes, alpha, scale, block, target, with_quot, flags)


def reduce_fp8_rotated(codes, alpha, scale, block: int, target: float = 1.0, with_quot: bool = False,
                       flags: int = 0):
    """Same result by the rotated-domain route (no Hadamard)."""
    return _reduce(lib().tfp8_ref_reduce_rotated_ex, codes, alpha, scale, block, target, with_quot,
                   flags)


def _accumulate(fn, codes, alpha, scale, grad, block, target, with_quot, flags):
    codes = np.ascontiguousarray(codes, np.uint8).reshape(-1)
    alpha = np.ascontiguousarray(alpha, np.float32)
    scale = np.ascontiguousarray(scale, np.float32)
    grad, gdt = _input(grad)
    n = codes.size
    qo = np.empty(n, np.uint8)
    ao = np.empty(n // block, np.float32)
    so = np.empty(n // block, np.float32)
    quot = np.empty(n, np.float64) if with_quot else None
    _check(fn(_ptr(codes), _ptr(alpha), _ptr(scale), _ptr(grad), gdt, n, block, target, flags,
              _ptr(qo), _ptr(ao), _ptr(so), _ptr(quot)))
    return (qo, ao, so, quot) if with_quot else (qo, ao, so)


def accumulate(codes, alpha, scale, grad, block: int, target: float = 1.0, with_quot: bool = False,
               flags: int = 0):
    """Compressed main gradient + dense local gradient (bf16 bits or fp32) -> compressed sum."""
    return _accumulate(lib().tfp8_ref_accumulate_ex, codes, alpha, scale, grad, block, target,
                       with_quot, flags)


def accumulate_rotated(codes, alpha, scale, grad, block: int, target: float = 1.0,
                       with_quot: bool = False, flags: int = 0):
    """Same result formed in the rotated domain."""
    return _accumulate(lib().tfp8_ref_accumulate_rotated_ex, codes, alpha, scale, grad, block,
                       target, with_quot, flags)


def raw_status(name: str, *args) -> int:
    """Call an oracle entry point with raw arguments and return its status (argument tests)."""
    return int(getattr(lib(), name)(*args))
