"""FP8 E4M3 (ASH + DS) compression of tensor-parallel tensors on MI355X (gfx950).

Thin binding of the C ABI in ``include/tfp8.h`` (``libtfp8.so``, built in this directory by
``build.py``).  This module only marshals arguments: PyTorch supplies device memory and the
current HIP stream, and every step of compress, decompress, the reduce and the accumulation runs
in the library's kernels.  There is no CPU path: without the built library, or for tensors not
on a GPU, the calls raise.

Method: page "TACO: Efficient Communication Compression of Intermediate Tensors for Scalable
Tensor-Parallel LLM Training" (section 2.B.1-2.B.2); local reduce and gradient accumulation:
page "AGoQ: Activation and Gradient Quantization for Memory-Efficient Distributed Training of
LLMs" (section 2.B).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "compress", "decompress", "reduce_fp8", "compress_raw", "decompress_raw", "reduce_fp8_raw",
    "status_string", "lib", "LIB_PATH", "TFP8Error", "BF16", "F32", "SUPPORTED_BLOCKS",
    "FLAG_INT8", "FLAG_NO_ROTATION", "accumulate", "accumulate_raw", "reduce_strided_raw",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtfp8.so")
BF16, F32 = 0, 1
FLAG_INT8, FLAG_NO_ROTATION = 1, 2  # variant flags of the *_ex entry points (include/tfp8.h)
SUPPORTED_BLOCKS = (64, 128, 256, 512)

_STATUS = {0: "TFP8_OK", -1: "TFP8_E_NULL", -2: "TFP8_E_SIZE", -3: "TFP8_E_BLOCK",
           -4: "TFP8_E_DTYPE", -5: "TFP8_E_ALIGN", -6: "TFP8_E_ARG", -7: "TFP8_E_HIP"}


class TFP8Error(RuntimeError):
    """A status other than TFP8_OK; ``.status`` holds the code."""

    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def _declare(L: ctypes.CDLL) -> ctypes.CDLL:
    """Argument and result types of the C ABI's entry points on an opened build of the library."""
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    L.tfp8_compress.argtypes = [vp, i32, i64, i32, f32, vp, vp, vp, vp]
    L.tfp8_compress.restype = i32
    L.tfp8_decompress.argtypes = [vp, vp, vp, i64, i32, vp, i32, vp]
    L.tfp8_decompress.restype = i32
    L.tfp8_reduce_fp8.argtypes = [vp, vp, vp, i32, i64, i32, f32, vp, vp, vp, vp]
    L.tfp8_reduce_fp8.restype = i32
    u32 = ctypes.c_uint32
    L.tfp8_compress_ex.argtypes = [vp, i32, i64, i32, f32, u32, vp, vp, vp, vp]
    L.tfp8_compress_ex.restype = i32
    L.tfp8_decompress_ex.argtypes = [vp, vp, vp, i64, i32, u32, vp, i32, vp]
    L.tfp8_decompress_ex.restype = i32
    L.tfp8_reduce_ex.argtypes = [vp, vp, vp, i32, i64, i32, f32, u32, vp, vp, vp, vp]
    L.tfp8_reduce_ex.restype = i32
    L.tfp8_reduce_strided.argtypes = [vp, i64, vp, i64, vp, i64, i32, i64, i32, f32, u32,
                                      vp, vp, vp, vp]
    L.tfp8_reduce_strided.restype = i32
    L.tfp8_accumulate.argtypes = [vp, vp, vp, vp, i32, i64, i32, f32, u32, vp, vp, vp, vp]
    L.tfp8_accumulate.restype = i32
    L.tfp8_status_string.argtypes = [i32]
    L.tfp8_status_string.restype = ctypes.c_char_p
    L.tfp8_version.argtypes = []
    L.tfp8_version.restype = i32
    return L


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run fp8_compression_tensor_amd/build.py "
                               "(or __graft_entry__.build())")
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def status_string(status: int) -> str:
    return lib().tfp8_status_string(int(status)).decode()


def _check(status: int):
    if status != 0:
        raise TFP8Error(status, status_string(status))


# ---------------------------------------------------------------------------------- raw calls
# Pointers are integers (device addresses); `stream` is a raw hipStream_t (0 = default stream).

def compress_raw(x_ptr: int, x_dtype: int, n: int, block: int, target: float, codes_ptr: int,
                 alpha_ptr: int, scale_ptr: int, stream: int = 0, flags: int = 0) -> int:
    if flags:
        return lib().tfp8_compress_ex(x_ptr, x_dtype, n, block, target, flags, codes_ptr,
                                      alpha_ptr, scale_ptr, stream)
    return lib().tfp8_compress(x_ptr, x_dtype, n, block, target, codes_ptr, alpha_ptr,
                               scale_ptr, stream)


def decompress_raw(codes_ptr: int, alpha_ptr: int, scale_ptr: int, n: int, block: int,
                   out_ptr: int, out_dtype: int, stream: int = 0, flags: int = 0) -> int:
    if flags:
        return lib().tfp8_decompress_ex(codes_ptr, alpha_ptr, scale_ptr, n, block, flags, out_ptr,
                                        out_dtype, stream)
    return lib().tfp8_decompress(codes_ptr, alpha_ptr, scale_ptr, n, block, out_ptr, out_dtype,
                                 stream)


def reduce_fp8_raw(codes_ptr: int, alpha_ptr: int, scale_ptr: int, P: int, n: int, block: int,
                   target: float, codes_out_ptr: int, alpha_out_ptr: int, scale_out_ptr: int,
                   stream: int = 0, flags: int = 0) -> int:
    if flags:
        return lib().tfp8_reduce_ex(codes_ptr, alpha_ptr, scale_ptr, P, n, block, target, flags,
                                    codes_out_ptr, alpha_out_ptr, scale_out_ptr, stream)
    return lib().tfp8_reduce_fp8(codes_ptr, alpha_ptr, scale_ptr, P, n, block, target,
                                 codes_out_ptr, alpha_out_ptr, scale_out_ptr, stream)


def reduce_strided_raw(codes_ptr: int, codes_stride: int, alpha_ptr: int, alpha_stride: int,
                       scale_ptr: int, scale_stride: int, P: int, n: int, block: int,
                       target: float, codes_out_ptr: int, alpha_out_ptr: int, scale_out_ptr: int,
                       stream: int = 0, flags: int = 0) -> int:
    """Contribution p at codes_ptr + p * codes_stride (bytes), alpha_ptr / scale_ptr + p times
    their stride (float32 elements)."""
    return lib().tfp8_reduce_strided(codes_ptr, codes_stride, alpha_ptr, alpha_stride, scale_ptr,
                                     scale_stride, P, n, block, target, flags, codes_out_ptr,
                                     alpha_out_ptr, scale_out_ptr, stream)


def accumulate_raw(codes_ptr: int, alpha_ptr: int, scale_ptr: int, grad_ptr: int, grad_dtype: int,
                   n: int, block: int, target: float, codes_out_ptr: int, alpha_out_ptr: int,
                   scale_out_ptr: int, stream: int = 0, flags: int = 0) -> int:
    return lib().tfp8_accumulate(codes_ptr, alpha_ptr, scale_ptr, grad_ptr, grad_dtype, n, block,
                                 target, flags, codes_out_ptr, alpha_out_ptr, scale_out_ptr, stream)


# ---------------------------------------------------------------------------- tensor wrappers

def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need_gpu(*ts):
    """Every tensor on the same GPU and contiguous (the library reads flat buffers)."""
    dev = None
    for t in ts:
        if not (isinstance(t, torch.Tensor) and t.is_cuda):
            raise ValueError("tfp8 operates on GPU tensors only (no CPU path)")
        if not t.is_contiguous():
            raise ValueError("tfp8 needs contiguous tensors")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on different devices ({dev} and {t.device})")


def _need_buf(t: torch.Tensor, dtype: torch.dtype, numel: int, name: str):
    """A buffer the kernels read or write: its dtype and exact element count, checked here
    because the C ABI takes bare pointers and cannot."""
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")


def _blocks(n: int, block: int) -> int:
    if block not in SUPPORTED_BLOCKS:
        raise ValueError(f"block must be one of {SUPPORTED_BLOCKS}, got {block}")
    if n % block:
        raise ValueError(f"{n} elements are not a multiple of the block size {block}")
    return n // block


def compress(x: torch.Tensor, block: int = 128, target: float = 1.0, out=None, flags: int = 0):
    """x (bfloat16 or float32, any shape, numel % block == 0) ->
    (codes uint8 of x's shape, alpha float32 [numel/block], scale float32 [numel/block])."""
    _need_gpu(x)
    if x.dtype == torch.bfloat16:
        dt = BF16
    elif x.dtype == torch.float32:
        dt = F32
    else:
        raise ValueError(f"unsupported input dtype {x.dtype}")
    n = x.numel()
    nb = _blocks(n, block)
    if out is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
        alpha = torch.empty(nb, dtype=torch.float32, device=x.device)
        scale = torch.empty(nb, dtype=torch.float32, device=x.device)
    else:
        codes, alpha, scale = out
        _need_gpu(x, codes, alpha, scale)
    _need_buf(codes, torch.uint8, n, "codes")
    _need_buf(alpha, torch.float32, nb, "alpha")
    _need_buf(scale, torch.float32, nb, "scale")
    with torch.cuda.device(x.device):
        _check(compress_raw(x.data_ptr(), dt, n, block, float(target), codes.data_ptr(),
                            alpha.data_ptr(), scale.data_ptr(), _stream(x), flags))
    return codes, alpha, scale


def decompress(codes: torch.Tensor, alpha: torch.Tensor, scale: torch.Tensor, block: int = 128,
               dtype: torch.dtype = torch.float32, out=None, flags: int = 0):
    """Reconstruct a float32 or bfloat16 tensor of codes' shape."""
    _need_gpu(codes, alpha, scale)
    if dtype == torch.float32:
        dt = F32
    elif dtype == torch.bfloat16:
        dt = BF16
    else:
        raise ValueError(f"unsupported output dtype {dtype}")
    n = codes.numel()
    nb = _blocks(n, block)
    _need_buf(codes, torch.uint8, n, "codes")
    _need_buf(alpha, torch.float32, nb, "alpha")
    _need_buf(scale, torch.float32, nb, "scale")
    if out is None:
        out = torch.empty(codes.shape, dtype=dtype, device=codes.device)
    else:
        _need_gpu(codes, out)
        _need_buf(out, dtype, n, "out")
    with torch.cuda.device(codes.device):
        _check(decompress_raw(codes.data_ptr(), alpha.data_ptr(), scale.data_ptr(), n, block,
                              out.data_ptr(), dt, _stream(codes), flags))
    return out


def _rows(t: torch.Tensor, dtype: torch.dtype, P: int, m: int, name: str) -> int:
    """A [P, m] view whose rows are contiguous, at any row stride (for example rows of one receive
    buffer); returns the row stride in elements."""
    if not (isinstance(t, torch.Tensor) and t.is_cuda):
        raise ValueError("tfp8 operates on GPU tensors only (no CPU path)")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2 or tuple(t.shape) != (P, m):
        raise ValueError(f"{name} must be [{P}, {m}], got {list(t.shape)}")
    if m > 1 and t.stride(1) != 1:
        raise ValueError(f"the rows of {name} must be contiguous")
    return t.stride(0) if P > 1 else m


def reduce_fp8(codes: torch.Tensor, alpha: torch.Tensor, scale: torch.Tensor, block: int = 128,
               target: float = 1.0, out=None, flags: int = 0):
    """codes [P, ...], alpha and scale [P, nb] -> (codes [...], alpha [nb], scale [nb]).

    Contiguous stacks go to tfp8_reduce_fp8.  Otherwise codes must be a [P, n] view and alpha,
    scale [P, nb] views whose rows are contiguous but may lie at any stride, for example rows of
    one buffer holding a [codes | alpha | scale] message per peer; those go to
    tfp8_reduce_strided and give the same result."""
    if codes.dim() < 2:
        raise ValueError("codes must be stacked as [P, ...]")
    P = codes.shape[0]
    n = codes[0].numel()
    nb = _blocks(n, block)
    strided = not (codes.is_contiguous() and alpha.is_contiguous() and scale.is_contiguous())
    if strided:
        cst = _rows(codes, torch.uint8, P, n, "codes")
        ast = _rows(alpha, torch.float32, P, nb, "alpha")
        sst = _rows(scale, torch.float32, P, nb, "scale")
        if not (codes.device == alpha.device == scale.device):
            raise ValueError("tensors on different devices")
    else:
        _need_gpu(codes, alpha, scale)
        _need_buf(codes, torch.uint8, P * n, "codes")
        _need_buf(alpha, torch.float32, P * nb, "alpha")
        _need_buf(scale, torch.float32, P * nb, "scale")
    if out is None:
        codes_out = torch.empty(codes.shape[1:], dtype=torch.uint8, device=codes.device)
        alpha_out = torch.empty(nb, dtype=torch.float32, device=codes.device)
        scale_out = torch.empty(nb, dtype=torch.float32, device=codes.device)
    else:
        codes_out, alpha_out, scale_out = out
        _need_gpu(codes_out, alpha_out, scale_out)
        if codes_out.device != codes.device:
            raise ValueError(
                f"tensors on different devices ({codes.device} and {codes_out.device})")
        _need_buf(codes_out, torch.uint8, n, "codes_out")
        _need_buf(alpha_out, torch.float32, nb, "alpha_out")
        _need_buf(scale_out, torch.float32, nb, "scale_out")
    with torch.cuda.device(codes.device):
        if strided:
            st = reduce_strided_raw(codes.data_ptr(), cst, alpha.data_ptr(), ast,
                                    scale.data_ptr(), sst, P, n, block, float(target),
                                    codes_out.data_ptr(), alpha_out.data_ptr(),
                                    scale_out.data_ptr(), _stream(codes), flags)
        else:
            st = reduce_fp8_raw(codes.data_ptr(), alpha.data_ptr(), scale.data_ptr(), P, n, block,
                                float(target), codes_out.data_ptr(), alpha_out.data_ptr(),
                                scale_out.data_ptr(), _stream(codes), flags)
        _check(st)
    return codes_out, alpha_out, scale_out


def accumulate(codes: torch.Tensor, alpha: torch.Tensor, scale: torch.Tensor, grad: torch.Tensor,
               block: int = 128, target: float = 1.0, out=None, flags: int = 0,
               inplace: bool = False):
    """Compressed main gradient + dense local gradient (bfloat16 or float32, same numel) ->
    compressed sum.  inplace=True overwrites (codes, alpha, scale) and returns them."""
    _need_gpu(codes, alpha, scale, grad)
    if grad.dtype == torch.bfloat16:
        dt = BF16
    elif grad.dtype == torch.float32:
        dt = F32
    else:
        raise ValueError(f"unsupported gradient dtype {grad.dtype}")
    n = codes.numel()
    if grad.numel() != n:
        raise ValueError("grad and codes must have the same number of elements")
    nb = _blocks(n, block)
    _need_buf(codes, torch.uint8, n, "codes")
    _need_buf(alpha, torch.float32, nb, "alpha")
    _need_buf(scale, torch.float32, nb, "scale")
    if inplace:
        if out is not None:
            raise ValueError("give either out or inplace=True, not both")
        out = (codes, alpha, scale)
    elif out is None:
        out = (torch.empty_like(codes), torch.empty_like(alpha), torch.empty_like(scale))
    else:
        _need_gpu(codes, *out)
        names = ("codes_out", "alpha_out", "scale_out")
        for t, ref, name in zip(out, (codes, alpha, scale), names):
            _need_buf(t, ref.dtype, ref.numel(), name)
    with torch.cuda.device(codes.device):
        _check(accumulate_raw(codes.data_ptr(), alpha.data_ptr(), scale.data_ptr(),
                              grad.data_ptr(), dt, n, block, float(target), out[0].data_ptr(),
                              out[1].data_ptr(), out[2].data_ptr(), _stream(codes), flags))
    return out
