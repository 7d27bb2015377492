"""Python binding of libbqmm, the gfx950 block-quantized projection matmul.

Argument marshalling only: every step runs in the HIP kernels of
``libbqmm.so`` (built in-tree by ``block_quantized_matmul_02_amd.build``).
The functions carry the C ABI's names (``include/bqmm.h``), take torch
tensors that live on the GPU, enqueue on torch's current stream and never
synchronize.  There is no CPU fallback: a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libbqmm.so")

BQM_OK = 0
BQM_EINVAL = 1
BQM_EUNSUPPORTED = 2
BQM_EHIP_BASE = 10000
GEMV_MAX_M = 15
E4M3_GEMV_MAX_M = 16

_lib = None


class BqmError(RuntimeError):
    def __init__(self, fn: str, rc: int):
        self.rc = rc
        super().__init__(f"{fn} failed: rc={rc} ({strerror(rc)})")


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_quantized_matmul_02_amd.build` or __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        L.bqm_q8_1_quantize.argtypes = [P, P, P, I, I, P]
        L.bqm_q8_0_gemv.argtypes = [P, I64, P, P, P, I, I, I, P]
        L.bqm_q8_0_gemm.argtypes = [P, I64, P, P, P, I, I, I, P]
        L.bqm_q8_0_gemm_f8acc.argtypes = [P, I64, P, P, P, I, I, I, P]
        L.bqm_q8_0_gemv_f32.argtypes = [P, I64, P, P, I, I, I, P]
        L.bqm_e4m3_nan_count.argtypes = [P, I64, P, P]
        L.bqm_e4m3_blk_quantize.argtypes = [P, P, P, I, I, P]
        L.bqm_e4m3_blk_gemm.argtypes = [P, P, P, P, P, I, I, I, P]
        L.bqm_e4m3_quantize_amax.argtypes = [P, P, P, F, I, I, P]
        L.bqm_e4m3_gemm.argtypes = [P, P, P, P, I, I, I, P]
        L.bqm_e4m3_gemm_exact.argtypes = [P, P, P, P, I, I, I, P]
        L.bqm_e4m3_gemv.argtypes = [P, P, F, P, I, I, I, P]
        L.bqm_q8_0_dequant_f16.argtypes = [P, I64, P, I, I, P]
        L.bqm_f16_cvt.argtypes = [P, P, I64, P]
        L.bqm_f16_gemm.argtypes = [P, P, P, I, I, I, P]
        for fn in ("bqm_q8_1_quantize", "bqm_q8_0_gemv", "bqm_q8_0_gemm", "bqm_e4m3_quantize_amax",
                   "bqm_e4m3_gemm", "bqm_e4m3_gemv", "bqm_q8_0_dequant_f16", "bqm_f16_cvt", "bqm_f16_gemm",
                   "bqm_q8_0_gemm_f8acc", "bqm_e4m3_nan_count", "bqm_e4m3_blk_quantize", "bqm_e4m3_blk_gemm",
                   "bqm_q8_0_gemv_f32", "bqm_e4m3_gemm_exact"):
            getattr(L, fn).restype = ctypes.c_int
        L.bqm_strerror.argtypes = [I]
        L.bqm_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def strerror(rc: int) -> str:
    return lib().bqm_strerror(int(rc)).decode()


def _stream(t):
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(t, dtype, name, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _raise(fn, rc):
    if rc != BQM_OK:
        raise BqmError(fn, rc)


def bqm_q8_1_quantize(x, xq=None, xds=None):
    """q8_1 quantization of f32 ``x [m, k]`` -> (int8 ``xq [m, k]``, f32 ``xds [m, k/32, 2]``)."""
    import torch

    m, k = x.shape
    _check(x, torch.float32, "x")
    if xq is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if xds is None:
        xds = torch.empty((m, k // 32, 2), dtype=torch.float32, device=x.device)
    _check(xq, torch.int8, "xq", (m, k))
    _check(xds, torch.float32, "xds", (m, k // 32, 2))
    _raise("bqm_q8_1_quantize", lib().bqm_q8_1_quantize(_ptr(x), _ptr(xq), _ptr(xds), m, k, _stream(x)))
    return xq, xds


def _q8_0_args(w, xq, xds, y, k, n):
    import torch

    m = xq.shape[0]
    _check(w, torch.uint8, "w")
    if w.dim() != 2 or w.shape[0] != n:
        raise ValueError(f"w must be [n={n}, row_bytes], got {tuple(w.shape)}")
    _check(xq, torch.int8, "xq", (m, k))
    _check(xds, torch.float32, "xds", (m, k // 32, 2))
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=xq.device)
    _check(y, torch.float32, "y", (m, n))
    return m, y


def bqm_q8_0_gemv(w, xq, xds, y=None):
    """Q8_0 GEMV, 1 <= m <= 15: ``w [n, row_bytes]`` uint8 Q8_0 rows -> f32 ``y [m, n]``."""
    n = w.shape[0]
    k = xq.shape[1]
    m, y = _q8_0_args(w, xq, xds, y, k, n)
    rc = lib().bqm_q8_0_gemv(_ptr(w), w.shape[1], _ptr(xq), _ptr(xds), _ptr(y), m, k, n, _stream(w))
    _raise("bqm_q8_0_gemv", rc)
    return y


def bqm_q8_0_gemm(w, xq, xds, y=None):
    """Q8_0 MMQ GEMM, any m: ``w [n, row_bytes]`` uint8 Q8_0 rows -> f32 ``y [m, n]``."""
    n = w.shape[0]
    k = xq.shape[1]
    m, y = _q8_0_args(w, xq, xds, y, k, n)
    rc = lib().bqm_q8_0_gemm(_ptr(w), w.shape[1], _ptr(xq), _ptr(xds), _ptr(y), m, k, n, _stream(w))
    _raise("bqm_q8_0_gemm", rc)
    return y


def bqm_q8_0_gemv_f32(w, x, y=None):
    """Decode step in one launch: q8_1 quantization of f32 ``x [m, k]`` and the Q8_0 GEMV against
    ``w [n, row_bytes]`` -> f32 ``y [m, n]``, bitwise equal to bqm_q8_1_quantize + bqm_q8_0_gemv."""
    import torch

    n = w.shape[0]
    m, k = x.shape
    _check(w, torch.uint8, "w")
    _check(x, torch.float32, "x")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _check(y, torch.float32, "y", (m, n))
    _raise("bqm_q8_0_gemv_f32", lib().bqm_q8_0_gemv_f32(_ptr(w), w.shape[1], _ptr(x), _ptr(y), m, k, n, _stream(w)))
    return y


def bqm_q8_0_gemm_f8acc(w, xq, xds, y=None):
    """The accumulator instrument's f32 arm: bqm_q8_0_gemm with the quant bytes read as e4m3
    and multiplied on the fp8 matrix cores (f32 accumulate); same arguments."""
    n = w.shape[0]
    k = xq.shape[1]
    m, y = _q8_0_args(w, xq, xds, y, k, n)
    rc = lib().bqm_q8_0_gemm_f8acc(_ptr(w), w.shape[1], _ptr(xq), _ptr(xds), _ptr(y), m, k, n, _stream(w))
    _raise("bqm_q8_0_gemm_f8acc", rc)
    return y


def bqm_e4m3_quantize_amax(x, w_scale: float, xq=None, scales=None):
    """Per-batch e4m3 quantization of f32 ``x [m, k]`` -> (uint8 codes ``[m, k]``, f32 ``scales[4]``)."""
    import torch

    m, k = x.shape
    _check(x, torch.float32, "x")
    if xq is None:
        xq = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(4, dtype=torch.float32, device=x.device)
    _check(xq, torch.uint8, "xq", (m, k))
    _check(scales, torch.float32, "scales", (4,))
    rc = lib().bqm_e4m3_quantize_amax(_ptr(x), _ptr(xq), _ptr(scales), ctypes.c_float(w_scale), m, k, _stream(x))
    _raise("bqm_e4m3_quantize_amax", rc)
    return xq, scales


def bqm_e4m3_gemm(w, xq, scales, y=None):
    """e4m3 GEMM: codes ``w [n, k]`` and ``xq [m, k]`` -> f32 ``y [m, n]`` scaled by ``scales[2]``."""
    import torch

    n, k = w.shape
    m = xq.shape[0]
    _check(w, torch.uint8, "w")
    _check(xq, torch.uint8, "xq", (m, k))
    _check(scales, torch.float32, "scales", (4,))
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=xq.device)
    _check(y, torch.float32, "y", (m, n))
    rc = lib().bqm_e4m3_gemm(_ptr(w), _ptr(xq), _ptr(scales), _ptr(y), m, k, n, _stream(w))
    _raise("bqm_e4m3_gemm", rc)
    return y


def bqm_e4m3_gemm_exact(w, xq, scales, y=None):
    """e4m3 GEMM with the bound (27 + k/128) * 2^-24 * sum|terms| on every output: same arguments and
    result as :func:`bqm_e4m3_gemm`."""
    import torch

    n, k = w.shape
    m = xq.shape[0]
    _check(w, torch.uint8, "w")
    _check(xq, torch.uint8, "xq", (m, k))
    _check(scales, torch.float32, "scales", (4,))
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=xq.device)
    _check(y, torch.float32, "y", (m, n))
    rc = lib().bqm_e4m3_gemm_exact(_ptr(w), _ptr(xq), _ptr(scales), _ptr(y), m, k, n, _stream(w))
    _raise("bqm_e4m3_gemm_exact", rc)
    return y


def bqm_e4m3_gemv(w, x, w_scale: float, y=None):
    """e4m3 decode GEMV, 1 <= m <= 16: codes ``w [n, k]`` against f32 ``x [m, k]`` -> f32 ``y [m, n]``
    = w_scale * x @ dec(w)^T."""
    import torch

    n, k = w.shape
    m = x.shape[0]
    _check(w, torch.uint8, "w")
    _check(x, torch.float32, "x", (m, k))
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _check(y, torch.float32, "y", (m, n))
    rc = lib().bqm_e4m3_gemv(_ptr(w), _ptr(x), ctypes.c_float(w_scale), _ptr(y), m, k, n, _stream(w))
    _raise("bqm_e4m3_gemv", rc)
    return y


def bqm_q8_0_dequant_f16(w, k: int, w16=None):
    """fp16 mirror of Q8_0 rows ``w [n, row_bytes]`` -> ``w16 [n, k]`` (torch.float16) = fp16(d * q)."""
    import torch

    n = w.shape[0]
    _check(w, torch.uint8, "w")
    if w16 is None:
        w16 = torch.empty((n, k), dtype=torch.float16, device=w.device)
    _check(w16, torch.float16, "w16", (n, k))
    _raise("bqm_q8_0_dequant_f16", lib().bqm_q8_0_dequant_f16(_ptr(w), w.shape[1], _ptr(w16), k, n, _stream(w)))
    return w16


def bqm_f16_cvt(x, x16=None):
    """f32 -> fp16 cast (round to nearest even) of a contiguous tensor, same shape."""
    import torch

    _check(x, torch.float32, "x")
    if x16 is None:
        x16 = torch.empty(x.shape, dtype=torch.float16, device=x.device)
    _check(x16, torch.float16, "x16", tuple(x.shape))
    _raise("bqm_f16_cvt", lib().bqm_f16_cvt(_ptr(x), _ptr(x16), x.numel(), _stream(x)))
    return x16


def bqm_f16_gemm(w16, x16, y=None):
    """fp16 GEMM: ``w16 [n, k]`` and ``x16 [m, k]`` (torch.float16) -> f32 ``y [m, n]`` = x16 @ w16^T."""
    import torch

    n, k = w16.shape
    m = x16.shape[0]
    _check(w16, torch.float16, "w16")
    _check(x16, torch.float16, "x16", (m, k))
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x16.device)
    _check(y, torch.float32, "y", (m, n))
    _raise("bqm_f16_gemm", lib().bqm_f16_gemm(_ptr(w16), _ptr(x16), _ptr(y), m, k, n, _stream(w16)))
    return y


def bqm_e4m3_nan_count(w, out=None):
    """Number of e4m3 NaN codes (magnitude 0x7F) in a uint8 tensor, as a device int64 tensor of one element."""
    import torch

    _check(w, torch.uint8, "w")
    if out is None:
        out = torch.empty(1, dtype=torch.int64, device=w.device)
    _check(out, torch.int64, "out", (1,))
    _raise("bqm_e4m3_nan_count", lib().bqm_e4m3_nan_count(_ptr(w), w.numel(), _ptr(out), _stream(w)))
    return out


def bqm_e4m3_blk_quantize(x, xq=None, xs=None):
    """Per (token, 128-k block) e4m3 quantization of f32 ``x [m, k]`` -> (uint8 ``xq [m, k]``,
    f32 ``xs [m, ceil(k/128)]``); k % 16 == 0, the last block short when k % 128 != 0."""
    import torch

    m, k = x.shape
    _check(x, torch.float32, "x")
    if xq is None:
        xq = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    if xs is None:
        xs = torch.empty((m, (k + 127) // 128), dtype=torch.float32, device=x.device)
    _check(xq, torch.uint8, "xq", (m, k))
    _check(xs, torch.float32, "xs", (m, (k + 127) // 128))
    _raise("bqm_e4m3_blk_quantize", lib().bqm_e4m3_blk_quantize(_ptr(x), _ptr(xq), _ptr(xs), m, k, _stream(x)))
    return xq, xs


def bqm_e4m3_blk_gemm(w, grid, xq, xs, y=None):
    """Block-128 FP8 GEMM: e4m3 ``w [n, k]`` with f32 ``grid [ceil(n/128), ceil(k/128)]``, ``xq``/``xs`` from
    bqm_e4m3_blk_quantize -> f32 ``y [m, n]``."""
    import torch

    n, k = w.shape
    m = xq.shape[0]
    _check(w, torch.uint8, "w")
    _check(grid, torch.float32, "grid", ((n + 127) // 128, (k + 127) // 128))
    _check(xq, torch.uint8, "xq", (m, k))
    _check(xs, torch.float32, "xs", (m, (k + 127) // 128))
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=w.device)
    _check(y, torch.float32, "y", (m, n))
    _raise("bqm_e4m3_blk_gemm", lib().bqm_e4m3_blk_gemm(_ptr(w), _ptr(grid), _ptr(xq), _ptr(xs), _ptr(y), m, k, n,
                                                        _stream(w)))
    return y
