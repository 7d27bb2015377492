"""CPU oracle for the block-quantized projection matmul (ctypes over ``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package; the product path
(``block_quantized_matmul_02_amd``) never does, and shares no code with it.

Every function takes and returns numpy arrays on the host.  The arithmetic
lives in ``oracle.c``; this file only marshals arguments.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-fopenmp", "-std=c11"]

_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` (plain gcc, OpenMP over output rows)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.oracle_fp16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_fp16_to_f32.restype = ctypes.c_float
        lib.oracle_q8_1_quantize.argtypes = [P, P, P, I, I]
        lib.oracle_q8_0_block_sums.argtypes = [P, I, P, I, I, I, P]
        lib.oracle_q8_0_matmul.argtypes = [P, I, P, P, I, I, I, P, P]
        lib.oracle_q8_0_matmul_sampled.argtypes = [P, I, P, P, I, I, P, P, P, P]
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_decode.restype = ctypes.c_float
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e4m3_encode_array.argtypes = [P, P, I]
        lib.oracle_e4m3_quantize_amax.argtypes = [P, P, P, ctypes.c_float, I, I]
        lib.oracle_e4m3_matmul.argtypes = [P, P, P, I, I, I, P, P]
        lib.oracle_e4m3_matmul_sampled.argtypes = [P, P, P, I, I, P, P, P, P]
        lib.oracle_e4m3_gemv.argtypes = [P, P, ctypes.c_float, I, I, I, P, P]
        lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_f16.restype = ctypes.c_uint16
        lib.oracle_f32_to_f16_array.argtypes = [P, P, I]
        lib.oracle_q8_0_dequant_f16.argtypes = [P, I, P, I, I]
        lib.oracle_f16_gemm.argtypes = [P, P, I, I, I, P, P]
        lib.oracle_e4m3_gemv_sampled.argtypes = [P, P, ctypes.c_float, I, I, P, P, P, P]
        lib.oracle_q8_0_matmul_e4m3.argtypes = [P, I, P, P, I, I, I, P, P]
        lib.oracle_e4m3_nan_count.argtypes = [P, I]
        lib.oracle_e4m3_nan_count.restype = ctypes.c_uint64
        lib.oracle_e4m3_blk_quantize.argtypes = [P, I, I, P, P]
        lib.oracle_e4m3_blk_matmul.argtypes = [P, P, P, P, I, I, I, P, P]
        lib.oracle_e4m3_blk_matmul_sampled.argtypes = [P, P, P, P, I, I, P, P, P, P]
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def fp16_to_f32(bits: int) -> float:
    return float(_load().oracle_fp16_to_f32(int(bits)))


def q8_1_quantize(x: np.ndarray):
    """f32 [m, k] -> (int8 [m, k], f32 [m, k/32, 2] = (d, s))."""
    x = _c(x, np.float32)
    m, k = x.shape
    assert k % 32 == 0
    xq = np.empty((m, k), dtype=np.int8)
    xds = np.empty((m, k // 32, 2), dtype=np.float32)
    _load().oracle_q8_1_quantize(_p(x), _p(xq), _p(xds), m, k)
    return xq, xds


def q8_0_block_sums(w: np.ndarray, xq: np.ndarray, k: int) -> np.ndarray:
    """int32 block sums S [m, n, k/32]."""
    w = _c(w, np.uint8)
    xq = _c(xq, np.int8)
    n, m = w.shape[0], xq.shape[0]
    S = np.empty((m, n, k // 32), dtype=np.int32)
    _load().oracle_q8_0_block_sums(_p(w), w.shape[1], _p(xq), m, k, n, _p(S))
    return S


def q8_0_matmul(w: np.ndarray, xq: np.ndarray, xds: np.ndarray, k: int):
    """(y fp64 [m, n], T = sum|terms| fp64 [m, n])."""
    w = _c(w, np.uint8)
    xq = _c(xq, np.int8)
    xds = _c(xds, np.float32)
    n, m = w.shape[0], xq.shape[0]
    y = np.empty((m, n), dtype=np.float64)
    T = np.empty((m, n), dtype=np.float64)
    _load().oracle_q8_0_matmul(_p(w), w.shape[1], _p(xq), _p(xds), m, k, n, _p(y), _p(T))
    return y, T


def q8_0_matmul_sampled(w, xq, xds, k: int, tok: np.ndarray, row: np.ndarray):
    """y and T for the (tok[i], row[i]) output elements only."""
    w = _c(w, np.uint8)
    xq = _c(xq, np.int8)
    xds = _c(xds, np.float32)
    tok = _c(tok, np.int64)
    row = _c(row, np.int64)
    y = np.empty(len(tok), dtype=np.float64)
    T = np.empty(len(tok), dtype=np.float64)
    _load().oracle_q8_0_matmul_sampled(_p(w), w.shape[1], _p(xq), _p(xds), k, len(tok),
                                       _p(tok), _p(row), _p(y), _p(T))
    return y, T


def e4m3_decode(codes) -> np.ndarray:
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib.oracle_e4m3_decode(c) for c in range(256)], dtype=np.float32)
    return table[codes]


def e4m3_encode(x) -> np.ndarray:
    x = _c(np.atleast_1d(x), np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().oracle_e4m3_encode_array(_p(x), _p(out), x.size)
    return out


def e4m3_quantize_amax(x: np.ndarray, w_scale: float):
    """f32 [m, k] -> (uint8 codes [m, k], f32 scales[4] = amax, mul, folded, x_scale)."""
    x = _c(x, np.float32)
    m, k = x.shape
    xq = np.empty((m, k), dtype=np.uint8)
    scales = np.empty(4, dtype=np.float32)
    _load().oracle_e4m3_quantize_amax(_p(x), _p(xq), _p(scales), ctypes.c_float(w_scale), m, k)
    return xq, scales


def e4m3_matmul(w: np.ndarray, xq: np.ndarray, scales: np.ndarray):
    w = _c(w, np.uint8)
    xq = _c(xq, np.uint8)
    scales = _c(scales, np.float32)
    n, k = w.shape
    m = xq.shape[0]
    y = np.empty((m, n), dtype=np.float64)
    T = np.empty((m, n), dtype=np.float64)
    _load().oracle_e4m3_matmul(_p(w), _p(xq), _p(scales), m, k, n, _p(y), _p(T))
    return y, T


def e4m3_matmul_sampled(w, xq, scales, tok, row):
    w = _c(w, np.uint8)
    xq = _c(xq, np.uint8)
    scales = _c(scales, np.float32)
    tok = _c(tok, np.int64)
    row = _c(row, np.int64)
    y = np.empty(len(tok), dtype=np.float64)
    T = np.empty(len(tok), dtype=np.float64)
    _load().oracle_e4m3_matmul_sampled(_p(w), _p(xq), _p(scales), w.shape[1], len(tok),
                                       _p(tok), _p(row), _p(y), _p(T))
    return y, T


def e4m3_gemv(w: np.ndarray, x: np.ndarray, w_scale: float):
    """Decode GEMV on raw e4m3 weights: y = w_scale * x @ dec(w)^T in fp64,
    x used as f32.  Returns (y [m, n], sum|terms| [m, n])."""
    w = _c(w, np.uint8)
    x = _c(x, np.float32)
    n, k = w.shape
    m = x.shape[0]
    y = np.empty((m, n), dtype=np.float64)
    T = np.empty((m, n), dtype=np.float64)
    _load().oracle_e4m3_gemv(_p(w), _p(x), ctypes.c_float(w_scale), m, k, n, _p(y), _p(T))
    return y, T


def e4m3_gemv_sampled(w, x, w_scale, tok, row):
    w = _c(w, np.uint8)
    x = _c(x, np.float32)
    tok = _c(tok, np.int64)
    row = _c(row, np.int64)
    y = np.empty(len(tok), dtype=np.float64)
    T = np.empty(len(tok), dtype=np.float64)
    _load().oracle_e4m3_gemv_sampled(_p(w), _p(x), ctypes.c_float(w_scale), w.shape[1], len(tok),
                                     _p(tok), _p(row), _p(y), _p(T))
    return y, T


def f32_to_f16(x) -> np.ndarray:
    """IEEE round-to-nearest-even f32 -> fp16 bit patterns (uint16), same shape."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_f32_to_f16_array(_p(x), _p(out), x.size)
    return out


def q8_0_dequant_f16(w: np.ndarray, k: int) -> np.ndarray:
    """Q8_0 rows [n, row_bytes] -> fp16 bit patterns [n, k]: fp16(d * q)."""
    w = _c(w, np.uint8)
    n = w.shape[0]
    out = np.empty((n, k), dtype=np.uint16)
    _load().oracle_q8_0_dequant_f16(_p(w), w.shape[1], _p(out), k, n)
    return out


def f16_gemm(w16: np.ndarray, x16: np.ndarray):
    """fp16 bit patterns w16 [n, k], x16 [m, k] -> (y = x16 @ w16^T in fp64, sum|terms|)."""
    w16 = _c(w16, np.uint16)
    x16 = _c(x16, np.uint16)
    n, k = w16.shape
    m = x16.shape[0]
    y = np.empty((m, n), dtype=np.float64)
    T = np.empty((m, n), dtype=np.float64)
    _load().oracle_f16_gemm(_p(w16), _p(x16), m, k, n, _p(y), _p(T))
    return y, T


def q8_0_matmul_e4m3(w: np.ndarray, xq: np.ndarray, xds: np.ndarray, k: int):
    """The accumulator instrument's f32 arm: the Q8_0 x q8_1 matmul with every
    quant byte read as an e4m3 code.  Returns (y [m, n] fp64, sum|terms| [m, n])."""
    w = _c(w, np.uint8)
    xq = _c(xq, np.int8).view(np.uint8)
    xds = _c(xds, np.float32)
    n = w.shape[0]
    m = xq.shape[0]
    y = np.empty((m, n), dtype=np.float64)
    T = np.empty((m, n), dtype=np.float64)
    _load().oracle_q8_0_matmul_e4m3(_p(w), w.shape[1], _p(xq), _p(xds), m, k, n, _p(y), _p(T))
    return y, T


def e4m3_nan_count(b: np.ndarray) -> int:
    """Number of e4m3 NaN codes (magnitude 0x7F) in a byte array."""
    b = _c(b, np.uint8)
    return int(_load().oracle_e4m3_nan_count(_p(b), b.size))


def e4m3_blk_quantize(x: np.ndarray):
    """Per (token, 128-k block) e4m3 quantization: (xq uint8 [m, k], xs f32 [m, ceil(k/128)])."""
    x = _c(x, np.float32)
    m, k = x.shape
    xq = np.empty((m, k), dtype=np.uint8)
    xs = np.empty((m, (k + 127) // 128), dtype=np.float32)
    _load().oracle_e4m3_blk_quantize(_p(x), m, k, _p(xq), _p(xs))
    return xq, xs


def e4m3_blk_matmul(w: np.ndarray, grid: np.ndarray, xq: np.ndarray, xs: np.ndarray):
    """Block-128 FP8 matmul in fp64: (y [m, n], sum|terms| [m, n])."""
    w = _c(w, np.uint8)
    grid = _c(grid, np.float32)
    xq = _c(xq, np.uint8)
    xs = _c(xs, np.float32)
    n, k = w.shape
    m = xq.shape[0]
    assert grid.shape == ((n + 127) // 128, (k + 127) // 128) and xs.shape == (m, (k + 127) // 128)
    y = np.empty((m, n), dtype=np.float64)
    T = np.empty((m, n), dtype=np.float64)
    _load().oracle_e4m3_blk_matmul(_p(w), _p(grid), _p(xq), _p(xs), m, k, n, _p(y), _p(T))
    return y, T


def e4m3_blk_matmul_sampled(w, grid, xq, xs, tok, row):
    w = _c(w, np.uint8)
    grid = _c(grid, np.float32)
    xq = _c(xq, np.uint8)
    xs = _c(xs, np.float32)
    tok = _c(tok, np.int64)
    row = _c(row, np.int64)
    y = np.empty(len(tok), dtype=np.float64)
    T = np.empty(len(tok), dtype=np.float64)
    _load().oracle_e4m3_blk_matmul_sampled(_p(w), _p(grid), _p(xq), _p(xs), w.shape[1], len(tok), _p(tok), _p(row),
                                           _p(y), _p(T))
    return y, T
