"""C-ABI checks that need no GPU: the library loads, exports every entry point
that include/bqmm.h declares, and rejects bad arguments before any HIP call.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bqmm.h")
PKG = os.path.join(ROOT, "block_quantized_matmul_02_amd")


@pytest.fixture(scope="module")
def L():
    import block_quantized_matmul_02_amd as bqm

    if not os.path.exists(bqm.LIB_PATH):
        from block_quantized_matmul_02_amd import build

        build.build()
    return bqm.lib()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bqm_\w+)\s*\(", text)))


def test_header_declares_the_calls_and_strerror():
    assert declared_symbols() == sorted([
        "bqm_q8_1_quantize", "bqm_q8_0_gemv", "bqm_q8_0_gemm", "bqm_e4m3_quantize_amax", "bqm_e4m3_gemm",
        "bqm_e4m3_gemv", "bqm_q8_0_dequant_f16", "bqm_f16_cvt", "bqm_f16_gemm", "bqm_q8_0_gemm_f8acc",
        "bqm_e4m3_nan_count", "bqm_e4m3_blk_quantize", "bqm_e4m3_blk_gemm", "bqm_q8_0_gemv_f32",
        "bqm_e4m3_gemm_exact", "bqm_strerror"])


def test_library_exports_every_declared_symbol(L):
    for name in declared_symbols():
        assert hasattr(L, name), name


def test_strerror(L):
    import block_quantized_matmul_02_amd as bqm

    assert bqm.strerror(0) == "ok"
    assert "invalid" in bqm.strerror(1)
    assert "unsupported" in bqm.strerror(2)
    assert "HIP" in bqm.strerror(10001)


P = ctypes.c_void_p
A16 = P(0x100000)        # 16-byte aligned stand-ins; never dereferenced (validation fails first)
B16 = P(0x200000)
C16 = P(0x300000)
D16 = P(0x400000)
MIS2 = P(0x100002)       # 2-byte aligned only
NUL = P(0)


def test_q8_1_quantize_validation(L):
    f = L.bqm_q8_1_quantize
    assert f(NUL, B16, C16, 1, 32, NUL) == 1
    assert f(A16, NUL, C16, 1, 32, NUL) == 1
    assert f(A16, B16, NUL, 1, 32, NUL) == 1
    assert f(A16, B16, C16, 0, 32, NUL) == 1
    assert f(A16, B16, C16, 1, 16, NUL) == 1
    assert f(A16, B16, C16, 1, 48, NUL) == 2          # k % 32
    assert f(MIS2, B16, C16, 1, 32, NUL) == 2         # x alignment
    assert f(A16, MIS2, C16, 1, 32, NUL) == 2
    assert f(A16, B16, MIS2, 1, 32, NUL) == 2


@pytest.mark.parametrize("fn", ["bqm_q8_0_gemv", "bqm_q8_0_gemm", "bqm_q8_0_gemm_f8acc"])
def test_q8_0_validation(L, fn):
    f = getattr(L, fn)
    rb = 4096 // 32 * 34
    assert f(NUL, rb, B16, C16, D16, 1, 4096, 8, NUL) == 1
    assert f(A16, rb, NUL, C16, D16, 1, 4096, 8, NUL) == 1
    assert f(A16, rb, B16, NUL, D16, 1, 4096, 8, NUL) == 1
    assert f(A16, rb, B16, C16, NUL, 1, 4096, 8, NUL) == 1
    assert f(A16, rb, B16, C16, D16, 0, 4096, 8, NUL) == 1
    assert f(A16, rb, B16, C16, D16, 1, 4096, 0, NUL) == 1
    assert f(A16, rb, B16, C16, D16, 1, 4096 + 32, 8, NUL) == 2     # k % 256
    assert f(A16, rb - 16, B16, C16, D16, 1, 4096, 8, NUL) == 2     # row shorter than k/32*34
    assert f(A16, rb + 8, B16, C16, D16, 1, 4096, 8, NUL) == 2      # row bytes % 16
    assert f(MIS2, rb, B16, C16, D16, 1, 4096, 8, NUL) == 2
    assert f(A16, rb, MIS2, C16, D16, 1, 4096, 8, NUL) == 2
    assert f(A16, rb, B16, P(0x300004), D16, 1, 4096, 8, NUL) == 2  # xds 8-byte alignment
    assert f(A16, rb, B16, C16, P(0x400002), 1, 4096, 8, NUL) == 2


def test_gemv_f32_validation(L):
    f = L.bqm_q8_0_gemv_f32
    rb = 4096 // 32 * 34
    assert f(NUL, rb, B16, D16, 1, 4096, 8, NUL) == 1
    assert f(A16, rb, NUL, D16, 1, 4096, 8, NUL) == 1
    assert f(A16, rb, B16, NUL, 1, 4096, 8, NUL) == 1
    assert f(A16, rb, B16, D16, 0, 4096, 8, NUL) == 1
    assert f(A16, rb, B16, D16, 16, 4096, 8, NUL) == 1             # m > 15
    assert f(A16, rb, B16, D16, 1, 4096, 0, NUL) == 1
    assert f(A16, rb, B16, D16, 1, 4096 + 32, 8, NUL) == 2         # k % 256
    assert f(A16, rb - 16, B16, D16, 1, 4096, 8, NUL) == 2
    assert f(A16, rb, P(0x100004), D16, 1, 4096, 8, NUL) == 2      # x 16-byte alignment
    assert f(A16, rb, B16, P(0x400002), 1, 4096, 8, NUL) == 2
    rb2 = 16384 // 32 * 34
    assert f(A16, rb2, B16, D16, 9, 16384, 8, NUL) == 2            # on-chip limit
    assert f(A16, rb, B16, D16, 3, 4096, 8, NUL) == 2              # decode only: m <= 2
    assert f(A16, rb2, B16, D16, 1, 16384, 8, NUL) == 2            # m*k <= 8192


def test_gemv_m_range_and_on_chip_limit(L):
    f = L.bqm_q8_0_gemv
    assert f(A16, 4352, B16, C16, D16, 16, 4096, 8, NUL) == 1          # m > 15
    rb = 16384 // 32 * 34
    assert f(A16, rb, B16, C16, D16, 9, 16384, 8, NUL) == 2            # m*k*9/8 > 96 KiB


def test_e4m3_validation(L):
    q = L.bqm_e4m3_quantize_amax
    F = ctypes.c_float
    assert q(NUL, B16, C16, F(1.0), 1, 16, NUL) == 1
    assert q(A16, NUL, C16, F(1.0), 1, 16, NUL) == 1
    assert q(A16, B16, NUL, F(1.0), 1, 16, NUL) == 1
    assert q(A16, B16, C16, F(1.0), 0, 16, NUL) == 1
    assert q(A16, B16, C16, F(float("nan")), 1, 16, NUL) == 1
    assert q(A16, B16, C16, F(float("inf")), 1, 16, NUL) == 1
    assert q(A16, B16, C16, F(1.0), 1, 18, NUL) == 2                   # k % 4
    assert q(MIS2, B16, C16, F(1.0), 1, 16, NUL) == 2
    g = L.bqm_e4m3_gemm
    assert g(NUL, B16, C16, D16, 1, 128, 8, NUL) == 1
    assert g(A16, B16, C16, D16, 1, 128, 0, NUL) == 1
    assert g(A16, B16, C16, D16, 1, 192, 8, NUL) == 2                  # k % 128
    assert g(A16, MIS2, C16, D16, 1, 128, 8, NUL) == 2
    x = L.bqm_e4m3_gemm_exact
    assert x(NUL, B16, C16, D16, 1, 128, 8, NUL) == 1
    assert x(A16, B16, NUL, D16, 1, 128, 8, NUL) == 1
    assert x(A16, B16, C16, D16, 0, 128, 8, NUL) == 1
    assert x(A16, B16, C16, D16, 1, 64, 8, NUL) == 1                   # k < 128
    assert x(A16, B16, C16, D16, 1, 128, 0, NUL) == 1
    assert x(A16, B16, C16, D16, 1, 192, 8, NUL) == 2                  # k % 128
    assert x(A16, B16, C16, D16, 1, 16384 + 128, 8, NUL) == 2          # k beyond the bound's range
    assert x(A16, MIS2, C16, D16, 1, 128, 8, NUL) == 2
    assert x(A16, B16, C16, MIS2, 1, 128, 8, NUL) == 2                 # y 4-byte alignment


def test_e4m3_gemv_validation(L):
    f = L.bqm_e4m3_gemv
    F = ctypes.c_float
    assert f(NUL, B16, F(1.0), D16, 1, 4096, 8, NUL) == 1
    assert f(A16, NUL, F(1.0), D16, 1, 4096, 8, NUL) == 1
    assert f(A16, B16, F(1.0), NUL, 1, 4096, 8, NUL) == 1
    assert f(A16, B16, F(1.0), D16, 0, 4096, 8, NUL) == 1
    assert f(A16, B16, F(1.0), D16, 17, 4096, 8, NUL) == 1             # m > 16
    assert f(A16, B16, F(1.0), D16, 1, 128, 8, NUL) == 1               # k < 256
    assert f(A16, B16, F(1.0), D16, 1, 4096, 0, NUL) == 1
    assert f(A16, B16, F(float("nan")), D16, 1, 4096, 8, NUL) == 1
    assert f(A16, B16, F(float("-inf")), D16, 1, 4096, 8, NUL) == 1
    assert f(A16, B16, F(1.0), D16, 1, 4096 + 128, 8, NUL) == 2        # k % 256
    assert f(A16, B16, F(1.0), D16, 1, 8192 + 256, 8, NUL) == 2        # k > 8192
    assert f(MIS2, B16, F(1.0), D16, 1, 4096, 8, NUL) == 2
    assert f(A16, P(0x200004), F(1.0), D16, 1, 4096, 8, NUL) == 2      # x 16-byte alignment
    assert f(A16, B16, F(1.0), P(0x400002), 1, 4096, 8, NUL) == 2


def test_f16_mirror_validation(L):
    d = L.bqm_q8_0_dequant_f16
    rb = 4096 // 32 * 34
    assert d(NUL, rb, B16, 4096, 8, NUL) == 1
    assert d(A16, rb, NUL, 4096, 8, NUL) == 1
    assert d(A16, rb, B16, 32, 8, NUL) == 1                 # k < 64
    assert d(A16, rb, B16, 4096, 0, NUL) == 1
    assert d(A16, rb, B16, 4096 + 32, 8, NUL) == 2          # k % 64
    assert d(A16, rb - 4, B16, 4096, 8, NUL) == 2           # row shorter than k/32*34
    assert d(A16, rb + 2, B16, 4096, 8, NUL) == 2           # row bytes % 4
    assert d(MIS2, rb, B16, 4096, 8, NUL) == 2
    assert d(A16, rb, P(0x200008), 4096, 8, NUL) == 2       # w16 16-byte alignment
    c = L.bqm_f16_cvt
    assert c(NUL, B16, 8, NUL) == 1
    assert c(A16, NUL, 8, NUL) == 1
    assert c(A16, B16, 0, NUL) == 1
    assert c(P(0x100004), B16, 8, NUL) == 2
    assert c(A16, P(0x200004), 8, NUL) == 2
    g = L.bqm_f16_gemm
    assert g(NUL, B16, C16, 1, 64, 8, NUL) == 1
    assert g(A16, B16, C16, 0, 64, 8, NUL) == 1
    assert g(A16, B16, C16, 1, 32, 8, NUL) == 1
    assert g(A16, B16, C16, 1, 96, 8, NUL) == 2             # k % 64
    assert g(A16, MIS2, C16, 1, 64, 8, NUL) == 2
    assert g(A16, B16, P(0x300002), 1, 64, 8, NUL) == 2


def test_e4m3_blk_validation(L):
    c = L.bqm_e4m3_nan_count
    assert c(NUL, 16, B16, NUL) == 1
    assert c(A16, 16, NUL, NUL) == 1
    assert c(A16, 0, B16, NUL) == 1
    assert c(MIS2, 16, B16, NUL) == 2
    assert c(A16, 16, P(0x200004), NUL) == 2                # 8-byte counter alignment
    q = L.bqm_e4m3_blk_quantize
    assert q(NUL, B16, C16, 1, 128, NUL) == 1
    assert q(A16, B16, C16, 0, 128, NUL) == 1
    assert q(A16, B16, C16, 1, 0, NUL) == 1                  # k < 16
    assert q(A16, B16, C16, 1, 8, NUL) == 1
    assert q(A16, B16, C16, 1, 200, NUL) == 2                # k % 16
    assert q(P(0x100004), B16, C16, 1, 128, NUL) == 2        # x 16-byte alignment
    assert q(A16, MIS2, C16, 1, 128, NUL) == 2
    g = L.bqm_e4m3_blk_gemm
    assert g(NUL, B16, C16, D16, A16, 1, 128, 8, NUL) == 1
    assert g(A16, NUL, C16, D16, A16, 1, 128, 8, NUL) == 1
    assert g(A16, B16, C16, D16, NUL, 1, 128, 8, NUL) == 1
    assert g(A16, B16, C16, D16, A16, 1, 128, 0, NUL) == 1
    assert g(A16, B16, C16, D16, A16, 1, 8, 8, NUL) == 1      # k < 16
    assert g(A16, B16, C16, D16, A16, 1, 256 + 8, 8, NUL) == 2        # k % 16
    assert g(MIS2, B16, C16, D16, A16, 1, 128, 8, NUL) == 2
    assert g(A16, B16, P(0x300004), D16, A16, 1, 128, 8, NUL) == 2   # xq 16-byte alignment


def test_product_path_never_touches_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for fname in files:
            if fname.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, fname)).read()
                assert not re.search(r"\boracle\b", text), f"{fname} mentions the oracle"


def test_missing_library_raises(monkeypatch):
    # No CPU fallback: without the built library every call fails loudly, and
    # host tensors are refused rather than computed on the CPU.
    import torch
    import block_quantized_matmul_02_amd as bqm
    monkeypatch.setattr(bqm, "LIB_PATH", os.path.join(PKG, "no_such_libbqmm.so"))
    monkeypatch.setattr(bqm, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        bqm.lib()
    with pytest.raises((RuntimeError, ValueError)):
        bqm.bqm_q8_1_quantize(torch.zeros(1, 32))



# --------------------------------------------------------------------------- size limits
# Each kernel addresses a workgroup's rows with 32-bit buffer offsets and
# launches a grid of bounded dimensions; sizes past those limits are refused
# with BQM_EUNSUPPORTED before anything is launched (the stand-in pointers are
# never dereferenced).

BIG_M = 65536 * 128      # 65,536 token tiles of 128: one more than a grid's y dimension holds


def test_q8_0_size_limits(L):
    k = 256 * 32769                                  # 256 activation rows of k bytes pass 2^31
    rb = k // 32 * 34
    for fn in (L.bqm_q8_0_gemm, L.bqm_q8_0_gemm_f8acc):
        assert fn(A16, rb, B16, C16, D16, 16, k, 8, NUL) == 2
        assert fn(A16, 13421776, B16, C16, D16, 16, 4096, 8, NUL) == 2        # 160 weight rows pass 2^31
        assert fn(A16, 272, B16, C16, D16, 2 ** 31 - 1, 256, 2 ** 31 - 1, NUL) == 2   # 2^31 tiles
    assert L.bqm_q8_0_gemv(A16, 33554432, B16, C16, D16, 1, 4096, 8, NUL) == 2     # 64 rows pass 2^31
    assert L.bqm_q8_0_gemv_f32(A16, 33554432, B16, D16, 1, 4096, 8, NUL) == 2


def test_e4m3_size_limits(L):
    F = ctypes.c_float
    k = 128 * 52430                                  # 320 weight rows of k bytes pass 2^31
    assert L.bqm_e4m3_gemm(A16, B16, C16, D16, 16, k, 8, NUL) == 2
    assert L.bqm_e4m3_gemm(A16, B16, C16, D16, BIG_M, 128, 8, NUL) == 2
    assert L.bqm_e4m3_gemm_exact(A16, B16, C16, D16, BIG_M, 128, 8, NUL) == 2
    assert L.bqm_e4m3_gemv(A16, B16, F(1.0), D16, 1, 4096, 33554432, NUL) == 2    # n*k past 2^37
    kb = 16 * 419431
    assert L.bqm_e4m3_blk_gemm(A16, B16, C16, D16, A16, 16, kb, 8, NUL) == 2
    assert L.bqm_e4m3_blk_gemm(A16, B16, C16, D16, A16, BIG_M, 128, 8, NUL) == 2
    assert L.bqm_e4m3_blk_quantize(A16, B16, C16, 2 ** 31 - 1, 16384, NUL) == 2   # 2^31 workgroups


def test_f16_mirror_size_limits(L):
    assert L.bqm_f16_gemm(A16, B16, C16, 16, 8388608, 8, NUL) == 2                 # 128 rows of 2k bytes
    assert L.bqm_f16_gemm(A16, B16, C16, BIG_M, 64, 8, NUL) == 2
    k = 2 ** 31 - 64
    assert L.bqm_q8_0_dequant_f16(A16, k // 32 * 34, B16, k, 2 ** 31 - 1, NUL) == 2   # 2^31 workgroups
