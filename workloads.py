"""Seeded synthetic workloads for the block-quantized projection matmul.

This module only draws random numbers and packs them into the byte layouts
the library reads.  It holds none of the method's arithmetic: no activation
quantization, no block dot products, no scale folding.  Both the CPU oracle
(``oracle/``) and the HIP library are fed from here, so the two sides see
identical bytes.

Layouts (the engine's Q8_0 weight tensor as described on the
``decode_kernel_census.rs`` page (memra-engine 0.113.0), fn ``q8``: a row is
``in_f/32`` blocks of ``32 + 2`` bytes, i.e. an fp16 scale followed by 32 int8
quants; the tensor is ``[out_f][in_f]``):

* ``w``  : ``uint8 [N, K/32*34]`` -- block ``b`` of row ``n`` is
  ``w[n, 34*b : 34*b+34]`` = fp16 little-endian scale, then 32 int8 quants.
* ``x``  : ``float32 [m, K]`` activations, row-major.
* e4m3 weights: ``uint8 [N, K]`` OCP E4M3FN codes plus one f32 per-tensor
  scale (``fp8_ffi.rs`` page (memra-engine 0.70.0), module doc: raw e4m3
  checkpoint bytes with a per-tensor f32 ``weight_scale``).

Draw order per call (fixed; changing it changes every workload):
``q8_0_weights``: quants ``integers(-127, 128, (N, K))`` first, then scales
``10**uniform(-3, -2, (N, K/32))`` rounded to fp16 by numpy.
``activations``: ``standard_normal((m, K))`` then, if ``outliers``,
``random((m, K)) < 0.01`` marks values that are multiplied by 10.
``e4m3_weights``: ``normal(0, 0.02, (N, K))``; the per-tensor scale is
``max|w| / 448`` and the codes are torch's ``float8_e4m3fn`` cast of
``w / scale`` (a library conversion, not this project's encoder).
``e4m3_blk_weights``: ``normal(0, 0.02, (N, K))``; the grid holds each
128x128 block's ``max|w| / 448`` (f32) and the codes are torch's
``float8_e4m3fn`` cast of ``w`` divided by its block's scale, clamped to
+-448 (the block-128 FP8 checkpoint format of the "fp8_ffi.rs" page's
per-block MMQ section: e4m3 codes plus a row-major f32 grid
``[ceil(N/128)][ceil(K/128)]``).
``accprobe_weights`` / ``accprobe_activations`` (the accumulator
instrument's quantizer-free bytes, "accprobe_bench.rs" page (memra-engine
0.124.1), fns ``synth_w_q8_0`` and ``synth_act_q8_1``: quant magnitudes at
most 126, so no byte is a NaN or non-finite value whether read as int8 or as
e4m3):
quants first -- ``wide``: ``integers(-126, 126, (N, K))`` with every value
``v >= -1`` moved up by one, i.e. uniform over -126..126 without -1 (int8 -1
is byte 0xFF, which the page's own magnitude clamp lets through although it is
an e4m3 NaN code); ``mid``: magnitude
``0x30 + integers(0, 32)`` (e4m3 normals, mid exponents) with the sign bit
``integers(0, 2)`` -- then scales, ``uniform(0.01, 0.03)`` rounded to fp16
for weights and ``uniform(0.0125, 0.0273)`` f32 for activations (their sum
slot is 0: the instrument's activation records carry no sum term).
"""
from __future__ import annotations

import numpy as np

QK = 32            # values per quantization block
Q8_0_BLOCK = 34    # bytes per Q8_0 block: fp16 scale + 32 int8 quants


def row_bytes(k: int) -> int:
    """Bytes of one Q8_0 weight row of ``k`` inputs."""
    assert k % QK == 0
    return k // QK * Q8_0_BLOCK


def pack_q8_0(quants: np.ndarray, scales_f16: np.ndarray) -> np.ndarray:
    """Pack int8 quants ``[N, K]`` and fp16 scales ``[N, K/32]`` into 34-byte blocks."""
    n, k = quants.shape
    nb = k // QK
    assert scales_f16.shape == (n, nb) and scales_f16.dtype == np.float16
    out = np.empty((n, nb, Q8_0_BLOCK), dtype=np.uint8)
    out[:, :, 0:2] = scales_f16.astype("<f2").view(np.uint8).reshape(n, nb, 2)
    out[:, :, 2:] = quants.astype(np.int8).view(np.uint8).reshape(n, nb, QK)
    return out.reshape(n, nb * Q8_0_BLOCK)


def unpack_q8_0(w: np.ndarray, k: int):
    """Split packed rows back into (int8 quants [N,K], fp16 scales [N,K/32])."""
    n = w.shape[0]
    nb = k // QK
    blocks = np.ascontiguousarray(w[:, : nb * Q8_0_BLOCK]).reshape(n, nb, Q8_0_BLOCK)
    scales = np.ascontiguousarray(blocks[:, :, 0:2]).view("<f2").reshape(n, nb)
    quants = np.ascontiguousarray(blocks[:, :, 2:]).view(np.int8).reshape(n, k)
    return quants, scales


def q8_0_weights(n: int, k: int, rng: np.random.Generator) -> np.ndarray:
    """Q8_0 weights: quants uniform in [-127, 127], fp16 scales log-uniform in [1e-3, 1e-2]."""
    quants = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    scales = (10.0 ** rng.uniform(-3.0, -2.0, size=(n, k // QK))).astype(np.float16)
    return pack_q8_0(quants, scales)


def activations(m: int, k: int, rng: np.random.Generator, outliers: bool = False) -> np.ndarray:
    """f32 N(0,1) activations; with ``outliers`` 1% of them are scaled by 10."""
    x = rng.standard_normal((m, k), dtype=np.float32)
    if outliers:
        mask = rng.random((m, k)) < 0.01
        x[mask] *= np.float32(10.0)
    return x


def wide_activations(m: int, k: int, rng: np.random.Generator, binades: int = 16) -> np.ndarray:
    """f32 activations whose magnitudes span 2*binades binades: N(0,1) times
    2^e with e uniform on [-binades, binades] per value."""
    x = rng.standard_normal((m, k), dtype=np.float32)
    e = rng.uniform(-binades, binades, size=(m, k))
    return (x * np.exp2(e)).astype(np.float32)


def e4m3_weights(n: int, k: int, rng: np.random.Generator):
    """e4m3 weights drawn from N(0, 0.02) and stored as codes plus one f32 scale."""
    import torch

    w = rng.normal(0.0, 0.02, size=(n, k)).astype(np.float32)
    w_scale = np.float32(np.abs(w).max() / np.float32(448.0))
    v = np.clip(w / w_scale, -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, float(w_scale)


def e4m3_blk_weights(n: int, k: int, rng: np.random.Generator):
    """Block-128 FP8 weights from N(0, 0.02): (codes uint8 [n, k], grid f32 [ceil(n/128), ceil(k/128)])."""
    import torch

    w = rng.normal(0.0, 0.02, size=(n, k)).astype(np.float32)
    nb, kb = (n + 127) // 128, (k + 127) // 128
    pad = np.zeros((nb * 128, kb * 128), np.float32)
    pad[:n, :k] = np.abs(w)
    grid = (pad.reshape(nb, 128, kb, 128).max(axis=(1, 3)) / np.float32(448.0)).astype(np.float32)
    g = np.repeat(np.repeat(grid, 128, axis=0), 128, axis=1)[:n, :k]
    v = np.clip(w / g, -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, grid


def _accprobe_quants(rows: int, k: int, rng: np.random.Generator, dist: str) -> np.ndarray:
    if dist == "wide":
        # -126..126 without -1: int8 -1 is byte 0xFF, an e4m3 NaN code
        v = rng.integers(-126, 126, size=(rows, k), dtype=np.int16)
        return np.where(v >= -1, v + 1, v).astype(np.int8)
    if dist == "mid":
        mag = (0x30 + rng.integers(0, 32, size=(rows, k))).astype(np.uint8)
        sign = (rng.integers(0, 2, size=(rows, k)).astype(np.uint8) << 7).astype(np.uint8)
        return (mag | sign).view(np.int8)
    raise ValueError(f"unknown byte distribution {dist!r}")


def accprobe_weights(n: int, k: int, rng: np.random.Generator, dist: str = "wide") -> np.ndarray:
    """Q8_0 rows whose quant bytes are non-NaN as int8 and as e4m3; fp16 scales in [0.01, 0.03]."""
    quants = _accprobe_quants(n, k, rng, dist)
    scales = rng.uniform(0.01, 0.03, size=(n, k // QK)).astype(np.float16)
    return pack_q8_0(quants, scales)


def accprobe_activations(m: int, k: int, rng: np.random.Generator, dist: str = "wide"):
    """Pre-quantized activations (xq int8 [m, K], xds f32 [m, K/32, 2]) with the same byte rule."""
    xq = _accprobe_quants(m, k, rng, dist)
    xds = np.zeros((m, k // QK, 2), dtype=np.float32)
    xds[:, :, 0] = rng.uniform(0.0125, 0.0273, size=(m, k // QK)).astype(np.float32)
    return xq, xds


# The accumulator instrument's shape sheet (K -> N), "accprobe_bench.rs", fn main.
ACCPROBE_SHAPES_27B = [(5120, 12288), (5120, 1024), (6144, 5120), (5120, 17408), (17408, 5120), (5120, 5120)]
ACCPROBE_SHAPES_1P7B = [(2048, 2048), (2048, 1024), (2048, 2048), (2048, 6144), (6144, 2048)]


# The workloads of the five measured configurations, by what they are.
GEMV_SWEEP_SHAPES = [(4096, 5152), (4096, 4096), (1280, 4096), (4096, 20480)]  # (K, N)
GEMM_NS = [4096, 5152, 20480]


def describe():
    return {
        "gemv_small": dict(m=1, k=4096, n=4096, seed=0),
        "gemv_head": dict(m=1, k=4096, n=64448, seed=0),
        "gemv_sweep": dict(ms=[1, 9], shapes=GEMV_SWEEP_SHAPES, seed=0),
        "mmq_prefill": dict(m=512, k=4096, ns=GEMM_NS, seed=0, outliers=True),
        "e4m3_prefill": dict(m=512, k=4096, n=20480, seed=0),
    }
