"""Pins for the CPU oracle: it is checked against things other than itself.

Each test ties an oracle function to a library routine (numpy's binary16,
torch's float8_e4m3fn, numpy matmul/einsum in int64 or fp64), to exact
rational arithmetic, to a closed form, or to a fact the memra-engine pages
state (``tests/golden/page_constants.json``).  The cases are chosen so that a
plausible mistake (dropped term, wrong sign or index, transposed operand,
wrong rounding mode, swapped scale slot) fails at least one of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


@pytest.fixture(scope="module")
def page():
    with open(GOLDEN) as f:
        return json.load(f)


# --------------------------------------------------------------------------- fp16


def test_fp16_decode_all_bit_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.fp16_to_f32(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# --------------------------------------------------------------------------- q8_1


def _blocks(x):
    m, k = x.shape
    return x.reshape(m, k // 32, 32)


def test_q8_1_ties_round_half_away_from_zero(page):
    # 127 in lane 0 makes d = 127/127 = 1 exactly, so x/d = x and every
    # k + 0.5 is an exact tie: away from zero gives k+1, not the even neighbour.
    k_vals = np.arange(31, dtype=np.float32)  # 0..30
    blk = np.concatenate([[127.0], k_vals + 0.5]).astype(np.float32)
    x = np.stack([blk, -blk]).astype(np.float32)
    xq, xds = oracle.q8_1_quantize(x)
    assert xds[0, 0, 0] == 1.0 and xds[1, 0, 0] == 1.0
    expect = np.concatenate([[127], k_vals.astype(np.int64) + 1])
    assert np.array_equal(xq[0].astype(np.int64), expect)
    assert np.array_equal(xq[1].astype(np.int64), -expect)
    # on the pages the int8 code of a block's largest magnitude is +-127
    assert page["int8_quantizer_amax_code"]["value"] == 127


def test_q8_1_constant_block_closed_form():
    for v in [1.0, 0.3, 7.25e-3, 123.456]:
        x = np.full((1, 64), v, dtype=np.float32)
        xq, xds = oracle.q8_1_quantize(x)
        assert np.all(xq == 127)
        d = xds[0, :, 0]
        # d is the correctly rounded f32 quotient amax/127: within half an ulp
        exact = Fraction(float(np.float32(v))) / 127
        for di in d:
            ulp = np.spacing(np.float32(di))
            assert abs(Fraction(float(di)) - exact) <= Fraction(float(ulp)) / 2
        assert np.all(xds[0, :, 1] == np.float32(d[0] * np.float32(127 * 32)))


def test_q8_1_zero_block():
    x = np.zeros((2, 64), dtype=np.float32)
    x[1, 32:] = np.linspace(-1, 1, 32)
    xq, xds = oracle.q8_1_quantize(x)
    assert np.all(xq[0] == 0) and np.all(xq[1, :32] == 0)
    assert np.all(xds[0] == 0) and np.all(xds[1, 0] == 0)
    assert xds[1, 1, 0] > 0


def test_q8_1_block_whose_scale_underflows_is_zero():
    # amax = 2^-149 (the smallest subnormal): amax/127 < 2^-150 rounds to 0 in
    # f32, so the block is treated like an all-zero block.
    x = np.zeros((1, 64), dtype=np.float32)
    x[0, 5] = np.float32(2.0 ** -149)
    x[0, 6] = -np.float32(0.0)
    x[0, 32] = np.float32(127 * 2.0 ** -149)     # d = 2^-149 exactly: the smallest non-zero scale
    xq, xds = oracle.q8_1_quantize(x)
    assert np.float32(x[0, 5]) / np.float32(127) == 0
    assert np.all(xq[0, :32] == 0) and np.all(xds[0, 0] == 0)
    assert xds[0, 1, 0] == np.float32(2.0 ** -149) and xq[0, 32] == 127


def test_q8_1_power_of_two_scaling_and_negation_are_exact():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    xq, xds = oracle.q8_1_quantize(x)
    for j in (-20, -3, 1, 5, 30):
        xq2, xds2 = oracle.q8_1_quantize(np.ldexp(x, j).astype(np.float32))
        assert np.array_equal(xq2, xq)
        assert np.array_equal(xds2, np.ldexp(xds, j).astype(np.float32))
    xq3, xds3 = oracle.q8_1_quantize(-x)
    assert np.array_equal(xq3, -xq)
    assert np.array_equal(xds3[..., 0], xds[..., 0])
    assert np.array_equal(xds3[..., 1], -xds[..., 1])


def test_q8_1_random_blocks_satisfy_the_definition():
    rng = np.random.default_rng(5)
    x = workloads.activations(8, 1024, rng, outliers=True)
    x[0, :32] = 0.0                                   # one all-zero block
    x[1, 32:64] = np.float32(1e-41)                   # subnormal block
    xq, xds = oracle.q8_1_quantize(x)
    xb = _blocks(x)
    qb = _blocks(xq.astype(np.int64))
    d = xds[..., 0]
    amax = np.abs(xb).max(axis=2)
    # d is amax/127 correctly rounded to f32 (checked in exact rationals)
    for a, di in zip(amax.ravel()[:300], d.ravel()[:300]):
        exact = Fraction(float(a)) / 127
        assert abs(Fraction(float(di)) - exact) <= Fraction(float(np.spacing(np.float32(di)))) / 2
    nz = amax > 0
    # q is the nearest integer to the f32 quotient x/d, ties away from zero, |q| <= 127
    ratio = (xb[nz] / d[nz][:, None]).astype(np.float32).astype(np.float64)
    q = qb[nz]
    diff = np.abs(ratio - q)
    assert np.all(diff <= 0.5)
    ties = diff == 0.5
    assert np.all(np.abs(q[ties]) > np.abs(ratio[ties]))
    assert np.all(np.abs(qb) <= 127)
    # the amax element of every non-zero block lands on +-127
    idx = np.abs(xb).argmax(axis=2)
    at_amax = np.take_along_axis(qb, idx[..., None], axis=2)[..., 0]
    assert np.all(np.abs(at_amax[nz]) == 127)
    assert np.all(qb[~nz] == 0) and np.all(d[~nz] == 0)
    # second pair value: d times the quant sum, one f32 rounding
    s = (d * qb.sum(axis=2).astype(np.float32)).astype(np.float32)
    assert np.array_equal(xds[..., 1], s)


def test_q8_1_layout_constants(page):
    assert page["q8_1_activation"]["f32_per_block"] == 2
    x = np.ones((3, 96), dtype=np.float32)
    xq, xds = oracle.q8_1_quantize(x)
    assert xq.shape == (3, 96) and xds.shape == (3, 3, 2)


# --------------------------------------------------------------------------- Q8_0 matmul


def _dequant_w(w, k):
    quants, scales = workloads.unpack_q8_0(w, k)
    return quants.astype(np.float64) * np.repeat(scales.astype(np.float64), 32, axis=1)


def _dequant_x(xq, xds):
    return xq.astype(np.float64) * np.repeat(xds[..., 0].astype(np.float64), 32, axis=1)


def test_q8_0_layout_matches_page_constants(page):
    assert page["q8_0_block_bytes"]["value"] == 34
    assert workloads.row_bytes(4096) == 4352
    assert workloads.row_bytes(4096) / 4096 == page["q8_0_over_e4m3_byte_ratio"]["value"]
    # the oracle reads the scale from bytes 0..1 and quants from 2..33
    q = np.arange(-16, 16, dtype=np.int8).reshape(1, 32)
    s = np.array([[0.5]], dtype=np.float16)
    w = workloads.pack_q8_0(q, s)
    assert w.shape == (1, 34) and w[0, 0] == 0x00 and w[0, 1] == 0x38
    xq = np.zeros((1, 32), dtype=np.int8)
    xq[0, 3] = 1
    xds = np.array([[[1.0, 1.0]]], dtype=np.float32)
    y, T = oracle.q8_0_matmul(w, xq, xds, 32)
    assert y[0, 0] == 0.5 * q[0, 3]


@pytest.mark.parametrize("qw,qx,dw,dx", [(3, -5, 0.25, 2.0), (-127, 127, 2.0 ** -10, 2.0 ** -7),
                                         (77, 13, 0.0068359375, 0.01234)])
def test_q8_0_closed_form_constant_inputs(qw, qx, dw, dx):
    # constant quants and scales: y = K * q_w * q_x * d_w * d_x
    k, n, m = 512, 3, 2
    w = workloads.pack_q8_0(np.full((n, k), qw, np.int8), np.full((n, k // 32), dw, np.float16))
    xq = np.full((m, k), qx, np.int8)
    xds = np.zeros((m, k // 32, 2), np.float32)
    xds[..., 0] = np.float32(dx)
    y, T = oracle.q8_0_matmul(w, xq, xds, k)
    exact = Fraction(k * qw * qx) * Fraction(float(np.float16(dw))) * Fraction(float(np.float32(dx)))
    assert np.all(np.abs(y - float(exact)) <= 1e-15 * abs(float(exact)))
    assert np.allclose(T, abs(float(exact)), rtol=1e-15)


def test_q8_0_block_sums_match_int64_einsum():
    rng = np.random.default_rng(11)
    k, n, m = 256, 37, 5
    w = workloads.q8_0_weights(n, k, rng)
    xq = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    S = oracle.q8_0_block_sums(w, xq, k)
    quants, _ = workloads.unpack_q8_0(w, k)
    ref = np.einsum("tbi,nbi->tnb", xq.reshape(m, k // 32, 32).astype(np.int64),
                    quants.reshape(n, k // 32, 32).astype(np.int64))
    assert np.array_equal(S.astype(np.int64), ref)


def test_q8_0_integer_activations_give_exact_integer_sums():
    # unit scales everywhere: y = sum_b S_b exactly (integers below 2^24)
    rng = np.random.default_rng(12)
    k, n, m = 512, 19, 3
    quants = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    w = workloads.pack_q8_0(quants, np.ones((n, k // 32), np.float16))
    x = rng.integers(-126, 127, size=(m, k)).astype(np.float32)
    x[:, ::32] = 127.0                      # amax 127 in every block -> d_x = 1, q_x = x
    xq, xds = oracle.q8_1_quantize(x)
    assert np.all(xds[..., 0] == 1.0) and np.array_equal(xq.astype(np.float32), x)
    y, _ = oracle.q8_0_matmul(w, xq, xds, k)
    ref = x.astype(np.int64) @ quants.astype(np.int64).T
    assert np.array_equal(y, ref.astype(np.float64))


def test_q8_0_matches_fp64_dequantize_then_matmul():
    rng = np.random.default_rng(13)
    k, n, m = 1280, 67, 9
    w = workloads.q8_0_weights(n, k, rng)
    xq, xds = oracle.q8_1_quantize(workloads.activations(m, k, rng, outliers=True))
    y, T = oracle.q8_0_matmul(w, xq, xds, k)
    ref = _dequant_x(xq, xds) @ _dequant_w(w, k).T
    assert y.shape == (m, n)
    assert np.all(np.abs(y - ref) <= 1e-12 * T)
    # T = sum over blocks of |d_w d_x S_b|
    quants, scales = workloads.unpack_q8_0(w, k)
    S = np.einsum("tbi,nbi->tnb", xq.reshape(m, -1, 32).astype(np.int64),
                  quants.reshape(n, -1, 32).astype(np.int64)).astype(np.float64)
    terms = S * xds[:, None, :, 0].astype(np.float64) * scales[None, :, :].astype(np.float64)
    assert np.allclose(T, np.abs(terms).sum(axis=2), rtol=1e-12, atol=0)


def test_q8_0_padded_rows_and_sampled_outputs():
    rng = np.random.default_rng(14)
    k, n, m = 256, 11, 4
    w = workloads.q8_0_weights(n, k, rng)
    pad = np.full((n, 16), 0xAB, np.uint8)                 # padding bytes must be ignored
    wp = np.concatenate([w, pad], axis=1)
    xq, xds = oracle.q8_1_quantize(workloads.activations(m, k, rng))
    y, T = oracle.q8_0_matmul(w, xq, xds, k)
    yp, Tp = oracle.q8_0_matmul(wp, xq, xds, k)
    assert np.array_equal(y, yp) and np.array_equal(T, Tp)
    tok = np.array([0, 3, 2, 1]); row = np.array([10, 0, 5, 7])
    ys, Ts = oracle.q8_0_matmul_sampled(wp, xq, xds, k, tok, row)
    assert np.array_equal(ys, y[tok, row]) and np.array_equal(Ts, T[tok, row])


def test_q8_0_tiny_brute_force_in_exact_rationals():
    rng = np.random.default_rng(15)
    k, n, m = 64, 3, 2
    w = workloads.q8_0_weights(n, k, rng)
    xq, xds = oracle.q8_1_quantize(workloads.activations(m, k, rng))
    y, T = oracle.q8_0_matmul(w, xq, xds, k)
    quants, scales = workloads.unpack_q8_0(w, k)
    for t in range(m):
        for r in range(n):
            exact = Fraction(0)
            for i in range(k):
                b = i // 32
                exact += (Fraction(float(scales[r, b])) * int(quants[r, i])
                          * Fraction(float(xds[t, b, 0])) * int(xq[t, i]))
            assert abs(Fraction(float(y[t, r])) - exact) <= Fraction(2) ** -50 * Fraction(float(T[t, r]))


# --------------------------------------------------------------------------- e4m3


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def test_e4m3_decode_matches_torch_and_page_facts(page):
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_decode(codes)
    ref = _torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert list(np.nonzero(nan)[0]) == [page["e4m3_nan_magnitude"]["value"], 0x80 | 0x7F]
    lo, hi = page["e4m3_denormal_codes"]["first"], page["e4m3_denormal_codes"]["last"]
    smallest_normal = got[0x08]
    assert np.all((got[lo:hi + 1] > 0) & (got[lo:hi + 1] < smallest_normal))
    assert got[0x7E] == page["e4m3_act_scale_divisor"]["value"]       # 448: max finite
    assert got[0x38] == 1.0


def test_e4m3_encode_round_trip_and_ties_to_even():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)
    pos = np.arange(0x7E, dtype=np.uint8)            # adjacent pairs (c, c+1), c < 0x7E
    lo, hi = oracle.e4m3_decode(pos), oracle.e4m3_decode(pos + 1)
    mid = ((lo.astype(np.float64) + hi) / 2).astype(np.float32)   # exact in f32
    enc = oracle.e4m3_encode(mid)
    even = np.where(pos % 2 == 0, pos, pos + 1)
    assert np.array_equal(enc, even)
    assert np.array_equal(oracle.e4m3_encode(-mid), even | 0x80)
    below = np.nextafter(mid, np.float32(0))
    above = np.nextafter(mid, np.float32(1e9))
    assert np.array_equal(oracle.e4m3_encode(below), pos)
    assert np.array_equal(oracle.e4m3_encode(above), pos + 1)


def test_e4m3_encode_saturates_and_keeps_zero_sign():
    x = np.array([448.0, 449.0, 1e30, np.inf, -500.0, -np.inf, 0.0, -0.0, -1e-30, 2.0 ** -10,
                  np.nextafter(np.float32(2.0 ** -10), np.float32(1))], dtype=np.float32)
    got = oracle.e4m3_encode(x)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x00, 0x80, 0x80, 0x00, 0x01]


def test_e4m3_encode_dense_sweep_matches_torch():
    rng = np.random.default_rng(21)
    mags = np.ldexp(rng.random(200000).astype(np.float32) + 0.5, rng.integers(-14, 10, 200000))
    x = (mags * np.where(rng.random(200000) < 0.5, -1, 1)).astype(np.float32)
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x), ref)


def test_e4m3_quantize_constant_and_zero_batches(page):
    w_scale = 0.0123
    for v in (0.75, -3.5e-3, 1234.0):
        x = np.full((3, 64), v, np.float32)
        xq, sc = oracle.e4m3_quantize_amax(x, w_scale)
        assert np.all(xq == (0x7E if v > 0 else 0xFE))
        a = np.float32(abs(v))
        assert sc[0] == a
        assert sc[1] == np.float32(np.float32(448.0) / a)           # [1] quant mul
        assert sc[3] == np.float32(a / np.float32(page["e4m3_act_scale_divisor"]["value"]))
        assert sc[2] == np.float32(sc[3] * np.float32(w_scale))    # [2] folded scale
    xq, sc = oracle.e4m3_quantize_amax(np.zeros((2, 32), np.float32), w_scale)
    assert np.all(xq == 0) and np.all(sc == 0)


def test_e4m3_quantize_random_batch_properties():
    rng = np.random.default_rng(22)
    x = workloads.activations(16, 512, rng)
    xq, sc = oracle.e4m3_quantize_amax(x, 0.5)
    amax = np.abs(x).max()
    assert sc[0] == amax
    i = np.abs(x).argmax()
    assert xq.ravel()[i] in (0x7E, 0xFE)                      # amax maps onto 448
    dec = oracle.e4m3_decode(xq).astype(np.float64)
    scaled = x.astype(np.float64) * float(sc[1])
    # each code is a nearest e4m3 value to the scaled input (relative spacing 2^-3)
    big = np.abs(scaled) >= 2.0 ** -6
    assert np.all(np.abs(dec[big] - scaled[big]) <= np.abs(scaled[big]) * 2.0 ** -4 * 1.0001)
    assert np.all(np.abs(dec[~big] - scaled[~big]) <= 2.0 ** -10)


def test_e4m3_matmul_one_hot_and_fp64_reference():
    rng = np.random.default_rng(23)
    codes, w_scale = workloads.e4m3_weights(13, 256, rng)
    assert not np.any((codes & 0x7F) == 0x7F)
    x = workloads.activations(5, 256, rng)
    xq, sc = oracle.e4m3_quantize_amax(x, w_scale)
    y, T = oracle.e4m3_matmul(codes, xq, sc)
    ref = _torch_decode(xq).astype(np.float64) @ _torch_decode(codes).astype(np.float64).T
    ref *= float(sc[2])
    assert np.all(np.abs(y - ref) <= 1e-15 * T)
    onehot = np.zeros((2, 256), np.uint8)
    onehot[0, 17] = 0x38                                     # 1.0
    onehot[1, 200] = 0xB8                                    # -1.0
    y1, _ = oracle.e4m3_matmul(codes, onehot, sc)
    assert np.array_equal(y1[0], _torch_decode(codes[:, 17]).astype(np.float64) * float(sc[2]))
    assert np.array_equal(y1[1], -_torch_decode(codes[:, 200]).astype(np.float64) * float(sc[2]))
    tok = np.array([4, 0, 2]); row = np.array([12, 3, 0])
    ys, Ts = oracle.e4m3_matmul_sampled(codes, xq, sc, tok, row)
    assert np.array_equal(ys, y[tok, row]) and np.array_equal(Ts, T[tok, row])


# --------------------------------------------------------------------------- e4m3 decode GEMV


@pytest.mark.parametrize("code,v", [(0x38, 1.0), (0x01, -3.25), (0x7E, 0.0078125), (0xC5, 1.5), (0x80, 7.0)])
def test_e4m3_gemv_closed_form_constant_inputs(code, v):
    # every weight the same code, every activation the same value:
    # y = w_scale * K * v * dec(code), an exact product here
    k, n, ws = 512, 3, 0.375
    w = np.full((n, k), code, np.uint8)
    x = np.full((2, k), v, np.float32)
    y, T = oracle.e4m3_gemv(w, x, ws)
    d = float(_torch_decode([code])[0])
    assert np.all(y == ws * k * v * d)
    assert np.all(T == abs(ws * k * v * d))


def test_e4m3_gemv_one_hot_picks_column_and_row():
    rng = np.random.default_rng(31)
    n, k = 37, 256
    codes, ws = workloads.e4m3_weights(n, k, rng)
    x = np.zeros((3, k), np.float32)
    x[0, 5] = 1.0
    x[1, 200] = -2.0
    x[2, 255] = 0.5
    y, _ = oracle.e4m3_gemv(codes, x, ws)
    dec = _torch_decode(codes).astype(np.float64)
    assert np.array_equal(y[0], dec[:, 5] * ws)
    assert np.array_equal(y[1], -2.0 * dec[:, 200] * ws)
    assert np.array_equal(y[2], 0.5 * dec[:, 255] * ws)


def test_e4m3_gemv_matches_fp64_matmul_of_torch_decoded_weights():
    rng = np.random.default_rng(32)
    n, k, m = 64, 1280, 9
    codes, ws = workloads.e4m3_weights(n, k, rng)
    x = workloads.activations(m, k, rng, outliers=True)
    y, T = oracle.e4m3_gemv(codes, x, ws)
    dec = _torch_decode(codes).astype(np.float64)
    ref = float(ws) * (x.astype(np.float64) @ dec.T)
    tref = abs(float(ws)) * (np.abs(x.astype(np.float64)) @ np.abs(dec).T)
    assert np.all(np.abs(y - ref) <= 1e-12 * tref)
    assert np.allclose(T, tref, rtol=1e-12, atol=0)
    ys, Ts = oracle.e4m3_gemv_sampled(codes, x, ws, np.array([0, 8, 4]), np.array([63, 0, 17]))
    assert np.array_equal(ys, y[[0, 8, 4], [63, 0, 17]])
    assert np.array_equal(Ts, T[[0, 8, 4], [63, 0, 17]])


def test_e4m3_gemv_tiny_brute_force_in_exact_rationals():
    rng = np.random.default_rng(33)
    n, k, m = 3, 7, 2
    codes = rng.integers(0, 256, size=(n, k)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x12          # no NaN codes
    x = rng.standard_normal((m, k)).astype(np.float32)
    ws = np.float32(0.0123)
    y, _ = oracle.e4m3_gemv(codes, x, float(ws))
    dec = _torch_decode(codes)
    for t in range(m):
        for r in range(n):
            exact = Fraction(float(ws)) * sum(Fraction(float(x[t, i])) * Fraction(float(dec[r, i])) for i in range(k))
            assert abs(Fraction(y[t, r]) - exact) <= abs(exact) * Fraction(1, 2**50) + Fraction(1, 2**1000)


# --------------------------------------------------------------------------- fp16 mirror


def _np_f16_bits(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def test_f32_to_f16_matches_numpy_on_every_code_midpoint_and_neighbour():
    # every finite fp16 value, the midpoints between neighbours (ties go to the
    # even code), one f32 ulp either side of each midpoint, the overflow edge
    codes = np.arange(0, 0x7C00, dtype=np.uint16)
    vals = codes.view(np.float16).astype(np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:].astype(np.float64)) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    edge = np.array([65504, 65519.996, 65520, 65536, 1e30, np.inf, 2.0**-25, 2.0**-24, 1e-30], np.float32)
    x = np.concatenate([vals, mids, up, dn, edge])
    x = np.concatenate([x, -x])
    assert np.array_equal(oracle.f32_to_f16(x), _np_f16_bits(x))


def test_f32_to_f16_random_and_nan():
    rng = np.random.default_rng(40)
    x = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-9, 6, 200000)).astype(np.float32)
    assert np.array_equal(oracle.f32_to_f16(x), _np_f16_bits(x))
    h = oracle.f32_to_f16(np.array([np.nan], np.float32))[0]
    assert (h & 0x7C00) == 0x7C00 and (h & 0x3FF) != 0


def test_q8_0_dequant_f16_closed_form_and_numpy():
    # d = 1 (0x3C00): fp16(q) is exactly q
    k = 64
    w = workloads.pack_q8_0(np.tile(np.arange(-32, 32, dtype=np.int8), (2, 1)),
                            np.full((2, 2), 1.0, np.float16))
    assert np.array_equal(oracle.q8_0_dequant_f16(w, k).view(np.float16).astype(np.float32),
                          np.tile(np.arange(-32, 32, dtype=np.float32), (2, 1)))
    rng = np.random.default_rng(41)
    n, k = 7, 512
    w = workloads.q8_0_weights(n, k, rng)
    q, d = workloads.unpack_q8_0(w, k)
    ref = _np_f16_bits(d.astype(np.float32).repeat(32, axis=1) * q.astype(np.float32))
    assert np.array_equal(oracle.q8_0_dequant_f16(w, k), ref)


def test_f16_gemm_matches_fp64_matmul_and_one_hot():
    rng = np.random.default_rng(42)
    n, k, m = 33, 1024, 5
    w16 = oracle.q8_0_dequant_f16(workloads.q8_0_weights(n, k, rng), k)
    x16 = oracle.f32_to_f16(workloads.activations(m, k, rng, outliers=True))
    y, T = oracle.f16_gemm(w16, x16)
    W = w16.view(np.float16).astype(np.float64)
    X = x16.view(np.float16).astype(np.float64)
    assert np.all(np.abs(y - X @ W.T) <= 1e-12 * (np.abs(X) @ np.abs(W).T))
    assert np.allclose(T, np.abs(X) @ np.abs(W).T, rtol=1e-12, atol=0)
    oh = np.zeros((2, k), np.float32)
    oh[0, 3] = 1.0
    oh[1, 1000] = -2.0
    y1, _ = oracle.f16_gemm(w16, oracle.f32_to_f16(oh))
    assert np.array_equal(y1[0], W[:, 3])
    assert np.array_equal(y1[1], -2.0 * W[:, 1000])


# --------------------------------------------------------------------------- accumulator instrument, f32 arm


def _torch_e4m3(b):
    return torch.from_numpy(np.ascontiguousarray(b).view(np.uint8)).view(torch.float8_e4m3fn).double().numpy()


@pytest.mark.parametrize("dist", ["wide", "mid"])
def test_q8_0_matmul_e4m3_matches_torch_decoded_fp64_matmul(dist):
    # bytes decoded by torch's float8_e4m3fn, scales by numpy's float16, one
    # fp64 einsum per block: an independent route to the same definition
    rng = np.random.default_rng(7)
    n, k, m = 29, 512, 6
    w = workloads.accprobe_weights(n, k, rng, dist)
    xq, xds = workloads.accprobe_activations(m, k, rng, dist)
    y, T = oracle.q8_0_matmul_e4m3(w, xq, xds, k)
    q, d = workloads.unpack_q8_0(w, k)
    Wq = _torch_e4m3(q).reshape(n, k // 32, 32)
    Xq = _torch_e4m3(xq).reshape(m, k // 32, 32)
    blk = np.einsum("tbi,nbi->tnb", Xq, Wq)
    scale = xds[:, None, :, 0].astype(np.float64) * d.astype(np.float64)[None, :, :]
    ref = (scale * blk).sum(axis=2)
    babs = np.einsum("tbi,nbi->tnb", np.abs(Xq), np.abs(Wq))
    assert np.all(np.abs(y - ref) <= 1e-13 * T)
    assert np.allclose(T, (np.abs(scale) * babs).sum(axis=2), rtol=1e-13, atol=0)
    # the int8 reading of the same bytes is a different number
    y8, _ = oracle.q8_0_matmul(w, xq, xds, k)
    assert not np.allclose(y, y8)


def test_q8_0_matmul_e4m3_one_hot_and_closed_form():
    k, n = 256, 4
    rng = np.random.default_rng(3)
    w = workloads.accprobe_weights(n, k, rng)
    q, d = workloads.unpack_q8_0(w, k)
    # one activation byte 0x38 (e4m3 1.0) at column 77 with d_x = 1: y = d_w * dec(q_w) exactly
    xq = np.zeros((1, k), np.int8)
    xq[0, 77] = 0x38
    xds = np.zeros((1, k // 32, 2), np.float32)
    xds[0, :, 0] = 1.0
    y, _ = oracle.q8_0_matmul_e4m3(w, xq, xds, k)
    expect = d[:, 77 // 32].astype(np.float64) * _torch_e4m3(q[:, 77])
    assert np.array_equal(y[0], expect)
    # constant bytes and scales: y = K * dec(cw) * dec(cx) * d_w * d_x
    cw, cx = np.int8(0x44), np.int8(-0x3B)              # 0x44 = 3.0, 0xC5 = -3.25 (OCP E4M3FN)
    wc = workloads.pack_q8_0(np.full((2, k), cw, np.int8), np.full((2, k // 32), 0.015625, np.float16))
    xqc = np.full((3, k), cx, np.int8)
    xdsc = np.zeros((3, k // 32, 2), np.float32)
    xdsc[:, :, 0] = 0.5
    yc, Tc = oracle.q8_0_matmul_e4m3(wc, xqc, xdsc, k)
    assert np.all(yc == k * 3.0 * -3.25 * 0.015625 * 0.5)
    assert np.all(Tc == -yc)


@pytest.mark.parametrize("dist", ["wide", "mid"])
def test_accprobe_bytes_are_finite_in_both_readings(dist):
    rng = np.random.default_rng(11)
    w = workloads.accprobe_weights(64, 1024, rng, dist)
    xq, _ = workloads.accprobe_activations(64, 1024, rng, dist)
    q, _ = workloads.unpack_q8_0(w, 1024)
    for b in (q, xq):
        assert np.abs(b.astype(np.int16)).max() <= 126
        assert not np.any((b.view(np.uint8) & 0x7F) == 0x7F)
        assert np.all(np.isfinite(_torch_e4m3(b)))
    if dist == "wide":
        assert len(np.unique(q)) == 252


# --------------------------------------------------------------------------- block-128 FP8


def test_e4m3_nan_count_matches_numpy_and_torch():
    rng = np.random.default_rng(21)
    b = rng.integers(0, 256, size=100003, dtype=np.uint8)
    want = int(np.count_nonzero((b & 0x7F) == 0x7F))
    assert want > 0
    assert oracle.e4m3_nan_count(b) == want
    assert oracle.e4m3_nan_count(b) == int(np.isnan(_torch_e4m3(b)).sum())
    clean = np.where((b & 0x7F) == 0x7F, b & 0x80, b).astype(np.uint8)
    assert oracle.e4m3_nan_count(clean) == 0


@pytest.mark.parametrize("m,k", [(3, 256), (5, 200), (2, 4096)])
def test_e4m3_blk_quantize_matches_torch_cast_per_block(m, k):
    rng = np.random.default_rng(m + k)
    x = workloads.activations(m, k, rng, outliers=True)
    x[0, :min(k, 128)] = 0.0                                  # an all-zero block
    if m > 1:
        x[1, -1] = -0.0
    xq, xs = oracle.e4m3_blk_quantize(x)
    kbn = (k + 127) // 128
    assert xs.shape == (m, kbn)
    for t in range(m):
        for kb in range(kbn):
            blk = x[t, 128 * kb:128 * kb + 128]
            amax = np.float32(np.abs(blk).max())
            if amax == 0:
                assert xs[t, kb] == 0
                assert np.all((xq[t, 128 * kb:128 * kb + 128] & 0x7F) == 0)
                continue
            mul = np.float32(448.0) / amax
            assert xs[t, kb] == amax / np.float32(448.0)
            v = np.clip(blk * mul, np.float32(-448.0), np.float32(448.0)).astype(np.float32)
            ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(xq[t, 128 * kb:128 * kb + 128], ref)


def test_e4m3_blk_quantize_closed_forms():
    x = np.full((1, 256), 3.0, np.float32)
    x[0, 128:] = -0.5
    xq, xs = oracle.e4m3_blk_quantize(x)
    assert np.all(xq[0, :128] == 0x7E) and np.all(xq[0, 128:] == 0xFE)
    assert xs[0, 0] == np.float32(3.0) / np.float32(448.0) and xs[0, 1] == np.float32(0.5) / np.float32(448.0)


def test_e4m3_blk_matmul_matches_fp64_of_torch_decoded_blocks():
    rng = np.random.default_rng(8)
    n, k, m = 300, 640, 7
    w, grid = workloads.e4m3_blk_weights(n, k, rng)
    xq, xs = oracle.e4m3_blk_quantize(workloads.activations(m, k, rng))
    y, T = oracle.e4m3_blk_matmul(w, grid, xq, xs)
    W = _torch_e4m3(w) * np.repeat(np.repeat(grid.astype(np.float64), 128, 0), 128, 1)[:n, :k]
    X = _torch_e4m3(xq) * np.repeat(xs.astype(np.float64), 128, 1)[:, :k]
    assert np.all(np.abs(y - X @ W.T) <= 1e-12 * T)
    assert np.allclose(T, np.abs(X) @ np.abs(W).T, rtol=1e-12, atol=0)
    # the sampled form gives the same numbers
    tok = np.array([0, 6, 3]); row = np.array([299, 0, 128])
    ys, Ts = oracle.e4m3_blk_matmul_sampled(w, grid, xq, xs, tok, row)
    assert np.array_equal(ys, y[tok, row]) and np.array_equal(Ts, T[tok, row])


def test_e4m3_blk_matmul_one_hot_and_closed_form():
    rng = np.random.default_rng(9)
    n, k = 200, 384
    w, grid = workloads.e4m3_blk_weights(n, k, rng)
    xq = np.zeros((2, k), np.uint8)
    xq[0, 5] = 0x38                                        # 1.0 in block 0
    xq[1, 300] = 0xB8                                      # -1.0 in block 2
    xs = np.array([[1.0, 1.0, 1.0], [1.0, 1.0, 0.25]], np.float32)
    y, _ = oracle.e4m3_blk_matmul(w, grid, xq, xs)
    wd = _torch_e4m3(w)
    rb = np.arange(n) // 128
    assert np.array_equal(y[0], grid[rb, 0].astype(np.float64) * wd[:, 5])
    assert np.array_equal(y[1], -0.25 * grid[rb, 2].astype(np.float64) * wd[:, 300])
    wc = np.full((3, 256), 0x44, np.uint8)                 # 3.0
    gc = np.full((1, 2), 0.5, np.float32)
    xc = np.full((2, 256), 0xC5, np.uint8)                 # -3.25
    xsc = np.full((2, 2), 0.125, np.float32)
    yc, Tc = oracle.e4m3_blk_matmul(wc, gc, xc, xsc)
    assert np.all(yc == 256 * 3.0 * -3.25 * 0.5 * 0.125) and np.all(Tc == -yc)
