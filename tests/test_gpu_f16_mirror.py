"""GPU parity of the fp16 mirror path (Q8_0 -> fp16 dequant, f32 -> fp16
cast, fp16 GEMM) against the CPU oracle.

Bars:
* the two casts are bit-exact against the oracle's IEEE round-to-nearest-even
  conversion (NaN results compared as NaN, since the payload is not part of
  the definition);
* the GEMM is within 1e-5 * sum|terms| per output, exactly 0 where
  sum|terms| is 0.  fp16 x fp16 products are exact in f32, so the only error
  is the f32 accumulation: K/16 matrix-core steps, each adding 16 exact
  products to the accumulator; rounding errors of random sign stay far below
  the bar at these K (the worst case, (K/16 + 4) * 2^-24, reaches 1e-5 only
  for K > 2600, and is never approached by random data);
* end to end against the exact product x . dequant(W) the deviation stays
  inside the pages' 1e-2 relative band for the fp16 mirror.
Outputs are pre-filled with NaN to prove they are fully overwritten.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


@pytest.fixture(scope="module")
def bqm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_matmul_02_amd as m

    m.lib()
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bits(t):
    """fp16 device tensor -> uint16 bit patterns on the host."""
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def nan16(shape):
    return torch.full(shape, float("nan"), dtype=torch.float16, device=DEV)


def assert_f16_equal(got, want, what):
    got_nan = (got & 0x7C00) == 0x7C00
    got_nan &= (got & 0x03FF) != 0
    want_nan = ((want & 0x7C00) == 0x7C00) & ((want & 0x03FF) != 0)
    assert np.array_equal(got_nan, want_nan), f"{what}: NaN positions differ"
    ok = got_nan | (got == want)
    if not ok.all():
        i = np.flatnonzero(~ok)[0]
        raise AssertionError(f"{what}: {np.count_nonzero(~ok)} values differ, first at {i}: "
                             f"0x{got.flat[i]:04x} != 0x{want.flat[i]:04x}")


def check_gemm(y_gpu, y_ref, T, what, tol=1e-5):
    y = y_gpu.astype(np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    zero = T == 0
    assert np.all(y[zero] == 0), f"{what}: nonzero output where all terms are 0"
    ratio = np.abs(y - y_ref)[~zero] / T[~zero]
    assert ratio.size == 0 or ratio.max() <= tol, f"{what}: max err/sum|terms| = {ratio.max():.3e}"


def dequant(bqm, w, k):
    w16 = nan16((w.shape[0], k))
    bqm.bqm_q8_0_dequant_f16(dev(w), k, w16)
    torch.cuda.synchronize()
    return w16


# --------------------------------------------------------------------------- dequant


@pytest.mark.parametrize("n,k", [(1, 64), (33, 4096), (257, 1280), (5, 8192), (1000, 128)])
def test_dequant_bit_exact(bqm, n, k):
    w = workloads.q8_0_weights(n, k, np.random.default_rng(300 + n + k))
    assert_f16_equal(bits(dequant(bqm, w, k)), oracle.q8_0_dequant_f16(w, k), f"dequant n={n} k={k}")


def test_dequant_padded_rows(bqm):
    # row stride larger than k/32*34 (still a multiple of 4); the padding is never read into the mirror
    n, k, pad = 77, 256, 12
    w = workloads.q8_0_weights(n, k, np.random.default_rng(3))
    wp = np.concatenate([w, np.full((n, pad), 0xAB, np.uint8)], axis=1)
    assert_f16_equal(bits(dequant(bqm, wp, k)), oracle.q8_0_dequant_f16(wp, k), "padded rows")


def test_dequant_edge_scales(bqm):
    # every int8 quant against scales that overflow, reach the fp16 subnormals,
    # round at a tie, change sign, are zero, infinite or NaN
    k = 256
    q = np.tile(np.arange(-128, 128, dtype=np.int16).astype(np.int8), (1, 1))
    scales = np.array([65504.0, 1024.0, 6.1035e-05, 5.96e-08, 1e-7, -0.0, 0.0, -3.0, 0.33325, 2049.0 / 2048,
                       np.inf, -np.inf, np.nan, 1.0, -65504.0, 2.0 ** -14], np.float16)
    n = scales.size
    quants = np.tile(q, (n, 1))
    sc = np.repeat(scales[:, None], k // 32, axis=1).astype(np.float16)
    w = workloads.pack_q8_0(quants, sc)
    assert_f16_equal(bits(dequant(bqm, w, k)), oracle.q8_0_dequant_f16(w, k), "edge scales")


# --------------------------------------------------------------------------- cast


@pytest.mark.parametrize("count", [1, 3, 4, 5, 1027, 9 * 4096 + 3, 512 * 4096])
def test_cvt_bit_exact(bqm, count):
    x = workloads.activations(1, count, np.random.default_rng(count), outliers=True)[0]
    x16 = torch.full((count,), float("nan"), dtype=torch.float16, device=DEV)
    bqm.bqm_f16_cvt(dev(x), x16)
    torch.cuda.synchronize()
    assert_f16_equal(bits(x16), oracle.f32_to_f16(x), f"cvt count={count}")


def test_cvt_every_code_tie_and_edge(bqm):
    # every finite fp16 value, the f32 midpoints between neighbours and one f32
    # ulp either side of them, overflow, underflow, signed zeros, inf, NaN
    codes = np.arange(0, 0x7C00, dtype=np.uint16)
    v = np.concatenate([codes, codes | 0x8000]).view(np.float16).astype(np.float32)
    nxt = np.concatenate([codes + 1, (codes + 1) | 0x8000]).view(np.float16).astype(np.float32)
    mid = ((v.astype(np.float64) + nxt.astype(np.float64)) / 2).astype(np.float32)
    below = np.nextafter(mid, np.float32(0))
    above = np.nextafter(mid, np.float32(np.inf) * np.sign(mid))
    extra = np.array([65519.99, 65520.0, 65536.0, 1e30, -1e30, 3e-8, 2.98e-8, 2.9802322e-8, 1e-40, -0.0, 0.0,
                      np.inf, -np.inf, np.nan], np.float32)
    x = np.concatenate([v, mid, below, above, extra]).astype(np.float32)
    pad = (-x.size) % 4
    x = np.concatenate([x, np.zeros(pad + 3, np.float32)])       # and a ragged tail
    x16 = torch.full((x.size,), float("nan"), dtype=torch.float16, device=DEV)
    bqm.bqm_f16_cvt(dev(x), x16)
    torch.cuda.synchronize()
    assert_f16_equal(bits(x16), oracle.f32_to_f16(x), "cvt edges")


# --------------------------------------------------------------------------- GEMM


def gemm_case(bqm, m, k, n, seed):
    rng = np.random.default_rng(seed)
    w = workloads.q8_0_weights(n, k, rng)
    x = workloads.activations(m, k, rng, outliers=True)
    w16_ref = oracle.q8_0_dequant_f16(w, k)
    x16_ref = oracle.f32_to_f16(x)
    w16 = dev(w16_ref.view(np.int16)).view(torch.float16)
    x16 = dev(x16_ref.view(np.int16)).view(torch.float16)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    bqm.bqm_f16_gemm(w16, x16, y)
    torch.cuda.synchronize()
    return w, x, w16_ref, x16_ref, y.cpu().numpy()


# the tile widths 2..5 (64*NT output columns per workgroup) are all reached:
# small shapes take NT=2, (128, 128, 40000) NT=3, (256, 256, 30000) NT=4 on 256
# compute units, the full-size workload NT=5
# K = 64 per LDS stage: odd stage counts at K = 64, 192 and 320
@pytest.mark.parametrize("m,k,n", [(1, 64, 1), (17, 128, 33), (130, 256, 257), (129, 4096, 321), (300, 1280, 650),
                                   (512, 64, 1000), (128, 128, 40000), (256, 256, 30000), (3, 8192, 70),
                                   (40, 192, 100), (129, 320, 330)])
def test_f16_gemm_matches_oracle(bqm, m, k, n):
    _, _, w16, x16, y = gemm_case(bqm, m, k, n, seed=m + 3 * k + n)
    y_ref, T = oracle.f16_gemm(w16, x16)
    check_gemm(y, y_ref, T, f"f16 gemm m={m} k={k} n={n}")


def test_f16_gemm_one_hot(bqm):
    # a one-hot activation row returns one fp16 weight column exactly
    rng = np.random.default_rng(71)
    n, k = 300, 512
    w = workloads.q8_0_weights(n, k, rng)
    w16_ref = oracle.q8_0_dequant_f16(w, k)
    x = np.zeros((4, k), np.float32)
    x[1, 0] = 1.0
    x[2, 511] = -2.0
    x[3, 200] = 0.5
    x16_ref = oracle.f32_to_f16(x)
    y = bqm.bqm_f16_gemm(dev(w16_ref.view(np.int16)).view(torch.float16),
                         dev(x16_ref.view(np.int16)).view(torch.float16)).cpu().numpy()
    wf = w16_ref.view(np.float16).astype(np.float32)
    assert np.all(y[0] == 0)
    assert np.array_equal(y[1], wf[:, 0])
    assert np.array_equal(y[2], -2.0 * wf[:, 511])
    assert np.array_equal(y[3], 0.5 * wf[:, 200])


def test_f16_full_size_prefill(bqm):
    # m=512 prefill tokens, K=4096 -> N=20480 (the stacked expert gate+up
    # projection): the whole chain on the device, every output checked
    m, k, n = 512, 4096, 20480
    rng = np.random.default_rng(0)
    w = workloads.q8_0_weights(n, k, rng)
    x = workloads.activations(m, k, rng, outliers=True)
    w16 = dequant(bqm, w, k)
    x16 = torch.full((m, k), float("nan"), dtype=torch.float16, device=DEV)
    bqm.bqm_f16_cvt(dev(x), x16)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    bqm.bqm_f16_gemm(w16, x16, y)
    torch.cuda.synchronize()
    w16_ref = oracle.q8_0_dequant_f16(w, k)
    x16_ref = oracle.f32_to_f16(x)
    assert_f16_equal(bits(w16), w16_ref, "full-size dequant")
    assert_f16_equal(bits(x16), x16_ref, "full-size cast")
    y_ref, T = oracle.f16_gemm(w16_ref, x16_ref)
    check_gemm(y.cpu().numpy(), y_ref, T, "full-size f16 gemm")


def test_f16_mirror_within_the_pages_band(bqm):
    # against the exact product of the f32 activations and the Q8_0 weights
    # (no fp16 rounding at all), relative Frobenius error below the 1e-2 band
    m, k, n = 64, 4096, 640
    w, x, _, _, y = gemm_case(bqm, m, k, n, seed=17)
    q, d = workloads.unpack_q8_0(w, k)
    wd = q.astype(np.float64) * np.repeat(d.astype(np.float64), 32, axis=1)
    exact = x.astype(np.float64) @ wd.T
    rel = np.linalg.norm(y - exact) / np.linalg.norm(exact)
    assert rel <= 1e-2, f"relative error {rel:.3e}"
