"""GPU parity on seeded random shapes, one list per entry point.

The fixed cases elsewhere pin chosen tile boundaries; the kernels also pick
among tile shapes, token staging and slot splits from cost models over
(m, k, n), so shapes drawn at random (m and n log-uniform or uniform, k a
random multiple of each entry point's granularity, rows padded at random
where the row stride is free) reach choices and ragged edges the fixed lists do not.
The shapes come from one seeded generator at collection time, so a failing
case is named by its parameters and reruns as it is.  The oracle's work
(m * n * k) is capped so that every case finishes in seconds.

Bars are those of the fixed-case tests: quantized bytes and scales
bit-exact; f32 outputs within 1e-5 * sum|terms| (the fp8-core e4m3 GEMM and
the block-128 GEMM within the bounds derived from the fp8 matrix core's
group truncation), exactly 0 where sum|terms| is 0; the one-launch decode
step bitwise equal to the two calls.  Outputs start as NaN.
"""
import math

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


# ---------------------------------------------------------------- shape draws


def _size(rng, lo, hi):
    """log-uniform or uniform in [lo, hi], each half of the time"""
    if rng.random() < 0.5:
        v = math.exp(rng.uniform(math.log(lo), math.log(hi + 1)))
    else:
        v = rng.uniform(lo, hi + 1)
    return int(min(hi, max(lo, math.floor(v))))


def draw(seed, count, m_range, k_step, k_range, n_range=None, budget=None):
    """count shapes (m, k) or (m, k, n): m and n from _size, k a uniform
    multiple of k_step in k_range, cut so that m*n*k (or m*k) stays within
    budget (a draw whose smallest k is over it is drawn again)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        m = _size(rng, *m_range)
        n = 1 if n_range is None else _size(rng, *n_range)
        k_hi = k_range[1] if budget is None else min(k_range[1], int(budget // (m * n)))
        k_hi -= k_hi % k_step
        if k_hi < k_range[0]:
            continue
        k = k_step * int(rng.integers(k_range[0] // k_step, k_hi // k_step + 1))
        out.append((m, k) if n_range is None else (m, k, n))
    return out


MMQ_SHAPES = draw(9001, 14, (1, 1100), 256, (256, 4096), (1, 24000), 3.0e9)
GEMV_SHAPES = draw(9002, 12, (1, 15), 256, (256, 8192), (1, 30000), 2.0e9)
GEMV_F32_SHAPES = [(m, k, n) for m, k, n in draw(9003, 40, (1, 2), 256, (256, 8192), (1, 30000), 2.0e9)
                   if m * k <= 8192][:8]
Q8_1_SHAPES = draw(9004, 8, (1, 3000), 32, (32, 8192), budget=2.0e7)
E4Q_SHAPES = draw(9005, 10, (1, 5000), 4, (4, 8192), budget=2.0e7)
E4M3_GEMM_SHAPES = draw(9006, 10, (1, 1100), 128, (128, 4096), (1, 24000), 3.0e9)
E4M3_GEMV_SHAPES = draw(9007, 10, (1, 16), 256, (256, 8192), (1, 30000), 2.0e9)
BLK_Q_SHAPES = draw(9008, 10, (1, 3000), 16, (16, 8192), budget=2.0e7)
BLK_GEMM_SHAPES = draw(9009, 10, (1, 1100), 16, (16, 4096), (1, 24000), 3.0e9)
F16_GEMM_SHAPES = draw(9010, 8, (1, 1100), 64, (64, 4096), (1, 24000), 3.0e9)
F8ACC_SHAPES = draw(9011, 8, (1, 1100), 256, (256, 4096), (1, 24000), 3.0e9)
NAN_COUNTS = [int(c) for c in np.random.default_rng(9012).integers(1, 50_000_000, size=6)]


def ids(shapes):
    return ["x".join(map(str, s)) for s in shapes]


# ---------------------------------------------------------------- helpers


@pytest.fixture(scope="module")
def bqm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_matmul_02_amd as m

    m.lib()   # raises if the library is not built
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def nan_out(m, n):
    return torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)


def close(y_gpu, y_ref, T, what, tol=1e-5):
    y = y_gpu.astype(np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    zero = T == 0
    assert np.all(y[zero] == 0), f"{what}: nonzero output where all terms are 0"
    ratio = np.abs(y - y_ref)[~zero] / T[~zero]
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= tol, f"{what}: max err/sum|terms| = {worst:.3e} > {tol:.3e}"
    return worst


def fp8_bound(k):        # v_mfma_scale_f32_32x32x64_f8f6f4 over k/64 steps
    return 7 * 2.0 ** -13 + (8 * (k // 64) + 1) * 2.0 ** -24


def exact_bound(k):      # fp16 matrix cores, exact code conversion
    return (27 + k / 128) * 2.0 ** -24


def blk_bound(k):        # fp8 matrix core per 128-k block, f32 folds
    return 7 * 2.0 ** -13 + ((k + 127) // 128 + 18) * 2.0 ** -24


def f8acc_bound(k):      # two 16-deep fp8 MFMAs per 32-block, f32 folds
    return 7 * 2.0 ** -13 + (k // 32 + 4) * 2.0 ** -24


def padded_q8_0(n, k, rng):
    w = workloads.q8_0_weights(n, k, rng)
    pad = 16 * int(rng.integers(0, 4))
    if pad:
        w = np.concatenate([w, rng.integers(0, 256, size=(n, pad), dtype=np.uint8)], axis=1)
    return w


def q8_1_both(bqm, x):
    xq_ref, xds_ref = oracle.q8_1_quantize(x)
    xq, xds = bqm.bqm_q8_1_quantize(dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(xq.cpu().numpy(), xq_ref)
    assert np.array_equal(xds.cpu().numpy().view(np.uint32), xds_ref.view(np.uint32))
    return xq, xds, xq_ref, xds_ref


# ---------------------------------------------------------------- Q8_0 path


@pytest.mark.parametrize("m,k", Q8_1_SHAPES, ids=ids(Q8_1_SHAPES))
def test_random_q8_1_quantize(bqm, m, k):
    rng = np.random.default_rng(m * 31 + k)
    q8_1_both(bqm, workloads.activations(m, k, rng, outliers=True))


@pytest.mark.parametrize("m,k,n", MMQ_SHAPES, ids=ids(MMQ_SHAPES))
def test_random_mmq(bqm, m, k, n):
    rng = np.random.default_rng(m * 7 + k * 3 + n)
    w = padded_q8_0(n, k, rng)
    x = workloads.activations(m, k, rng, outliers=True)
    xq, xds, xq_ref, xds_ref = q8_1_both(bqm, x)
    y = nan_out(m, n)
    bqm.bqm_q8_0_gemm(dev(w), xq, xds, y)
    torch.cuda.synchronize()
    y_ref, T = oracle.q8_0_matmul(w, xq_ref, xds_ref, k)
    close(y.cpu().numpy(), y_ref, T, f"mmq {m}x{k}x{n} row bytes {w.shape[1]}")


@pytest.mark.parametrize("m,k,n", GEMV_SHAPES, ids=ids(GEMV_SHAPES))
def test_random_gemv(bqm, m, k, n):
    rng = np.random.default_rng(m * 7 + k * 3 + n + 1)
    w = padded_q8_0(n, k, rng)
    x = workloads.activations(m, k, rng)
    xq, xds, xq_ref, xds_ref = q8_1_both(bqm, x)
    y = nan_out(m, n)
    bqm.bqm_q8_0_gemv(dev(w), xq, xds, y)
    torch.cuda.synchronize()
    y_ref, T = oracle.q8_0_matmul(w, xq_ref, xds_ref, k)
    close(y.cpu().numpy(), y_ref, T, f"gemv {m}x{k}x{n} row bytes {w.shape[1]}")


@pytest.mark.parametrize("m,k,n", GEMV_F32_SHAPES, ids=ids(GEMV_F32_SHAPES))
def test_random_gemv_f32(bqm, m, k, n):
    rng = np.random.default_rng(m * 7 + k * 3 + n + 2)
    w = padded_q8_0(n, k, rng)
    x = workloads.activations(m, k, rng)
    wd, xd = dev(w), dev(x)
    y1 = nan_out(m, n)
    bqm.bqm_q8_0_gemv_f32(wd, xd, y=y1)
    xq, xds = bqm.bqm_q8_1_quantize(xd)
    y2 = bqm.bqm_q8_0_gemv(wd, xq, xds)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32)), "one launch != two calls"
    xq_ref, xds_ref = oracle.q8_1_quantize(x)
    y_ref, T = oracle.q8_0_matmul(w, xq_ref, xds_ref, k)
    close(y1.cpu().numpy(), y_ref, T, f"gemv_f32 {m}x{k}x{n}")


# ---------------------------------------------------------------- e4m3 path


@pytest.mark.parametrize("m,k", E4Q_SHAPES, ids=ids(E4Q_SHAPES))
def test_random_e4m3_quantize(bqm, m, k):
    rng = np.random.default_rng(m * 31 + k + 5)
    x = workloads.activations(m, k, rng, outliers=True)
    w_scale = float(np.float32(rng.uniform(1e-3, 1e-1)))
    xq_ref, sc_ref = oracle.e4m3_quantize_amax(x, w_scale)
    xq, sc = bqm.bqm_e4m3_quantize_amax(dev(x), w_scale)
    torch.cuda.synchronize()
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), sc_ref.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), xq_ref)


@pytest.mark.parametrize("kernel", ["fp8", "exact"])
@pytest.mark.parametrize("m,k,n", E4M3_GEMM_SHAPES, ids=ids(E4M3_GEMM_SHAPES))
def test_random_e4m3_gemm(bqm, m, k, n, kernel):
    rng = np.random.default_rng(m * 7 + k * 3 + n + 6)
    codes, w_scale = workloads.e4m3_weights(n, k, rng)
    x = workloads.activations(m, k, rng)
    xq_ref, sc_ref = oracle.e4m3_quantize_amax(x, w_scale)
    fn, bound = {"fp8": (bqm.bqm_e4m3_gemm, fp8_bound), "exact": (bqm.bqm_e4m3_gemm_exact, exact_bound)}[kernel]
    y = nan_out(m, n)
    fn(dev(codes), dev(xq_ref), dev(sc_ref), y)
    torch.cuda.synchronize()
    y_ref, T = oracle.e4m3_matmul(codes, xq_ref, sc_ref)
    worst = close(y.cpu().numpy(), y_ref, T, f"e4m3 {kernel} {m}x{k}x{n}", tol=bound(k))
    print(f"e4m3 {kernel} {m}x{k}x{n}: max err/T = {worst:.3e}", flush=True)


@pytest.mark.parametrize("m,k,n", E4M3_GEMV_SHAPES, ids=ids(E4M3_GEMV_SHAPES))
def test_random_e4m3_gemv(bqm, m, k, n):
    rng = np.random.default_rng(m * 7 + k * 3 + n + 7)
    codes, w_scale = workloads.e4m3_weights(n, k, rng)
    x = workloads.activations(m, k, rng, outliers=True)
    y = nan_out(m, n)
    bqm.bqm_e4m3_gemv(dev(codes), dev(x), w_scale, y)
    torch.cuda.synchronize()
    y_ref, T = oracle.e4m3_gemv(codes, x, w_scale)
    close(y.cpu().numpy(), y_ref, T, f"e4m3 gemv {m}x{k}x{n}")


# ---------------------------------------------------------------- block-128 FP8


@pytest.mark.parametrize("m,k", BLK_Q_SHAPES, ids=ids(BLK_Q_SHAPES))
def test_random_blk_quantize(bqm, m, k):
    rng = np.random.default_rng(m * 31 + k + 8)
    x = workloads.activations(m, k, rng, outliers=True)
    xq, xs = bqm.bqm_e4m3_blk_quantize(dev(x))
    torch.cuda.synchronize()
    xq_ref, xs_ref = oracle.e4m3_blk_quantize(x)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), xs_ref.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), xq_ref)


@pytest.mark.parametrize("m,k,n", BLK_GEMM_SHAPES, ids=ids(BLK_GEMM_SHAPES))
def test_random_blk_gemm(bqm, m, k, n):
    rng = np.random.default_rng(m * 7 + k * 3 + n + 9)
    w, grid = workloads.e4m3_blk_weights(n, k, rng)
    xq, xs = oracle.e4m3_blk_quantize(workloads.activations(m, k, rng, outliers=True))
    y = nan_out(m, n)
    bqm.bqm_e4m3_blk_gemm(dev(w), dev(grid), dev(xq), dev(xs), y)
    torch.cuda.synchronize()
    y_ref, T = oracle.e4m3_blk_matmul(w, grid, xq, xs)
    worst = close(y.cpu().numpy(), y_ref, T, f"blk {m}x{k}x{n}", tol=blk_bound(k))
    print(f"blk {m}x{k}x{n}: max err/T = {worst:.3e}", flush=True)


# ---------------------------------------------------------------- fp16 mirror


@pytest.mark.parametrize("m,k,n", F16_GEMM_SHAPES, ids=ids(F16_GEMM_SHAPES))
def test_random_f16_mirror(bqm, m, k, n):
    rng = np.random.default_rng(m * 7 + k * 3 + n + 10)
    w = workloads.q8_0_weights(n, k, rng)
    x = workloads.activations(m, k, rng, outliers=True)
    w16 = torch.full((n, k), float("nan"), dtype=torch.float16, device=DEV)
    x16 = torch.full((m, k), float("nan"), dtype=torch.float16, device=DEV)
    bqm.bqm_q8_0_dequant_f16(dev(w), k, w16)
    bqm.bqm_f16_cvt(dev(x).view(-1), x16.view(-1))
    y = nan_out(m, n)
    bqm.bqm_f16_gemm(w16, x16, y)
    torch.cuda.synchronize()
    w16_ref = oracle.q8_0_dequant_f16(w, k)
    x16_ref = oracle.f32_to_f16(x)
    assert np.array_equal(w16.view(torch.int16).cpu().numpy().view(np.uint16), w16_ref)
    assert np.array_equal(x16.view(torch.int16).cpu().numpy().view(np.uint16), x16_ref)
    y_ref, T = oracle.f16_gemm(w16_ref, x16_ref)
    close(y.cpu().numpy(), y_ref, T, f"f16 mirror {m}x{k}x{n}")


# ---------------------------------------------------------------- instrument and NaN scan


@pytest.mark.parametrize("dist", ["wide", "mid"])
@pytest.mark.parametrize("m,k,n", F8ACC_SHAPES, ids=ids(F8ACC_SHAPES))
def test_random_f8acc(bqm, m, k, n, dist):
    rng = np.random.default_rng(m * 7 + k * 3 + n + 11)
    w = workloads.accprobe_weights(n, k, rng, dist)
    xq, xds = workloads.accprobe_activations(m, k, rng, dist)
    y = nan_out(m, n)
    bqm.bqm_q8_0_gemm_f8acc(dev(w), dev(xq), dev(xds), y)
    torch.cuda.synchronize()
    y_ref, T = oracle.q8_0_matmul_e4m3(w, xq, xds, k)
    worst = close(y.cpu().numpy(), y_ref, T, f"f8acc {m}x{k}x{n} {dist}", tol=f8acc_bound(k))
    print(f"f8acc {m}x{k}x{n} {dist}: max err/T = {worst:.3e}", flush=True)


@pytest.mark.parametrize("count", NAN_COUNTS)
def test_random_nan_count(bqm, count):
    rng = np.random.default_rng(count)
    b = rng.integers(0, 256, size=count, dtype=np.uint8)
    got = bqm.bqm_e4m3_nan_count(dev(b)).item()
    assert got == oracle.e4m3_nan_count(b)
