"""GPU parity of the matrix-core verify GEMV (bqm_q8_0_gemv with 3..15 tokens
and K <= 4096).

Bars: every token's row of an m-token call is bitwise equal to a
single-token call of the dot4 kernel (the per-row order is reproduced: the
pages require identical per-row FP order across decode and verify), and
within 1e-5 * sum|terms| of the oracle, exactly 0 where the sum is 0.  The
shapes reach every chunk count (1..8 chunks of 8 block pairs per row), a last
chunk of 4 pairs, several row groups per workgroup iteration, ragged n, padded
rows, scale products in the f32 subnormal range and blocks whose scale is 0.
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


def close(y, y_ref, T, what, tol=1e-5):
    y = y.astype(np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    zero = T == 0
    assert np.all(y[zero] == 0), f"{what}: nonzero output where all terms are 0"
    ratio = np.abs(y - y_ref)[~zero] / T[~zero]
    assert ratio.size == 0 or ratio.max() <= tol, f"{what}: max err/sum|terms| = {ratio.max():.3e}"


def run(bqm, w, x, m):
    """The m-token call and the single-token calls of the same tokens, bits."""
    n = w.shape[0]
    wd = dev(w)
    xq, xds = bqm.bqm_q8_1_quantize(dev(x))
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    bqm.bqm_q8_0_gemv(wd, xq, xds, y)
    singles = [bqm.bqm_q8_0_gemv(wd, xq[t:t + 1].contiguous(), xds[t:t + 1].contiguous()) for t in range(m)]
    torch.cuda.synchronize()
    return y.cpu().numpy(), np.concatenate([s.cpu().numpy() for s in singles])


def assert_bitwise(y, ys, what):
    diff = y.view(np.uint32) != ys.view(np.uint32)
    if diff.any():
        t, r = np.argwhere(diff)[0]
        raise AssertionError(f"{what}: {diff.sum()} outputs differ from single-token calls, first (token {t}, row {r}): "
                             f"{y[t, r]!r} != {ys[t, r]!r}")


# k -> chunks per row: 256: 1 (4 pairs), 512: 1, 1280: 3 (last 4 pairs),
# 2048: 4, 2304: 5 (last 4), 3072: 6, 4096: 8
CASES = [(3, 256, 16), (15, 256, 300), (4, 512, 33), (9, 1280, 4096), (3, 1280, 129), (7, 2048, 77),
         (15, 2304, 200), (5, 3072, 1000), (3, 4096, 17), (9, 4096, 5152), (12, 4096, 257), (15, 4096, 1500)]


@pytest.mark.parametrize("m,k,n", CASES)
def test_mma_gemv_equals_single_token_and_oracle(bqm, m, k, n):
    rng = np.random.default_rng(900 + m * 13 + k + n)
    w = workloads.q8_0_weights(n, k, rng)
    x = workloads.activations(m, k, rng, outliers=True)
    x[0, 64:96] = 0.0                                       # an all-zero activation block
    y, ys = run(bqm, w, x, m)
    assert_bitwise(y, ys, f"m={m} k={k} n={n}")
    xq_ref, xds_ref = oracle.q8_1_quantize(x)
    y_ref, T = oracle.q8_0_matmul(w, xq_ref, xds_ref, k)
    close(y, y_ref, T, f"m={m} k={k} n={n}")


def test_mma_gemv_every_token_count(bqm):
    rng = np.random.default_rng(77)
    k, n = 4096, 333
    w = workloads.q8_0_weights(n, k, rng)
    x = workloads.activations(15, k, rng)
    for m in range(3, 16):
        y, ys = run(bqm, w, x[:m], m)
        assert_bitwise(y, ys, f"m={m}")


def test_mma_gemv_subnormal_scale_products(bqm):
    # d_x about 1e-36 against d_w in [1e-3, 1e-2]: every d_w*d_x is an f32
    # subnormal, so the matrix-core scale product must keep subnormals exactly
    # as the VALU multiply of the single-token kernel does; zero weight scales
    # give zero products.
    rng = np.random.default_rng(5)
    m, k, n = 9, 1280, 300
    quants = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    scales = (10 ** rng.uniform(-3, -2, size=(n, k // 32))).astype(np.float16)
    scales[::7, 3] = 0.0
    w = workloads.pack_q8_0(quants, scales)
    x = (workloads.activations(m, k, rng) * np.float32(1e-34)).astype(np.float32)
    y, ys = run(bqm, w, x, m)
    assert_bitwise(y, ys, "subnormal scale products")
    assert np.count_nonzero(y) > y.size // 2          # the products were not flushed to zero


def test_mma_gemv_padded_rows(bqm):
    rng = np.random.default_rng(8)
    m, k, n, pad = 6, 2048, 45, 32
    w = workloads.q8_0_weights(n, k, rng)
    w = np.concatenate([w, rng.integers(0, 256, size=(n, pad), dtype=np.uint8)], axis=1)
    x = workloads.activations(m, k, rng)
    y, ys = run(bqm, w, x, m)
    assert_bitwise(y, ys, "padded rows")
    xq_ref, xds_ref = oracle.q8_1_quantize(x)
    y_ref, T = oracle.q8_0_matmul(w, xq_ref, xds_ref, k)
    close(y, y_ref, T, "padded rows")


def test_mma_gemv_head(bqm):
    # the decode head, K=4096 -> N=64448, as a 9-token verify batch: bitwise
    # against single-token calls and within the bound of the oracle, on every
    # output
    m, k, n = 9, 4096, 64448
    rng = np.random.default_rng(0)
    w = workloads.q8_0_weights(n, k, rng)
    x = workloads.activations(m, k, rng)
    y, ys = run(bqm, w, x, m)
    assert_bitwise(y, ys, "head")
    xq_ref, xds_ref = oracle.q8_1_quantize(x)
    y_ref, T = oracle.q8_0_matmul(w, xq_ref, xds_ref, k)
    close(y, y_ref, T, "head")
