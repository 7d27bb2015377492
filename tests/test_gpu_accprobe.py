"""GPU parity of the accumulator instrument's f32 arm (bqm_q8_0_gemm_f8acc)
against the CPU oracle.

The arm reads every quant byte as an e4m3 code and sums each 32-block on the
fp8 matrix cores (two 16-deep v_mfma_f32_32x32x16_fp8_fp8 steps) in f32,
then folds by d_w * d_x like the int8 MMQ.

The bar comes from the matrix core's measured datapath, not from f32
arithmetic.  Measured on MI355X (448 + one small product at each position):
the 8 products a lane supplies to one instruction are aligned to the largest
of them and every other product is truncated to 13 bits below that one's
leading bit (448 = 1.75 * 2^8 keeps multiples of 2^-5); products in other
lanes' groups and the accumulator input are added without that loss.  An
e4m3 x e4m3 product has at most 8 significant bits, so the largest product of
a group is exact and each of the other 7 errs by less than 2^-13 of it.  The
group sums are then accumulated in f32, and the fold adds at most
(K/32 + 1) * 2^-24 * T.  Hence

    |y - y_ref| <= (7 * 2^-13 + (K/32 + 4) * 2^-24) * T,

T the sum of the magnitudes of every product term (8.5e-4 * T at K = 4096;
the cases below print their maxima: the full-range "wide" bytes reach about
7e-5 * T at K = 256 here (1.9e-4 * T over the 10 M outputs of a random
646 x 256 x 16124 case) and 2.3e-5 * T at 512 x 5120 x 5120, the mid-exponent bytes
below 1e-7 * T).  Exactly 0
where T is 0.  The int8 arm is bqm_q8_0_gemm itself, covered by the MMQ's
parity tests.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


def tolerance(k):
    return 7 * 2.0 ** -13 + (k // 32 + 4) * 2.0 ** -24


@pytest.fixture(scope="module")
def bqm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_matmul_02_amd as m

    m.lib()
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run(bqm, w, xq, xds):
    m, n = xq.shape[0], w.shape[0]
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    bqm.bqm_q8_0_gemm_f8acc(dev(w), dev(xq), dev(xds), y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check(y_gpu, y_ref, T, what, tol):
    y = y_gpu.astype(np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    zero = T == 0
    assert np.all(y[zero] == 0), f"{what}: nonzero output where all terms are 0"
    ratio = np.abs(y - y_ref)[~zero] / T[~zero]
    worst = ratio.max() if ratio.size else 0.0
    print(f"{what}: max err/T = {worst:.3e}", flush=True)
    assert worst <= tol, f"{what}: max err/sum|terms| = {worst:.3e} > {tol}"


@pytest.mark.parametrize("dist", ["wide", "mid"])
@pytest.mark.parametrize("m,k,n", [(1, 256, 1), (17, 256, 33), (130, 512, 257), (64, 4096, 640),
                                   (200, 1024, 129), (65, 2048, 70)])
def test_f8acc_matches_oracle(bqm, m, k, n, dist):
    rng = np.random.default_rng(2000 + m + k + n)
    w = workloads.accprobe_weights(n, k, rng, dist)
    xq, xds = workloads.accprobe_activations(m, k, rng, dist)
    y_ref, T = oracle.q8_0_matmul_e4m3(w, xq, xds, k)
    check(run(bqm, w, xq, xds), y_ref, T, f"f8acc m={m} k={k} n={n} {dist}", tolerance(k))


@pytest.mark.parametrize("dist", ["wide", "mid"])
def test_f8acc_wide_tile(bqm, dist):
    # m=512, N=20480: the MMQ's 256-token x 160-row tile, with the f32 arm's
    # block sums
    m, k, n = 512, 512, 20480
    rng = np.random.default_rng(4000)
    w = workloads.accprobe_weights(n, k, rng, dist)
    xq, xds = workloads.accprobe_activations(m, k, rng, dist)
    y_ref, T = oracle.q8_0_matmul_e4m3(w, xq, xds, k)
    check(run(bqm, w, xq, xds), y_ref, T, f"f8acc wide tile {dist}", tolerance(k))


@pytest.mark.parametrize("dist", ["wide", "mid"])
def test_f8acc_96_row_tile(bqm, dist):
    # m=512, N=5152: the MMQ's 128-token x 96-row tile (12 waves), with the f32
    # arm's block sums; the last row tile holds 64 of 96 rows
    m, k, n = 512, 512, 5152
    rng = np.random.default_rng(4100)
    w = workloads.accprobe_weights(n, k, rng, dist)
    xq, xds = workloads.accprobe_activations(m, k, rng, dist)
    y_ref, T = oracle.q8_0_matmul_e4m3(w, xq, xds, k)
    check(run(bqm, w, xq, xds), y_ref, T, f"f8acc 96-row tile {dist}", tolerance(k))


def test_f8acc_group_truncation_as_measured(bqm):
    # 448 plus one small product in the same 8-value lane group keeps only
    # multiples of 2^-5; in the other lane half it is added exactly.  This
    # pins the datapath the tolerance above is derived from.
    k = 256
    w = workloads.pack_q8_0(np.full((1, k), 0x38, np.int8), np.ones((1, k // 32), np.float16))   # weights 1.0
    xq = np.zeros((2, k), np.int8)
    xq[:, 0] = 0x7E                      # 448
    xq[0, 1] = 0x21                      # 0.140625, same group as k = 0
    xq[1, 16] = 0x21                     # same value, the other lane half
    xds = np.zeros((2, k // 32, 2), np.float32)
    xds[:, :, 0] = 1.0
    y = run(bqm, w, xq, xds)[:, 0]
    assert y[0] == np.float32(448.125)
    assert y[1] == np.float32(448.140625)


def test_f8acc_one_hot_is_exact(bqm):
    # one activation byte 0x38 (e4m3 1.0) per token with d_x = 1: every
    # output is one exact product d_w * dec(q_w)
    k, n = 512, 96
    rng = np.random.default_rng(5)
    w = workloads.accprobe_weights(n, k, rng)
    cols = [0, 31, 32, 300, 511]
    xq = np.zeros((len(cols), k), np.int8)
    for t, c in enumerate(cols):
        xq[t, c] = 0x38
    xds = np.zeros((len(cols), k // 32, 2), np.float32)
    xds[:, :, 0] = 1.0
    y = run(bqm, w, xq, xds)
    y_ref, _ = oracle.q8_0_matmul_e4m3(w, xq, xds, k)
    assert np.array_equal(y.astype(np.float64), y_ref)


def test_f8acc_instrument_shape_every_output(bqm):
    # m=512 on the square reference shape of the instrument's sheet, 5120 -> 5120
    m, k, n = 512, 5120, 5120
    rng = np.random.default_rng(0)
    w = workloads.accprobe_weights(n, k, rng)
    xq, xds = workloads.accprobe_activations(m, k, rng)
    y_ref, T = oracle.q8_0_matmul_e4m3(w, xq, xds, k)
    check(run(bqm, w, xq, xds), y_ref, T, "f8acc 512x5120x5120", tolerance(k))
