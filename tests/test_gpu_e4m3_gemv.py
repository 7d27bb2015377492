"""GPU parity of the e4m3 decode GEMV against the CPU oracle.

Bar: within 1e-5 * sum|terms| per output (f32 chains of 16 fma, a slot tree
of at most 3 levels and a 6-level lane tree: (16 + 3 + 6) * 2^-24 < 1.5e-6),
exactly 0 where sum|terms| is 0; every token's result identical whatever m
(decode == verify, across the one-token, staged-token and slot-split
kernels); outputs pre-filled with NaN to prove they are fully overwritten.
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


def check(y_gpu, y_ref, T, what, tol=1e-5):
    y = y_gpu.astype(np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    zero = T == 0
    assert np.all(y[zero] == 0), f"{what}: nonzero output where all terms are 0"
    ratio = np.abs(y - y_ref)[~zero] / T[~zero]
    assert ratio.size == 0 or ratio.max() <= tol, f"{what}: max err/sum|terms| = {ratio.max():.3e}"


def run(bqm, codes, x, ws):
    m, n = x.shape[0], codes.shape[0]
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    bqm.bqm_e4m3_gemv(dev(codes), dev(x), ws, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


CASES = [(1, 256, 1), (1, 4096, 1000), (1, 1280, 333), (2, 1280, 333), (3, 4096, 257), (4, 8192, 64),
         (1, 8192, 65), (5, 2304, 100), (9, 4096, 129), (16, 1024, 77), (7, 768, 5), (1, 512, 4099)]


@pytest.mark.parametrize("m,k,n", CASES)
def test_e4m3_gemv_matches_oracle(bqm, m, k, n):
    rng = np.random.default_rng(1000 + 7 * m + k + n)
    codes, ws = workloads.e4m3_weights(n, k, rng)
    x = workloads.activations(m, k, rng, outliers=True)
    y = run(bqm, codes, x, ws)
    y_ref, T = oracle.e4m3_gemv(codes, x, ws)
    check(y, y_ref, T, f"m={m} k={k} n={n}")


def test_e4m3_gemv_zero_activation_and_one_hot(bqm):
    rng = np.random.default_rng(5)
    n, k = 300, 4096
    codes, ws = workloads.e4m3_weights(n, k, rng)
    x = np.zeros((3, k), np.float32)
    x[1, 77] = 1.0
    x[2, 4095] = -0.5
    y = run(bqm, codes, x, ws)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert np.all(y[0] == 0)
    assert np.array_equal(y[1], np.float32(ws) * dec[:, 77])
    assert np.array_equal(y[2], np.float32(ws) * (-0.5 * dec[:, 4095]))


@pytest.mark.parametrize("k", [4096, 1280, 8192])
def test_e4m3_gemv_decode_equals_verify_bitwise(bqm, k):
    rng = np.random.default_rng(9 + k)
    n = 513
    codes, ws = workloads.e4m3_weights(n, k, rng)
    x = workloads.activations(9, k, rng)
    y9 = run(bqm, codes, x, ws)
    for t in range(9):
        y1 = run(bqm, codes, x[t:t + 1], ws)
        assert np.array_equal(y1[0], y9[t]), f"token {t}: decode differs from the 9-token call"


@pytest.mark.parametrize("m", [1, 9])
def test_e4m3_gemv_full_size_stacked_expert(bqm, m):
    # K=4096 -> N=20480 (the stacked expert gate+up shape), every output
    rng = np.random.default_rng(20480 + m)
    n, k = 20480, 4096
    codes, ws = workloads.e4m3_weights(n, k, rng)
    x = workloads.activations(m, k, rng)
    y = run(bqm, codes, x, ws)
    y_ref, T = oracle.e4m3_gemv(codes, x, ws)
    check(y, y_ref, T, f"m={m} 4096->20480")


def singles(bqm, codes, x, ws):
    return np.concatenate([run(bqm, codes, x[t:t + 1], ws) for t in range(x.shape[0])])


def assert_bitwise(y, ys, what):
    diff = y.view(np.uint32) != ys.view(np.uint32)
    if diff.any():
        t, r = np.argwhere(diff)[0]
        raise AssertionError(f"{what}: {diff.sum()} outputs differ from single-token calls, first (token {t}, row {r})")


# k -> chunk slots per lane: 1280: 2 (the second partly empty), 2048: 2,
# 2304: 3 (a fourth, empty slot wave), 4096: 4, 4352: 5 and 8192: 8 (eight
# slot waves, 4-token groups)
@pytest.mark.parametrize("k,n", [(1280, 37), (2048, 5), (2304, 130), (4096, 3), (4352, 61), (8192, 9)])
def test_e4m3_gemv_slot_split_every_token_count(bqm, k, n):
    # every m = 2..16 bitwise equal to single-token calls (one, two, three and
    # four token groups; n below and above the rows of one item)
    rng = np.random.default_rng(31 * k + n)
    codes, ws = workloads.e4m3_weights(n, k, rng)
    x = workloads.activations(16, k, rng, outliers=True)
    ys = singles(bqm, codes, x, ws)
    y_ref, T = oracle.e4m3_gemv(codes, x, ws)
    check(ys, y_ref, T, f"single tokens k={k} n={n}")
    for m in range(2, 17):
        y = run(bqm, codes, x[:m], ws)
        assert_bitwise(y, ys[:m], f"m={m} k={k} n={n}")


def test_e4m3_gemv_slot_split_groups_on_xcds(bqm):
    # enough rows that token groups of the same rows are placed on one XCD
    # (m = 11: two groups of 6 and 5 tokens; m = 16 at k = 8192: four groups)
    rng = np.random.default_rng(77)
    for m, k, n in [(11, 4096, 4099), (16, 8192, 2050)]:
        codes, ws = workloads.e4m3_weights(n, k, rng)
        x = workloads.activations(m, k, rng)
        y = run(bqm, codes, x, ws)
        y_ref, T = oracle.e4m3_gemv(codes, x, ws)
        check(y, y_ref, T, f"m={m} k={k} n={n}")
        sel = [0, m // 2, m - 1]
        assert_bitwise(y[sel], singles(bqm, codes, x[sel], ws), f"m={m} k={k} n={n}")
