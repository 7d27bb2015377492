"""GPU parity of the one-launch decode step, bqm_q8_0_gemv_f32 (q8_1
quantization of the f32 activation inside every workgroup, then the Q8_0
GEMV).

Bars: bitwise equal to bqm_q8_1_quantize followed by bqm_q8_0_gemv (same
rule, same device code, same per-row operation order), and within
1e-5 * sum|terms| of the oracle (its q8_1 quantization, then its fp64
matmul), exactly 0 where the sum is 0.  The entry point is for decode
(m <= 2, m*k <= 8192: 1, 2, 4 or 8 float4 per thread, with and without
register-held activation operands); larger m or m*k are refused.  Covers
ragged n, padded rows, an all-zero and an underflowing activation block, and
the full decode head on every output.
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


def both_paths(bqm, w, x):
    m, n = x.shape[0], w.shape[0]
    wd, xd = dev(w), dev(x)
    y1 = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    bqm.bqm_q8_0_gemv_f32(wd, xd, y=y1)
    xq, xds = bqm.bqm_q8_1_quantize(xd)
    y2 = bqm.bqm_q8_0_gemv(wd, xq, xds)
    torch.cuda.synchronize()
    return y1.cpu().numpy(), y2.cpu().numpy()


CASES = [(1, 256, 1), (1, 256, 47), (2, 512, 100), (1, 1280, 67), (1, 2048, 300), (1, 4096, 4096),
         (2, 4096, 129), (1, 8192, 65), (2, 1280, 4096), (1, 4096, 5152), (2, 2048, 77),
         # 16-wave workgroups of the one-launch step (one row per tile, at least
         # 16 rows per CU): one item per wave, and two with a ragged last one
         (2, 4096, 4096), (1, 3072, 4100)]


@pytest.mark.parametrize("m,k,n", CASES)
def test_gemv_f32_equals_two_call_path_and_oracle(bqm, m, k, n):
    rng = np.random.default_rng(500 + m * 7 + k + n)
    w = workloads.q8_0_weights(n, k, rng)
    x = workloads.activations(m, k, rng, outliers=True)
    x[0, 32:64] = 0.0                                       # an all-zero block
    x[-1, :32] *= np.float32(1e-44)                         # amax/127 underflows to 0
    y1, y2 = both_paths(bqm, w, x)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), f"m={m} k={k} n={n}: differs from two calls"
    xq_ref, xds_ref = oracle.q8_1_quantize(x)
    y_ref, T = oracle.q8_0_matmul(w, xq_ref, xds_ref, k)
    close(y1, y_ref, T, f"gemv_f32 m={m} k={k} n={n}")


def test_gemv_f32_padded_rows(bqm):
    rng = np.random.default_rng(3)
    m, k, n, pad = 1, 4096, 37, 16
    w = workloads.q8_0_weights(n, k, rng)
    w = np.concatenate([w, rng.integers(0, 256, size=(n, pad), dtype=np.uint8)], axis=1)
    x = workloads.activations(m, k, rng)
    y1, y2 = both_paths(bqm, w, x)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_gemv_f32_decode_equals_verify_bitwise(bqm):
    rng = np.random.default_rng(43)
    k, n = 4096, 777
    w = dev(workloads.q8_0_weights(n, k, rng))
    x = dev(workloads.activations(2, k, rng))
    singles = [bqm.bqm_q8_0_gemv_f32(w, x[t:t + 1].contiguous()) for t in range(2)]
    y = bqm.bqm_q8_0_gemv_f32(w, x)
    for t in range(2):
        assert torch.equal(y[t].view(torch.int32), singles[t][0].view(torch.int32)), f"token {t}"
    xq, xds = bqm.bqm_q8_1_quantize(x)
    y9 = bqm.bqm_q8_0_gemv(w, xq, xds)
    assert torch.equal(y.view(torch.int32), y9.view(torch.int32))


@pytest.mark.parametrize("m,k", [(3, 256), (2, 8192), (1, 16384)])
def test_gemv_f32_refuses_beyond_decode(bqm, m, k):
    w = dev(workloads.q8_0_weights(8, k, np.random.default_rng(0)))
    x = dev(np.zeros((m, k), np.float32))
    with pytest.raises(RuntimeError):
        bqm.bqm_q8_0_gemv_f32(w, x)


@pytest.mark.parametrize("m", [1, 2])
def test_gemv_f32_decode_head(bqm, m):
    # the decode head, K=4096 -> N=64448 at m=1 and 2: bitwise against the
    # two-call path and against the oracle on every output
    k, n = 4096, 64448
    rng = np.random.default_rng(m)
    w = workloads.q8_0_weights(n, k, rng)
    x = workloads.activations(m, k, rng)
    y1, y2 = both_paths(bqm, w, x)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    xq_ref, xds_ref = oracle.q8_1_quantize(x)
    y_ref, T = oracle.q8_0_matmul(w, xq_ref, xds_ref, k)
    close(y1, y_ref, T, f"gemv_f32 head m={m}")
