"""GPU parity at the largest sizes: weight matrices past 4 GiB.

Every kernel addresses memory through 32-bit offsets inside buffer resources
whose base is moved per workgroup, tile or work item (in 64-bit arithmetic),
or through 64-bit indexes.  Matrices of 2^31 bytes and more are where a
32-bit product or a resource laid over the whole matrix would wrap or clip,
so these cases put rows on both sides of the 2 GiB and 4 GiB marks (and the
last rows) among the sampled outputs and check them against the oracle one
by one, at the same bars as the smaller cases.  Decode == verify is checked
bitwise at this size too.

Data: Q8_0 rows of K = 4096 with the usual quant and scale distributions,
generated in row chunks; e4m3 weights as uniform random codes without the
two NaN codes (the N(0, 0.02) generator would need 8 bytes of host memory
per weight at this size), with a fixed scale.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"
K = 4096
N_Q8 = 1_000_003          # 4096-input Q8_0 rows: 4,352,013,056 bytes
N_E8 = 1_050_001          # 4096-input e4m3 rows: 4,300,804,096 bytes


@pytest.fixture(scope="module")
def bqm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_matmul_02_amd as m

    m.lib()
    return m


def log(msg):
    print(msg, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def sample_rows(n, row_bytes, rng, extra=48):
    """Rows around the 2 GiB and 4 GiB byte marks, the first and last rows,
    and random ones."""
    marks = []
    for b in (2 ** 31, 2 ** 32):
        r = b // row_bytes
        marks += list(range(max(0, r - 2), min(n, r + 3)))
    rows = [0, 1, 2, n - 3, n - 2, n - 1] + marks + list(rng.integers(0, n, size=extra))
    return np.unique(np.array(rows, dtype=np.int64))


def pairs(rows, m, rng):
    """(token, row) pairs: every sampled row with two random tokens and token 0."""
    tok = np.concatenate([np.zeros(len(rows), np.int64), rng.integers(0, m, size=2 * len(rows))])
    row = np.concatenate([rows, rows, rows])
    return tok, row


def check_sampled(y_dev, tok, row, y_ref, T, what, tol=1e-5):
    y = y_dev[torch.from_numpy(tok).to(DEV), torch.from_numpy(row).to(DEV)].cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    zero = T == 0
    assert np.all(y[zero] == 0), f"{what}: nonzero output where all terms are 0"
    ratio = np.abs(y - y_ref)[~zero] / T[~zero]
    worst = float(ratio.max()) if ratio.size else 0.0
    log(f"{what}: {len(tok)} sampled outputs, max err/T = {worst:.3e}")
    assert worst <= tol, f"{what}: max err/sum|terms| = {worst:.3e} > {tol:.3e}"


@pytest.fixture(scope="module")
def q8_big(bqm):
    rng = np.random.default_rng(4242)
    nb = K // 32
    w = np.empty((N_Q8, nb * 34), np.uint8)
    blocks = w.reshape(N_Q8, nb, 34)
    step = 65536
    for r0 in range(0, N_Q8, step):
        r1 = min(N_Q8, r0 + step)
        blocks[r0:r1, :, 2:] = rng.integers(-127, 128, size=(r1 - r0, nb, 32), dtype=np.int8).view(np.uint8)
        sc = (10.0 ** rng.uniform(-3.0, -2.0, size=(r1 - r0, nb))).astype("<f2")
        blocks[r0:r1, :, 0:2] = sc.view(np.uint8).reshape(r1 - r0, nb, 2)
    assert w.nbytes > 2 ** 32
    log(f"Q8_0 weights {N_Q8} x {K}: {w.nbytes} bytes")
    return w, dev(w)


@pytest.fixture(scope="module")
def e8_big(bqm):
    rng = np.random.default_rng(4343)
    w = np.empty((N_E8, K), np.uint8)
    step = 65536
    for r0 in range(0, N_E8, step):
        r1 = min(N_E8, r0 + step)
        c = rng.integers(0, 256, size=(r1 - r0, K), dtype=np.uint8)
        c[(c & 0x7F) == 0x7F] = 0x00          # no NaN codes
        w[r0:r1] = c
    assert w.nbytes > 2 ** 32
    log(f"e4m3 weights {N_E8} x {K}: {w.nbytes} bytes")
    return w, dev(w)


# --------------------------------------------------------------------------- Q8_0


def test_q8_0_gemv_past_4gib(bqm, q8_big):
    w, wd = q8_big
    rng = np.random.default_rng(1)
    rows = sample_rows(N_Q8, w.shape[1], rng)
    x = workloads.activations(9, K, rng)
    xq_ref, xds_ref = oracle.q8_1_quantize(x)
    xq, xds = bqm.bqm_q8_1_quantize(dev(x))
    log("gemv m=1 (two launches), m=1 (one launch) and m=9 on the 4.35 GB matrix")
    y1 = bqm.bqm_q8_0_gemv(wd, xq[:1].contiguous(), xds[:1].contiguous())
    yf = bqm.bqm_q8_0_gemv_f32(wd, dev(x[:1]))
    y9 = bqm.bqm_q8_0_gemv(wd, xq, xds)
    torch.cuda.synchronize()
    assert np.array_equal(xq.cpu().numpy(), xq_ref)
    assert torch.equal(yf.view(torch.int32), y1.view(torch.int32)), "one launch != two launches"
    assert torch.equal(y9[0].view(torch.int32), y1[0].view(torch.int32)), "verify token 0 != decode"
    tok, row = pairs(rows, 1, rng)
    y_ref, T = oracle.q8_0_matmul_sampled(w, xq_ref, xds_ref, K, tok, row)
    check_sampled(y1, tok, row, y_ref, T, "gemv m=1")
    tok, row = pairs(rows, 9, rng)
    y_ref, T = oracle.q8_0_matmul_sampled(w, xq_ref, xds_ref, K, tok, row)
    check_sampled(y9, tok, row, y_ref, T, "gemv m=9")


@pytest.mark.parametrize("m", [40, 512])
def test_q8_0_mmq_past_4gib(bqm, q8_big, m):
    # m=40: the 128 x 64 tile; m=512: the 256 x 160 tile (2 GB of output)
    w, wd = q8_big
    rng = np.random.default_rng(2 + m)
    rows = sample_rows(N_Q8, w.shape[1], rng)
    x = workloads.activations(m, K, rng, outliers=True)
    xq_ref, xds_ref = oracle.q8_1_quantize(x)
    xq, xds = bqm.bqm_q8_1_quantize(dev(x))
    log(f"mmq m={m} on the 4.35 GB matrix")
    y = bqm.bqm_q8_0_gemm(wd, xq, xds)
    torch.cuda.synchronize()
    tok, row = pairs(rows, m, rng)
    y_ref, T = oracle.q8_0_matmul_sampled(w, xq_ref, xds_ref, K, tok, row)
    check_sampled(y, tok, row, y_ref, T, f"mmq m={m}")
    del y
    torch.cuda.empty_cache()


def test_f16_mirror_past_4gib(bqm, q8_big):
    # 600,000 rows dequantized to fp16: 4.9 GB of output, then the fp16 GEMM on it
    w, wd = q8_big
    n = 600_000
    rng = np.random.default_rng(3)
    log(f"dequant {n} x {K} to fp16, then the fp16 GEMM at m=16")
    w16 = bqm.bqm_q8_0_dequant_f16(wd[:n], K)
    x = workloads.activations(16, K, rng, outliers=True)
    x16_ref = oracle.f32_to_f16(x)
    x16 = dev(x16_ref.view(np.int16)).view(torch.float16)
    y = bqm.bqm_f16_gemm(w16, x16)
    torch.cuda.synchronize()
    rows = sample_rows(n, 2 * K, rng)
    got16 = w16[torch.from_numpy(rows).to(DEV)].view(torch.int16).cpu().numpy().view(np.uint16)
    want16 = oracle.q8_0_dequant_f16(w[rows], K)
    assert np.array_equal(got16, want16), "dequant differs on sampled rows"
    y_ref, T = oracle.f16_gemm(want16, x16_ref)         # [16, len(rows)]
    got = y[:, torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64)
    zero = T == 0
    assert np.all(got[zero] == 0)
    worst = float((np.abs(got - y_ref)[~zero] / T[~zero]).max())
    log(f"f16 gemm m=16 over 4.9 GB of fp16 weights: max err/T = {worst:.3e}")
    assert worst <= 1e-5
    del w16, y
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- e4m3


def test_e4m3_gemv_past_4gib(bqm, e8_big):
    w, wd = e8_big
    rng = np.random.default_rng(4)
    rows = sample_rows(N_E8, K, rng)
    x = workloads.activations(9, K, rng, outliers=True)
    ws = 1.0e-3
    log("e4m3 gemv m=1 and m=9 on the 4.3 GB matrix")
    y1 = bqm.bqm_e4m3_gemv(wd, dev(x[:1]), ws)
    y9 = bqm.bqm_e4m3_gemv(wd, dev(x), ws)
    torch.cuda.synchronize()
    assert torch.equal(y9[0].view(torch.int32), y1[0].view(torch.int32)), "verify token 0 != decode"
    for m, y in ((1, y1), (9, y9)):
        tok, row = pairs(rows, m, rng)
        y_ref, T = oracle.e4m3_gemv_sampled(w, x, ws, tok, row)
        check_sampled(y, tok, row, y_ref, T, f"e4m3 gemv m={m}")


def test_e4m3_gemms_past_4gib(bqm, e8_big):
    w, wd = e8_big
    rng = np.random.default_rng(5)
    rows = sample_rows(N_E8, K, rng)
    m = 128
    x = workloads.activations(m, K, rng)
    ws = 1.0e-3
    xq_ref, sc_ref = oracle.e4m3_quantize_amax(x, ws)
    xq, sc = bqm.bqm_e4m3_quantize_amax(dev(x), ws)
    torch.cuda.synchronize()
    assert np.array_equal(xq.cpu().numpy(), xq_ref)
    tok, row = pairs(rows, m, rng)
    y_ref, T = oracle.e4m3_matmul_sampled(w, xq_ref, sc_ref, tok, row)
    fp8_tol = 7 * 2.0 ** -13 + (8 * (K // 64) + 1) * 2.0 ** -24
    exact_tol = (27 + K / 128) * 2.0 ** -24
    for name, tol in (("bqm_e4m3_gemm", fp8_tol), ("bqm_e4m3_gemm_exact", exact_tol)):
        log(f"{name} m={m} on the 4.3 GB matrix")
        y = getattr(bqm, name)(wd, xq, sc)
        torch.cuda.synchronize()
        check_sampled(y, tok, row, y_ref, T, name, tol=tol)
        del y
    # block-128: the same codes with a random per-(128 x 128) grid
    grid = rng.uniform(1e-4, 1e-3, size=((N_E8 + 127) // 128, K // 128)).astype(np.float32)
    bxq, bxs = oracle.e4m3_blk_quantize(x)
    log(f"bqm_e4m3_blk_gemm m={m} on the 4.3 GB matrix")
    y = bqm.bqm_e4m3_blk_gemm(wd, dev(grid), dev(bxq), dev(bxs))
    torch.cuda.synchronize()
    y_ref, T = oracle.e4m3_blk_matmul_sampled(w, grid, bxq, bxs, tok, row)
    check_sampled(y, tok, row, y_ref, T, "blk gemm", tol=7 * 2.0 ** -13 + (K // 128 + 18) * 2.0 ** -24)
    del y
    torch.cuda.empty_cache()


def test_e4m3_nan_count_past_4gib(bqm, e8_big):
    w, wd = e8_big
    flat = wd.view(-1)
    log("NaN count over the 4.3 GB matrix")
    assert bqm.bqm_e4m3_nan_count(wd).item() == 0
    spots = [2 ** 32 + 5, w.size - 1, 2 ** 31 - 1]
    saved = [int(flat[p].item()) for p in spots]
    for p, c in zip(spots, (0x7F, 0xFF, 0x7F)):
        flat[p] = c
    try:
        assert bqm.bqm_e4m3_nan_count(wd).item() == 3
    finally:
        for p, v in zip(spots, saved):
            flat[p] = v
    assert bqm.bqm_e4m3_nan_count(wd).item() == 0
