"""Every entry point inside a captured HIP graph (how bench.py times them, and
how an engine's decode step would run them): each replay must reproduce the
eager launches bit for bit, with eager work and synchronisations between the
replays (the NaN count's zeroing kernel included)."""
import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def bqm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_matmul_02_amd as m

    m.lib()
    return m


def test_graph_replays_match_eager(bqm):
    dev = "cuda:0"
    rng = np.random.default_rng(77)
    k = 4096
    w = torch.from_numpy(workloads.q8_0_weights(1000, k, rng)).to(dev)
    x1 = torch.from_numpy(workloads.activations(1, k, rng)).to(dev)
    x9 = torch.from_numpy(workloads.activations(9, k, rng)).to(dev)
    x64 = torch.from_numpy(workloads.activations(64, k, rng, outliers=True)).to(dev)
    codes, ws = workloads.e4m3_weights(320, k, rng)
    w8 = torch.from_numpy(codes).to(dev)
    bcodes, bgrid = workloads.e4m3_blk_weights(700, k, rng)
    wb = torch.from_numpy(bcodes).to(dev)
    gb = torch.from_numpy(bgrid).to(dev)
    wa = torch.from_numpy(workloads.accprobe_weights(300, k, rng, "wide")).to(dev)
    aq, ad = workloads.accprobe_activations(64, k, rng, "wide")
    aq, ad = torch.from_numpy(aq).to(dev), torch.from_numpy(ad).to(dev)

    def bufs():
        return {
            "xq1": torch.empty((1, k), dtype=torch.int8, device=dev),
            "xd1": torch.empty((1, k // 32, 2), dtype=torch.float32, device=dev),
            "y1": torch.empty((1, 1000), dtype=torch.float32, device=dev),
            "xq9": torch.empty((9, k), dtype=torch.int8, device=dev),
            "xd9": torch.empty((9, k // 32, 2), dtype=torch.float32, device=dev),
            "y9": torch.empty((9, 1000), dtype=torch.float32, device=dev),
            "xq64": torch.empty((64, k), dtype=torch.int8, device=dev),
            "xd64": torch.empty((64, k // 32, 2), dtype=torch.float32, device=dev),
            "y64": torch.empty((64, 1000), dtype=torch.float32, device=dev),
            "q8": torch.empty((64, k), dtype=torch.uint8, device=dev),
            "sc": torch.empty(4, dtype=torch.float32, device=dev),
            "y8": torch.empty((64, 320), dtype=torch.float32, device=dev),
            "y8x": torch.empty((64, 320), dtype=torch.float32, device=dev),
            "yf": torch.empty((1, 1000), dtype=torch.float32, device=dev),
            "ye1": torch.empty((1, 320), dtype=torch.float32, device=dev),
            "ye9": torch.empty((9, 320), dtype=torch.float32, device=dev),
            "nan": torch.empty(1, dtype=torch.int64, device=dev),
            "bq": torch.empty((64, k), dtype=torch.uint8, device=dev),
            "bs": torch.empty((64, k // 128), dtype=torch.float32, device=dev),
            "yb": torch.empty((64, 700), dtype=torch.float32, device=dev),
            "w16": torch.empty((1000, k), dtype=torch.float16, device=dev),
            "x16": torch.empty((64, k), dtype=torch.float16, device=dev),
            "y16": torch.empty((64, 1000), dtype=torch.float32, device=dev),
            "ya": torch.empty((64, 300), dtype=torch.float32, device=dev),
        }

    def step(b):
        bqm.bqm_q8_1_quantize(x1, b["xq1"], b["xd1"])
        bqm.bqm_q8_0_gemv(w, b["xq1"], b["xd1"], b["y1"])
        bqm.bqm_q8_1_quantize(x9, b["xq9"], b["xd9"])
        bqm.bqm_q8_0_gemv(w, b["xq9"], b["xd9"], b["y9"])
        bqm.bqm_q8_1_quantize(x64, b["xq64"], b["xd64"])
        bqm.bqm_q8_0_gemm(w, b["xq64"], b["xd64"], b["y64"])
        bqm.bqm_e4m3_quantize_amax(x64, ws, b["q8"], b["sc"])
        bqm.bqm_e4m3_gemm(w8, b["q8"], b["sc"], b["y8"])
        bqm.bqm_e4m3_gemm_exact(w8, b["q8"], b["sc"], b["y8x"])
        bqm.bqm_q8_0_gemv_f32(w, x1, b["yf"])
        bqm.bqm_e4m3_gemv(w8, x1, ws, b["ye1"])
        bqm.bqm_e4m3_gemv(w8, x9, ws, b["ye9"])
        bqm.bqm_e4m3_nan_count(wb, b["nan"])
        bqm.bqm_e4m3_blk_quantize(x64, b["bq"], b["bs"])
        bqm.bqm_e4m3_blk_gemm(wb, gb, b["bq"], b["bs"], b["yb"])
        bqm.bqm_q8_0_dequant_f16(w, k, b["w16"])
        bqm.bqm_f16_cvt(x64, b["x16"])
        bqm.bqm_f16_gemm(b["w16"], b["x16"], b["y16"])
        bqm.bqm_q8_0_gemm_f8acc(wa, aq, ad, b["ya"])

    eager = bufs()
    step(eager)
    torch.cuda.synchronize()

    graph_bufs = bufs()
    for v in graph_bufs.values():
        v.zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(graph_bufs)
    torch.cuda.synchronize()

    for rep in range(3):
        for v in graph_bufs.values():      # clear between replays (eager work)
            v.zero_()
        scratch = bufs()                    # unrelated eager launches between replays
        step(scratch)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, ref in eager.items():
            assert torch.equal(graph_bufs[name], ref), f"replay {rep}: {name} differs from the eager launch"


def test_two_streams_at_once_match_serial(bqm):
    # The library keeps no state between calls and uses no memory beyond the
    # caller's buffers, so the same calls issued on two streams at once (each
    # with its own buffers) give the serial results bit for bit; the stream
    # argument orders the work (the reads below wait on each stream's event).
    dev = "cuda:0"
    rng = np.random.default_rng(78)
    k = 4096
    w = torch.from_numpy(workloads.q8_0_weights(5000, k, rng)).to(dev)
    codes, ws = workloads.e4m3_weights(3000, k, rng)
    w8 = torch.from_numpy(codes).to(dev)
    xs = [torch.from_numpy(workloads.activations(m, k, rng, outliers=True)).to(dev) for m in (1, 9, 300)]

    def work(x1, x9, x300):
        xq, xd = bqm.bqm_q8_1_quantize(x300)
        q8, sc = bqm.bqm_e4m3_quantize_amax(x300, ws)
        return [bqm.bqm_q8_0_gemv_f32(w, x1), bqm.bqm_e4m3_gemv(w8, x9, ws),
                bqm.bqm_q8_0_gemm(w, xq, xd), bqm.bqm_e4m3_gemm(w8, q8, sc), bqm.bqm_e4m3_gemm_exact(w8, q8, sc)]

    serial = work(*xs)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    out = {}
    for _ in range(3):
        for name, s in (("a", s1), ("b", s2)):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                out[name] = work(*xs)
        for s in (s1, s2):
            torch.cuda.current_stream().wait_stream(s)
        for name in ("a", "b"):
            for i, (got, ref) in enumerate(zip(out[name], serial)):
                assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), f"stream {name}, call {i}"
