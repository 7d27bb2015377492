"""The entry points inside a captured HIP graph (how bench.py times them, and
how an engine's decode step would run them): each replay must reproduce the
eager launches bit for bit, with eager work and synchronisations between the
replays."""
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
