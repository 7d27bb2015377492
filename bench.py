"""Benchmark of the block-quantized projection matmul on one MI355X.

One step is one pass of the hot path over one batch of the decode-head
workload: the q8_1 quantization of the f32 activation (m=1, K=4096) and the
Q8_0 GEMV against the 4096 -> 64448 head (280 MB of weights), in one launch
(bqm_q8_0_gemv_f32; the two-launch path, bqm_q8_1_quantize + bqm_q8_0_gemv,
is timed beside it).  ``value`` is the step's algorithmic bytes (weights +
f32 activation + output) per second.  Inputs are resident in HBM before timing starts; three copies of the
weights are rotated so every step streams its weights from HBM rather than
the 256 MB Infinity Cache.

The same JSON line also carries the prefill rows, each timed the same way:
the m=512 MMQ GEMM (q8_1 quantize + int8 GEMM) at N in {4096, 5152, 20480}
and the FP8-E4M3 GEMM (amax quantize + fp8 GEMM) at N=20480, with int8/fp8
TOPS and their fraction of the matrix-core peak; the e4m3 decode GEMV
(raw e4m3 weights, f32 activations) at m=1 and 9 on the head shape; the fp16
mirror prefill (f32 -> fp16 cast + fp16 GEMM, m=512, K=4096, N=20480, with the
one-off Q8_0 -> fp16 dequant timed beside it); the block-128 FP8 prefill
(per-(token, 128-k block) e4m3 quantize + per-block GEMM, m=512, K=4096,
N=20480, with the one-off NaN scan of the weight); the accumulator instrument
(the MMQ with its int8 MFMA + s32 block sums against the same kernel with
fp8 MFMAs + f32 block sums, m=512, the 27B projection shapes, both arms timed
interleaved per rep, medians, geomean of the ratio); a roofline object for the
dominant kernel (the GEMV), measured with HIP events on the launch stream;
and the CPU oracle timed on the host cores on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Q8_0 GEMV GB/s (m=1) + MMQ int8 TOPS (m=512), % of MI355X roofline"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0          # dense int8 MFMA
FP8_PEAK_TFLOPS = 5000.0         # dense fp8 MFMA
FP16_PEAK_TFLOPS = 2500.0        # dense fp16 MFMA
ROTATE = 3                       # weight copies for the 280 MB head (841 MB rotated)
ROTATE_BYTES = 600_000_000       # smaller weights: copies enough for >= 600 MB, past the 256 MB cache


def copies_for(nbytes: int) -> int:
    """Weight copies to rotate so that every launch streams its weights from HBM."""
    return max(ROTATE, min(64, -(-ROTATE_BYTES // nbytes)))


def q8_0_bytes(m, k, n):
    """Algorithmic bytes of one Q8_0 matmul: weights + xq + xds + y."""
    return n * (k // 32) * 34 + m * k + m * (k // 32) * 8 + m * n * 4


def recorded_traffic():
    """HBM bytes per launch of the head GEMV from the committed counter passes
    (profiles/gemv_head_traffic.json), or None when the kernel sources have
    changed since the counters were taken (the record carries their hash)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemv_head_traffic.json")
    try:
        rec = json.load(open(path))
        h = hashlib.sha256()
        for fn in rec["sources"]:
            h.update(open(os.path.join(ROOT, "block_quantized_matmul_02_amd", "csrc", fn), "rb").read())
        return int(rec["traffic_bytes"]) if h.hexdigest() == rec["sources_sha256"] else None
    except (OSError, KeyError, ValueError):
        return None


class region:
    """A named marker range around GPU work (torch's range markers, roctx on
    ROCm), so a profiler run with ``--marker-trace --kernel-rename`` names each
    kernel dispatch by the workload and call it belongs to; it costs nothing
    without a profiler."""

    def __init__(self, torch, name):
        self.torch, self.name = torch, name

    def __enter__(self):
        if self.name:
            self.torch.cuda.nvtx.range_push(self.name)
        return self

    def __exit__(self, *exc):
        if self.name:
            self.torch.cuda.nvtx.range_pop()
        return False


def timed_loop(torch, stream, steps, fns, label=None):
    """Time ``steps`` passes of ``fns`` (a list of (name, callable)); with a
    ``label`` every dispatch runs inside the marker range "label: name" (the
    whole loop: "label: step").

    The launches are captured once into a HIP graph (torch.cuda.graph) and
    replayed, so host-side launch overhead is out of the measurement: the
    kernels run back to back as they would inside an engine's decode step.
    Untimed replays run first until three in a row agree within 0.5% (the
    clocks have settled); the step time then comes from events on the replay
    stream around one replay of the ``steps`` passes.  Each callable's duration comes from a second graph
    that launches it ``steps`` times back to back, timed the same way.
    Returns (total ms of the step loop, {name: mean ms per call})."""
    def capture(calls):
        for s in range(2):                # first calls outside capture (one-time setup)
            for fn in calls:
                fn(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in range(steps):
                for fn in calls:
                    fn(s)
        torch.cuda.synchronize()
        return g

    def one_replay(g):
        rs = torch.cuda.current_stream()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(rs)
        g.replay()
        b.record(rs)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    def replay_ms(g, reps=1):
        # untimed warm replays until the clocks have settled: at least 50 ms
        # of GPU work and three replays in a row within 0.5% of each other
        # (at most 2 s), so a short --warmup does not time ramping clocks
        hist, t_end = [one_replay(g)], time.perf_counter() + 2.0
        while time.perf_counter() < t_end:
            hist.append(one_replay(g))
            last = hist[-3:]
            if len(hist) >= 4 and sum(hist[1:]) >= 50.0 and max(last) <= 1.005 * min(last):
                break
        times = [one_replay(g) for _ in range(reps)]
        return sorted(times)[len(times) // 2]

    # the step loop: exactly `steps` passes, timed once; each kernel: the
    # median of 9 replays of `steps` back-to-back launches
    tag = (lambda what: f"{label}: {what}") if label else (lambda what: None)
    with region(torch, tag("step")):
        total_ms = replay_ms(capture([fn for _, fn in fns]))
    per = {}
    for name, fn in fns:
        with region(torch, tag(name)):
            per[name] = replay_ms(capture([fn]), reps=9) / steps
    return total_ms, per


# the accumulator instrument's two shape sheets (accprobe_bench.rs, fn main:
# shapes_27b and shapes_1p7b), (in_f, out_f, projection)
ACCPROBE_LABELS_27B = [(5120, 12288, "q_proj"), (5120, 1024, "k/v_proj"), (6144, 5120, "o_proj"),
                       (5120, 17408, "gate/up_proj"), (17408, 5120, "down_proj"), (5120, 5120, "square-ref")]
ACCPROBE_LABELS_1P7B = [(2048, 2048, "q_proj"), (2048, 1024, "k/v_proj"), (2048, 2048, "o_proj"),
                        (2048, 6144, "gate/up_proj"), (6144, 2048, "down_proj")]


def host_description(threads):
    """The host the CPU oracle ran on: logical CPUs, OpenMP threads, model."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_count": os.cpu_count(), "omp_threads": threads, "model": model,
            "sched_affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def cpu_oracle_legs(single: bool):
    """Time the CPU oracle (plain C, OpenMP over output rows) on the measured
    workloads, on whatever OpenMP team this process has.  Each entry gives
    the rate in the GPU row's own unit.  The m=512 GEMMs run once at full
    size with the host's threads; on one thread they run on the first 1024
    weight rows only (the full size would take minutes), which the entry says.
    Bounded: about 15 s with 16 threads, about 15 s on one."""
    import oracle
    import workloads

    res = {"threads": oracle.num_threads()}

    def loop(fn, seconds):
        r, t0 = 0, time.perf_counter()
        while True:
            fn()
            r += 1
            dt = time.perf_counter() - t0
            if dt >= seconds:
                return r, dt

    # decode head step (quantize + GEMV, m=1, K=4096, N=64448): the headline's workload
    m, k, n = 1, 4096, 64448
    w = workloads.q8_0_weights(n, k, np.random.default_rng(0))
    x = workloads.activations(m, k, np.random.default_rng(1))

    def head():
        q, d = oracle.q8_1_quantize(x)
        oracle.q8_0_matmul(w, q, d, k)
    r, dt = loop(head, 3.0 if single else 4.0)
    byts = n * (k // 32) * 34 + m * k * 4 + m * n * 4
    res["decode_head_step"] = {"value": round(r * byts / dt / 1e9, 2), "unit": "GB/s",
                               "sample": f"the decode-head step (q8_1 quantize + Q8_0 matmul, m=1, K=4096, "
                                         f"N=64448) repeated {r} times in {dt:.1f} s"}
    del w

    # GEMV m=1, 4096 -> 4096 step: median of 3 timed loops
    m, k, n = 1, 4096, 4096
    w = workloads.q8_0_weights(n, k, np.random.default_rng(0))
    x = workloads.activations(m, k, np.random.default_rng(1))

    def gemv():
        q, d = oracle.q8_1_quantize(x)
        oracle.q8_0_matmul(w, q, d, k)
    rates = []
    for _ in range(3):
        r, dt = loop(gemv, 0.7)
        rates.append(r / dt)
    byts = n * (k // 32) * 34 + m * k * 4 + m * n * 4
    rate = sorted(rates)[1]
    res["gemv_m1_4096x4096_step"] = {"value": round(rate * byts / 1e9, 2), "unit": "GB/s",
                                     "us_per_step": round(1e6 / rate, 1),
                                     "sample": "q8_1 quantize + Q8_0 matmul, m=1, K=4096, N=4096; median of 3 "
                                               "loops of >= 0.7 s"}

    # MMQ GEMM m=512, K=4096, N=20480 (1% outliers x10): quantize + matmul, one run
    m, k, n = 512, 4096, 20480
    rows = 1024 if single else n
    w = workloads.q8_0_weights(n, k, np.random.default_rng(0))[:rows]
    x = workloads.activations(m, k, np.random.default_rng(1), outliers=True)
    t0 = time.perf_counter()
    q, d = oracle.q8_1_quantize(x)
    tq = time.perf_counter() - t0
    oracle.q8_0_matmul(w, q, d, k)
    dt = time.perf_counter() - t0
    ops = 2.0 * m * rows * k
    res["mmq_m512_n20480"] = {"value": round(ops / dt / 1e9, 2), "unit": "GOPS (2*m*n*k / s)",
                              "seconds": round(dt, 3), "quantize_s": round(tq, 4),
                              "sample": f"q8_1 quantize + Q8_0 matmul, m=512, K=4096, "
                                        f"{'the first 1024 of the' if single else 'all'} 20480 weight rows, one run"}
    del w

    # FP8 GEMM m=512, K=4096, N=20480: amax quantize + e4m3 matmul, one run
    codes, w_scale = workloads.e4m3_weights(n, k, np.random.default_rng(0))
    codes = np.ascontiguousarray(codes[:rows])
    x = workloads.activations(m, k, np.random.default_rng(1))
    t0 = time.perf_counter()
    xq8, sc = oracle.e4m3_quantize_amax(x, w_scale)
    tq = time.perf_counter() - t0
    oracle.e4m3_matmul(codes, xq8, sc)
    dt = time.perf_counter() - t0
    ops = 2.0 * m * rows * k
    res["e4m3_m512_n20480"] = {"value": round(ops / dt / 1e9, 2), "unit": "GFLOPS (2*m*n*k / s)",
                               "seconds": round(dt, 3), "quantize_s": round(tq, 4),
                               "sample": f"e4m3 amax quantize + fp64 e4m3 matmul, m=512, K=4096, "
                                         f"{'the first 1024 of the' if single else 'all'} 20480 weight rows, one run"}
    return res


def cpu_single_thread_child():
    """The CPU legs on one thread, in a child process (OpenMP fixes its team
    size when a process starts); None if the child fails."""
    import subprocess
    try:
        res = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-leg"],
                             env={**os.environ, "OMP_NUM_THREADS": "1"}, capture_output=True, text=True,
                             timeout=300)
        return json.loads(res.stdout.strip().splitlines()[-1])
    except (subprocess.SubprocessError, ValueError, OSError, IndexError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--sweep-shapes", default=None,
                    help="comma-separated KxN shapes for the decode/verify sweep (default: all four)")
    ap.add_argument("--only", choices=["gemv", "sweep", "mmq", "e4m3", "e4m3_gemv", "f16", "accprobe", "e4m3_blk", "copy"], default=None,
                    help="run one part only (for profiler passes); 'copy' runs a plain 1 GiB device copy "
                         "that calibrates the HBM byte counters")
    ap.add_argument("--cpu-leg", action="store_true",
                    help="internal: time the CPU oracle legs on this process's OpenMP team and print JSON "
                         "(no GPU use)")
    args = ap.parse_args()
    if args.cpu_leg:
        print(json.dumps(cpu_oracle_legs(single=True)), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the path would shard "
              "along N (weight rows) with no exchange, and only the one-GPU share is built and timed",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import block_quantized_matmul_02_amd as bqm
    import workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    rng = np.random.default_rng(0)
    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
           "data": "synthetic"}

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    if args.only == "copy":
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "launches": args.steps}), flush=True)
        return

    # ---------------------------------------------------------------- decode head GEMV
    if args.only in (None, "gemv"):
        m, k, n = 1, 4096, 64448
        log(f"[bench] generating head weights {n}x{k} Q8_0")
        w_host = workloads.q8_0_weights(n, k, rng)
        x_host = workloads.activations(m, k, rng)
        ws = [torch.from_numpy(w_host).to(dev)]
        for _ in range(ROTATE - 1):
            ws.append(ws[0].clone())
        x = torch.from_numpy(x_host).to(dev)
        xq = torch.empty((m, k), dtype=torch.int8, device=dev)
        xds = torch.empty((m, k // 32, 2), dtype=torch.float32, device=dev)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        # the step: one launch that quantizes x to q8_1 in every workgroup and
        # runs the GEMV (bitwise equal to the two-launch path timed below)
        fns = [("gemv_f32", lambda s: bqm.bqm_q8_0_gemv_f32(ws[s % ROTATE], x, y))]
        log("[bench] gemv warmup")
        hl = f"Q8_0 decode head m=1 {k}->{n}, one launch"
        timed_loop(torch, stream, args.warmup, fns, hl)
        log("[bench] gemv timed")
        total_ms, per = timed_loop(torch, stream, args.steps, fns, hl)
        fns2 = [("quantize", lambda s: bqm.bqm_q8_1_quantize(x, xq, xds)),
                ("gemv", lambda s: bqm.bqm_q8_0_gemv(ws[s % ROTATE], xq, xds, y))]
        hl2 = f"Q8_0 decode head m=1 {k}->{n}, two launches"
        timed_loop(torch, stream, args.warmup, fns2, hl2)
        total2_ms, per2 = timed_loop(torch, stream, args.steps, fns2, hl2)
        step_bytes = n * (k // 32) * 34 + m * k * 4 + m * n * 4       # weights + f32 activation + y
        ms_step = total_ms / args.steps
        achieved = step_bytes / (per["gemv_f32"] * 1e-3) / 1e9
        out.update({
            "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
            "unit": "GB/s",
            "ms_per_step": round(ms_step, 5),
            "config": {"workload": "decode head GEMV: m=1, K=4096, N=64448, Q8_0 weights, f32 activation "
                                   "quantized on the device to q8_1 (in the GEMV launch)",
                       "m": m, "k": k, "n": n, "weight_copies_rotated": ROTATE, "parallelism": "none"},
            "roofline": {"bound": "hbm", "kernel": "q8_0_gemv_kernel<1, false, 1, true, true, 1024>",
                         "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(),
                         "bytes_per_launch": step_bytes, "avg_launch_us": round(per["gemv_f32"] * 1e3, 3)},
            "steps_detail_us": {k2: round(v * 1e3, 3) for k2, v in per.items()},
            "two_launch_step": {"step_us": round(total2_ms / args.steps * 1e3, 3),
                                **{k2 + "_us": round(v * 1e3, 3) for k2, v in per2.items()},
                                "gemv_gbs": round(q8_0_bytes(m, k, n) / (per2["gemv"] * 1e-3) / 1e9, 1)},
        })
        del ws
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- decode / verify sweep
    if args.only in (None, "sweep"):
        sweep = {}
        shapes = workloads.GEMV_SWEEP_SHAPES
        if args.sweep_shapes:
            shapes = [tuple(int(v) for v in s.split("x")) for s in args.sweep_shapes.split(",")]
        for k, n in shapes:
            w0 = torch.from_numpy(workloads.q8_0_weights(n, k, rng)).to(dev)
            copies = max(3, -(-600_000_000 // w0.numel()))        # rotate >= 600 MB past the 256 MB cache
            ws = [w0] + [w0.clone() for _ in range(copies - 1)]
            for m in (1, 9):
                log(f"[bench] sweep m={m} {k}->{n}")
                x = torch.from_numpy(workloads.activations(m, k, rng)).to(dev)
                y = torch.empty((m, n), dtype=torch.float32, device=dev)
                xq = torch.empty((m, k), dtype=torch.int8, device=dev)
                xds = torch.empty((m, k // 32, 2), dtype=torch.float32, device=dev)
                byts = n * (k // 32) * 34 + m * k * 4 + m * n * 4
                row = {}
                if m <= 2 and m * k <= 8192:          # the one-launch step is for decode
                    fns = [("gemv_f32", lambda s: bqm.bqm_q8_0_gemv_f32(ws[s % copies], x, y))]
                    sl = f"Q8_0 sweep m={m} {k}->{n}, one launch"
                    timed_loop(torch, stream, args.warmup, fns, sl)
                    _, per = timed_loop(torch, stream, args.steps, fns, sl)
                    row["one_launch_us"] = round(per["gemv_f32"] * 1e3, 2)
                fns2 = [("quantize", lambda s: bqm.bqm_q8_1_quantize(x, xq, xds)),
                        ("gemv", lambda s: bqm.bqm_q8_0_gemv(ws[s % copies], xq, xds, y))]
                sl2 = f"Q8_0 sweep m={m} {k}->{n}, two launches"
                timed_loop(torch, stream, args.warmup, fns2, sl2)
                t2, per2 = timed_loop(torch, stream, args.steps, fns2, sl2)
                row["two_launch_step_us"] = round(t2 / args.steps * 1e3, 2)
                row["two_launch_gemv_us"] = round(per2["gemv"] * 1e3, 2)
                best = min(row.get("one_launch_us", 1e9), row["two_launch_step_us"])
                gbs = byts / (best * 1e-6) / 1e9
                row.update({"step_us": best, "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
                # the census convention (decode_kernel_census.rs, fn q8 and fn
                # report): weight bytes only, per GEMV launch, in TB/s and % of peak
                wbytes = n * (k // 32) * 34
                gemv_us = min(row.get("one_launch_us", 1e9), row["two_launch_gemv_us"])
                row.update({"gemv_us": gemv_us,
                            "weights_tbs": round(wbytes / (gemv_us * 1e-6) / 1e12, 3),
                            "weights_pct_peak": round(100 * wbytes / (gemv_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)})
                sweep[f"m{m} {k}->{n}"] = row
            del ws, w0
        torch.cuda.empty_cache()
        out["gemv_sweep"] = {"workload": "decode/verify sweep: q8_1 quantize + Q8_0 GEMV per step (the faster of "
                                         "the one-launch and two-launch paths), weights rotated past the cache",
                             **sweep}

    # ---------------------------------------------------------------- prefill MMQ
    if args.only in (None, "mmq"):
        mmq = {}
        m, k = 512, 4096
        x_host = workloads.activations(m, k, rng, outliers=True)
        x = torch.from_numpy(x_host).to(dev)
        xq = torch.empty((m, k), dtype=torch.int8, device=dev)
        xds = torch.empty((m, k // 32, 2), dtype=torch.float32, device=dev)
        for n in workloads.GEMM_NS:
            log(f"[bench] mmq n={n}")
            w0 = torch.from_numpy(workloads.q8_0_weights(n, k, rng)).to(dev)
            nc = copies_for(w0.numel())
            ws = [w0] + [w0.clone() for _ in range(nc - 1)]
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            fns = [("quantize", lambda s: bqm.bqm_q8_1_quantize(x, xq, xds)),
                   ("gemm", lambda s: bqm.bqm_q8_0_gemm(ws[s % nc], xq, xds, y))]
            ml = f"MMQ m={m} {k}->{n}"
            timed_loop(torch, stream, args.warmup, fns, ml)
            total_ms, per = timed_loop(torch, stream, args.steps, fns, ml)
            ops = 2.0 * m * n * k
            tops = ops / (per["gemm"] * 1e-3) / 1e12
            mmq[str(n)] = {"workload": f"MMQ GEMM m=512, K=4096, N={n}, Q8_0 x q8_1 (1% outliers x10)",
                           "gemm_us": round(per["gemm"] * 1e3, 2), "quantize_us": round(per["quantize"] * 1e3, 2),
                           "tops": round(tops, 1), "unit": "TOPS",
                           "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
                           "step_tops": round(ops / (total_ms / args.steps * 1e-3) / 1e12, 1)}
            del ws, w0, y
            torch.cuda.empty_cache()
        out["mmq_m512"] = mmq

    # ---------------------------------------------------------------- FP8 prefill
    if args.only in (None, "e4m3"):
        m, k, n = 512, 4096, 20480
        log("[bench] e4m3 n=20480")
        codes, w_scale = workloads.e4m3_weights(n, k, rng)
        w0 = torch.from_numpy(codes).to(dev)
        nc = copies_for(w0.numel())
        ws = [w0] + [w0.clone() for _ in range(nc - 1)]
        x = torch.from_numpy(workloads.activations(m, k, rng)).to(dev)
        xq8 = torch.empty((m, k), dtype=torch.uint8, device=dev)
        sc = torch.empty(4, dtype=torch.float32, device=dev)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        fns = [("quantize", lambda s: bqm.bqm_e4m3_quantize_amax(x, w_scale, xq8, sc)),
               ("gemm", lambda s: bqm.bqm_e4m3_gemm(ws[s % nc], xq8, sc, y))]
        el = f"e4m3 GEMM m={m} {k}->{n}"
        timed_loop(torch, stream, args.warmup, fns, el)
        total_ms, per = timed_loop(torch, stream, args.steps, fns, el)
        # the bounded kernel (fp16 matrix cores, within 1e-5 * sum|terms| for any data)
        fx = [("gemm_exact", lambda s: bqm.bqm_e4m3_gemm_exact(ws[s % nc], xq8, sc, y))]
        timed_loop(torch, stream, args.warmup, fx, el)
        _, perx = timed_loop(torch, stream, args.steps, fx, el)
        ops = 2.0 * m * n * k
        tf = ops / (per["gemm"] * 1e-3) / 1e12
        tfx = ops / (perx["gemm_exact"] * 1e-3) / 1e12
        out["e4m3_m512"] = {"workload": "FP8-E4M3 GEMM m=512, K=4096, N=20480, per-batch amax/448",
                            "gemm_us": round(per["gemm"] * 1e3, 2), "quantize_us": round(per["quantize"] * 1e3, 2),
                            "tflops": round(tf, 1), "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4),
                            "step_tflops": round(ops / (total_ms / args.steps * 1e-3) / 1e12, 1),
                            "bound_err_over_T": "7*2^-13 + (8k/64+1)*2^-24 (fp8 cores)",
                            "exact_gemm_us": round(perx["gemm_exact"] * 1e3, 2), "exact_tflops": round(tfx, 1),
                            "exact_frac_fp16_peak": round(tfx / FP16_PEAK_TFLOPS, 4),
                            "exact_bound_err_over_T": "(27 + k/128)*2^-24 (fp16 cores)"}
        del ws, w0, y
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- e4m3 decode GEMV
    if args.only in (None, "e4m3_gemv"):
        k, n = 4096, 64448
        log("[bench] e4m3 gemv n=64448")
        codes, w_scale = workloads.e4m3_weights(n, k, rng)
        w0 = torch.from_numpy(codes).to(dev)
        ws = [w0] + [w0.clone() for _ in range(ROTATE - 1)]
        e8 = {}
        for m in (1, 9):
            x = torch.from_numpy(workloads.activations(m, k, rng)).to(dev)
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            fns = [("gemv", lambda s: bqm.bqm_e4m3_gemv(ws[s % ROTATE], x, w_scale, y))]
            gl = f"e4m3 GEMV m={m} {k}->{n}"
            timed_loop(torch, stream, args.warmup, fns, gl)
            _, per = timed_loop(torch, stream, args.steps, fns, gl)
            byts = n * k + m * k * 4 + m * n * 4
            gbs = byts / (per["gemv"] * 1e-3) / 1e9
            e8[f"m{m}"] = {"workload": f"e4m3 decode GEMV m={m}, K=4096, N=64448, raw e4m3 weights, f32 activations",
                           "gemv_us": round(per["gemv"] * 1e3, 2), "gbs": round(gbs, 1),
                           "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        out["e4m3_gemv"] = e8
        del ws, w0
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- fp16 mirror prefill
    if args.only in (None, "f16"):
        m, k, n = 512, 4096, 20480
        log("[bench] f16 mirror n=20480")
        wq = torch.from_numpy(workloads.q8_0_weights(n, k, rng)).to(dev)
        nc = copies_for(2 * n * k)
        w16s = [torch.empty((n, k), dtype=torch.float16, device=dev) for _ in range(nc)]
        for w16 in w16s:
            bqm.bqm_q8_0_dequant_f16(wq, k, w16)
        x = torch.from_numpy(workloads.activations(m, k, rng, outliers=True)).to(dev)
        x16 = torch.empty((m, k), dtype=torch.float16, device=dev)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        fns = [("cvt", lambda s: bqm.bqm_f16_cvt(x, x16)),
               ("gemm", lambda s: bqm.bqm_f16_gemm(w16s[s % nc], x16, y))]
        fl = f"fp16 mirror m={m} {k}->{n}"
        timed_loop(torch, stream, args.warmup, fns, fl)
        total_ms, per = timed_loop(torch, stream, args.steps, fns, fl)
        dq = [("dequant", lambda s: bqm.bqm_q8_0_dequant_f16(wq, k, w16s[s % nc]))]
        timed_loop(torch, stream, 2, dq, fl)
        _, per_dq = timed_loop(torch, stream, args.steps, dq, fl)
        ops = 2.0 * m * n * k
        tf = ops / (per["gemm"] * 1e-3) / 1e12
        dq_bytes = q8_0_bytes(0, k, n) + 2 * n * k
        out["f16_mirror_m512"] = {
            "workload": "fp16 mirror prefill m=512, K=4096, N=20480: f32->fp16 cast + fp16 GEMM (f32 accumulate)",
            "gemm_us": round(per["gemm"] * 1e3, 2), "cvt_us": round(per["cvt"] * 1e3, 2),
            "tflops": round(tf, 1), "frac_fp16_peak": round(tf / FP16_PEAK_TFLOPS, 4),
            "step_tflops": round(ops / (total_ms / args.steps * 1e-3) / 1e12, 1),
            "dequant_us": round(per_dq["dequant"] * 1e3, 2),
            "dequant_gbs": round(dq_bytes / (per_dq["dequant"] * 1e-3) / 1e9, 1)}
        del w16s, wq, y
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- block-128 FP8 prefill
    if args.only in (None, "e4m3_blk"):
        m, k, n = 512, 4096, 20480
        log("[bench] e4m3 block-128 n=20480")
        codes, grid_h = workloads.e4m3_blk_weights(n, k, rng)
        w0 = torch.from_numpy(codes).to(dev)
        nc = copies_for(w0.numel())
        ws = [w0] + [w0.clone() for _ in range(nc - 1)]
        grid = torch.from_numpy(grid_h).to(dev)
        x = torch.from_numpy(workloads.activations(m, k, rng, outliers=True)).to(dev)
        xq8 = torch.empty((m, k), dtype=torch.uint8, device=dev)
        xs = torch.empty((m, k // 128), dtype=torch.float32, device=dev)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        fns = [("quantize", lambda s: bqm.bqm_e4m3_blk_quantize(x, xq8, xs)),
               ("gemm", lambda s: bqm.bqm_e4m3_blk_gemm(ws[s % nc], grid, xq8, xs, y))]
        bl = f"block-128 FP8 m={m} {k}->{n}"
        timed_loop(torch, stream, args.warmup, fns, bl)
        total_ms, per = timed_loop(torch, stream, args.steps, fns, bl)
        cnt = torch.empty(1, dtype=torch.int64, device=dev)
        scan = [("nan_scan", lambda s: bqm.bqm_e4m3_nan_count(ws[s % nc], cnt))]
        timed_loop(torch, stream, 2, scan, bl)
        _, per_scan = timed_loop(torch, stream, args.steps, scan, bl)
        ops = 2.0 * m * n * k
        tf = ops / (per["gemm"] * 1e-3) / 1e12
        out["e4m3_blk_m512"] = {
            "workload": "block-128 FP8 GEMM m=512, K=4096, N=20480: per-(token, 128-k) e4m3 activations, "
                        "per-128x128 f32 weight grid, one fold per 128-k block",
            "gemm_us": round(per["gemm"] * 1e3, 2), "quantize_us": round(per["quantize"] * 1e3, 2),
            "tflops": round(tf, 1), "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4),
            "step_tflops": round(ops / (total_ms / args.steps * 1e-3) / 1e12, 1),
            "nan_scan_us": round(per_scan["nan_scan"] * 1e3, 2),
            "nan_scan_gbs": round(n * k / (per_scan["nan_scan"] * 1e-3) / 1e9, 1),
            "nan_codes": int(cnt.item())}
        del ws, w0, y
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- accumulator instrument
    if args.only in (None, "accprobe"):
        m, reps, batch = 512, 9, 10
        probe = {}
        sheets = {"27b": ACCPROBE_LABELS_27B, "1p7b": ACCPROBE_LABELS_1P7B}
        for sheet, shapes in sheets.items():
            probe[sheet] = {}
            for dist in ("wide", "mid"):
                cells, ln_sum = {}, 0.0
                for k, n, label in shapes:
                    log(f"[bench] accprobe {sheet} {dist} {label} {k}->{n}")
                    w = torch.from_numpy(workloads.accprobe_weights(n, k, rng, dist)).to(dev)
                    xq_h, xds_h = workloads.accprobe_activations(m, k, rng, dist)
                    xq = torch.from_numpy(xq_h).to(dev)
                    xds = torch.from_numpy(xds_h).to(dev)
                    y = torch.empty((m, n), dtype=torch.float32, device=dev)
                    arms = {"f32": lambda: bqm.bqm_q8_0_gemm_f8acc(w, xq, xds, y),
                            "s32": lambda: bqm.bqm_q8_0_gemm(w, xq, xds, y)}
                    for fn in arms.values():
                        for _ in range(3):
                            fn()
                    t = {"f32": [], "s32": []}
                    for _ in range(reps):
                        for arm in ("f32", "s32"):           # interleaved inside each rep
                            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                            with region(torch, f"instrument {sheet} {dist} m={m} {k}->{n}: {arm}"):
                                e0.record(stream)
                                for _ in range(batch):
                                    arms[arm]()
                                e1.record(stream)
                                e1.synchronize()
                            t[arm].append(e0.elapsed_time(e1) / batch)
                    a, b = sorted(t["f32"])[reps // 2], sorted(t["s32"])[reps // 2]
                    ratio = a / b
                    flop = 2.0 * m * k * n
                    cells[f"{label} {k}->{n}"] = {"f32acc_us": round(a * 1e3, 2), "s32acc_us": round(b * 1e3, 2),
                                                  "ratio": round(ratio, 4), "delta_pp": round(100 * (ratio - 1), 1),
                                                  "f32_tflop": round(flop / (a * 1e-3) / 1e12, 1),
                                                  "s32_tflop": round(flop / (b * 1e-3) / 1e12, 1)}
                    ln_sum += np.log(ratio)
                    del w, xq, xds, y
                geo = float(np.exp(ln_sum / len(cells)))
                probe[sheet][dist] = {"shapes": cells, "geomean_ratio": round(geo, 4),
                                      "delta_pp": round(100 * (geo - 1), 1)}
        torch.cuda.empty_cache()
        out["accprobe_m512"] = {"workload": "accumulator instrument, m=512, the 27B and 1.7B projection sheets: the "
                                            "MMQ with int8 MFMA + s32 block sums (s32) vs fp8 MFMA + f32 block sums "
                                            "(f32), same tiles and fold count; medians of 9 interleaved reps of 10 "
                                            "launches, geomean of the ratio per sheet and byte distribution",
                                **probe}

    # ---------------------------------------------------------------- CPU oracle baseline
    if not args.no_cpu and args.only is None:
        log("[bench] cpu oracle baseline (host threads)")
        multi = cpu_oracle_legs(single=False)
        log("[bench] cpu oracle baseline (one thread, child process)")
        single = cpu_single_thread_child()
        head = multi["decode_head_step"]
        out["cpu_baseline"] = {
            "value": head["value"], "unit": "GB/s", "cores": multi["threads"], "kind": "oracle",
            "sample": head["sample"],
            "single_thread_value": (single or {}).get("decode_head_step", {}).get("value"),
            "host": host_description(multi["threads"]),
            "configs": {k2: v for k2, v in multi.items() if k2 != "threads"},
            "single_thread": {k2: v for k2, v in (single or {}).items() if k2 != "threads"} or None,
        }

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
