#!/usr/bin/env python
"""Benchmark of the tiled block-32 quantized matmul hot path on one MI355X.

Step (the decode hot path, one token): dynamic int8 quantization of the
activation row, then the tiled GEMV over the repacked weights -- on the
Q8_0 K=4096 N=4096 M=1 workload (fp16 scales |N(0,1)|*0.01, int8 codes
uniform in [-127, 127], fp32 activations N(0,1), seed 0).  The weights are
repacked on the GPU once, at load (as the pages place repacking), into R
distinct copies (R * 17.8 MB >= 1 GiB) that the steps rotate through, so
every step streams its weights from HBM rather than from the 256 MB
Infinity Cache.  All inputs are resident in HBM before the timed region;
the K timed steps are replayed from a HIP graph.

Printed: one JSON line.  value = weight-tile bytes per step / step time
(GB/s).  roofline = the GEMV kernel alone: algorithmic bytes (weight tiles
+ int8 activations + fp16 activation scales + fp32 outputs) per launch over
its average duration: launches replayed back to back from a HIP graph on the
current stream, bracketed by HIP events recorded on that stream.
Also reported: the int8-MFMA GEMM on the IQ4_NL M=512 K=N=4096 workload
(TOPS and fraction of the int8 peak), the load-time repack, and the CPU
oracle timed on this host's cores.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA
ROTATE_BYTES = 1 << 30         # defeat the 256 MB Infinity Cache


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="bounded CPU work for the oracle baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the GEMM and repack measurements")
    p.add_argument("--eager", action="store_true", help="time eager launches, not a graph")
    return p.parse_args()


def gemv_bytes(w):
    """Algorithmic bytes of one qgemv launch: tiles + q + d + y."""
    nkt = w.K // 32
    return w.weight_bytes + w.M * w.K + w.M * nkt * 2 + w.M * w.N * 4


def capture(torch, fn, n):
    """A HIP graph of fn(0) .. fn(n-1), captured on a side stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(n):
                fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g.replay()                             # untimed replay: first-launch costs
    torch.cuda.synchronize()
    return g


def kernel_us(torch, fn, n=200):
    """Average duration of the kernel that fn(i) launches: n launches replayed
    back to back from a HIP graph, timed by HIP events recorded on the stream
    the kernels run on (the current stream, which replays the graph)."""
    g = capture(torch, fn, n)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n * 1e3


def measure_gemv(torch, tq, synth, args):
    import numpy as np
    w = synth.WORKLOADS["q8_0_gemv_k4096_n4096_m1"]
    inp = synth.make_inputs(w)
    flat = torch.from_numpy(inp.flat).cuda()
    R = max(2, -(-ROTATE_BYTES // w.weight_bytes))
    tiles = [tq.repack_tiles(w.qtype, flat, w.K, w.N) for _ in range(R)]
    del flat
    X = 64
    rng = np.random.default_rng(1)
    xs = torch.from_numpy(np.concatenate(
        [inp.x, rng.standard_normal((X - 1, w.K), dtype=np.float32)])).cuda()
    q = torch.empty((w.M, w.K), dtype=torch.int8, device="cuda")
    d = torch.empty((w.M, w.K // 32), dtype=torch.float16, device="cuda")
    y = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")

    def step(i):
        tq.quantize_act(xs[i % X: i % X + 1], q=q, d=d)
        tq.qgemv(w.qtype, tiles[i % R], w.K, w.N, q, d, out=y)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    if args.eager:
        run = lambda: [step(i) for i in range(K)]
    else:
        run = capture(torch, step, K).replay

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0

    gemv_us = kernel_us(torch, lambda i: tq.qgemv(w.qtype, tiles[i % R], w.K, w.N, q, d, out=y))
    quant_us = kernel_us(torch, lambda i: tq.quantize_act(xs[i % X: i % X + 1], q=q, d=d))
    return w, R, dt, gemv_us, quant_us


def measure_gemm(torch, tq, synth, n=200):
    import numpy as np
    w = synth.WORKLOADS["iq4_nl_gemm_m512_k4096_n4096"]
    inp = synth.make_inputs(w)
    flat = torch.from_numpy(inp.flat).cuda()
    R = max(2, -(-ROTATE_BYTES // w.weight_bytes))
    tiles = [tq.repack_tiles(w.qtype, flat, w.K, w.N) for _ in range(R)]
    x = torch.from_numpy(inp.x.view(np.int16)).cuda().view(torch.bfloat16)
    q, d = tq.quantize_act(x)
    y = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    f = lambda i: tq.qgemm(w.qtype, tiles[i % R], w.K, w.N, q, d, lut=inp.lut, out=y)
    for i in range(20):
        f(i)
    us = kernel_us(torch, f, n)
    quant_us = kernel_us(torch, lambda i: tq.quantize_act(x, q=q, d=d), 50)
    tops = 2.0 * w.M * w.N * w.K / us / 1e6
    return {"workload": w.name, "metric": "qgemm int8 TOPS", "value": round(tops, 2),
            "unit": "TOPS", "kernel_us": round(us, 3), "quantize_act_us": round(quant_us, 3),
            "roofline": {"bound": "mfma", "achieved": round(tops, 2), "peak": INT8_PEAK_TOPS,
                         "unit": "TOP/s", "frac": round(tops / INT8_PEAK_TOPS, 4),
                         "traffic": None}}


def measure_repack(torch, tq, synth, n=50):
    w = synth.WORKLOADS["q4_0_gemv_k4096_n14336_m1"]
    inp = synth.make_inputs(w)
    fb = inp.flat.size
    R = max(2, -(-ROTATE_BYTES // fb))
    flats = [torch.from_numpy(inp.flat).cuda() for _ in range(min(R, 32))]
    out = torch.empty(w.weight_bytes, dtype=torch.uint8, device="cuda")
    f = lambda i: tq.repack_tiles(w.qtype, flats[i % len(flats)], w.K, w.N, out=out)
    for i in range(5):
        f(i)
    us = kernel_us(torch, f, n)
    gbs = (fb + w.weight_bytes) / us / 1e3
    return {"workload": "repack " + w.name, "kernel_us": round(us, 3), "GB_s": round(gbs, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": None}}


def cpu_baseline(synth, w, seconds):
    """The oracle as it stands (single-threaded C), timed on this host."""
    import oracle
    inp = synth.make_inputs(w)
    tiles = oracle.repack(w.qtype, inp.flat, w.K, w.N)
    n = 0
    t0 = time.perf_counter()
    while True:
        q, d = oracle.quantize_act(inp.x)
        oracle.matmul(w.qtype, tiles, w.K, w.N, q, d)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(w.weight_bytes * n / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n} full steps (quantize_act + fp64 matmul) of {w.name} in {dt:.1f} s, "
                      "1 thread"}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures a single GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import block_quantized_matmul_repack_amd as tq
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    tq.lib()

    w, R, dt, gemv_us, quant_us = measure_gemv(torch, tq, synth, args)
    K = args.steps
    ms = dt / K * 1e3
    value = w.weight_bytes / (dt / K) / 1e9
    achieved = gemv_bytes(w) / gemv_us / 1e3
    line = {
        "metric": "qgemv weight-stream GB/s (% of HBM peak); qgemm int8 TOPS (% MFMA peak)",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": w.name, "qtype": "q8_0", "K": w.K, "N": w.N, "M": w.M,
                   "step": "quantize_act + qgemv", "weight_copies": R,
                   "launch": "eager" if args.eager else "hip graph",
                   "hbm_frac_of_value": round(value / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None,
                     "kernel": "qgemv", "kernel_us": round(gemv_us, 3),
                     "bytes_per_launch": gemv_bytes(w)},
        "quantize_act_us": round(quant_us, 3),
    }
    if not args.no_extra:
        line["qgemm"] = measure_gemm(torch, tq, synth)
        line["repack"] = measure_repack(torch, tq, synth)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(synth, w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
