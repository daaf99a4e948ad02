#!/usr/bin/env python
"""Benchmark of the tiled block-32 quantized matmul hot path on one MI355X.

Step (the decode hot path, one token): dynamic int8 quantization of the
activation row and the tiled GEMV over the repacked weights, fused in one
launch (tq_qgemv_x; the two-launch form is timed as well) -- on the
Q8_0 K=4096 N=4096 M=1 workload (fp16 scales |N(0,1)|*0.01, int8 codes
uniform in [-127, 127], fp32 activations N(0,1), seed 0).  The weights are
repacked on the GPU once, at load (as the pages place repacking), into R
distinct copies (R * 17.8 MB >= 1 GiB) that the steps rotate through, so
every step streams its weights from HBM rather than from the 256 MB
Infinity Cache.  All inputs are resident in HBM before the timed region;
the K timed steps are replayed from a HIP graph.

Printed: one JSON line.  value = weight-tile bytes per step / step time
(GB/s).  roofline = the fused decode kernel: algorithmic bytes (weight tiles
+ fp32 activations + fp32 outputs) per launch over
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
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA (fp8 x fp4 issues at the fp8 rate)
ROTATE_BYTES = 1 << 30         # defeat the 256 MB Infinity Cache

# HBM traffic of the kernels, from rocprofv3 --pmc passes (FETCH_SIZE, then
# WRITE_SIZE, each in its own run) of `bench.py --launch-only <kernel>`: KiB
# per dispatch as the counters read them, averaged over the dispatches.  The
# same counters read for a plain 256 MiB device copy (`--launch-only copy`)
# give FETCH_SIZE 131083.55 KiB and WRITE_SIZE 262144 KiB for 262144 KiB moved
# each way, so FETCH_SIZE is scaled by 262144 / 131084.5 and WRITE_SIZE by 1.
# "src" is the SHA-256 of the kernel's sources when the counters were taken;
# once they differ, traffic is reported as null.
FETCH_SCALE = 262144.0 / 131083.55
WRITE_SCALE = 1.0
TRAFFIC = {
    "decode": {"fetch_kib": 8780.32, "write_kib": 112.00,
               "src": "2beef0cbad9cd442180bffefa0041c71debc773f13101dc1652c52ec158bfbb4"},
    "gemm": {"fetch_kib": 13363.18, "write_kib": 8192.00,
             "src": "cf4e64f80418ffcf75536c463148f42c21f551048dbe477e30a9d190bff3956d"},
    "repack": {"fetch_kib": 16143.90, "write_kib": 32256.00,
               "src": "7f60c5b9af92b655461bb894d3e2454e839c4b6ff51fe0636c10b7976b2b5183"},
    "mx": {"fetch_kib": 12871.09, "write_kib": 8192.00,
           "src": "e0375ab973c733c2d3825ab444b6d9baf635ebe937af40029474141d9138b660"},
}
KERNEL_SOURCES = {
    "decode": ("qgemv.hip", "tq_internal.h"),
    "gemm": ("qgemm.hip", "tq_internal.h"),
    "repack": ("repack.hip", "tq_internal.h"),
    "mx": ("mx.hip", "tq_internal.h"),
}
LAUNCH_ONLY = ("decode", "gemm", "repack", "mx", "copy")


def source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "block_quantized_matmul_repack_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_bytes(kernel):
    """Counter-measured HBM bytes per launch, or None if the kernel's sources
    changed since the counters were taken (or none were taken)."""
    t = TRAFFIC.get(kernel)
    if t is None or t["src"] != source_hash(kernel):
        return None
    return int(round(1024 * (t["fetch_kib"] * FETCH_SCALE + t["write_kib"] * WRITE_SCALE)))


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
    p.add_argument("--launch-only", choices=sorted(LAUNCH_ONLY), default=None,
                   help="no timing: launch one kernel --steps times on the bench's inputs "
                        "(for rocprofv3 --pmc counter passes) and exit")
    return p.parse_args()


def gemv_x_bytes(w):
    """Algorithmic bytes of one fused decode launch: tiles + fp32 x + fp32 y."""
    return w.weight_bytes + 4 * w.M * w.K + 4 * w.M * w.N


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


def setup_decode(torch, tq, synth):
    """Decode-step inputs in HBM; returns (workload, copies, step, step2, parts)."""
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

    def step(i):                 # one decode token: quantize + GEMV in one launch
        tq.qgemv_x(w.qtype, tiles[i % R], w.K, w.N, xs[i % X: i % X + 1], out=y)

    def step2(i):                # the same with the quantization as its own launch
        tq.quantize_act(xs[i % X: i % X + 1], q=q, d=d)
        tq.qgemv(w.qtype, tiles[i % R], w.K, w.N, q, d, out=y)

    # the weight copies viewed as fp32 rows of 1024: a plain row-sum reads
    # exactly the step's tile bytes (one reduction block per row, no
    # cross-block scratch)
    rows = [t.view(torch.float32).view(-1, 1024) for t in tiles]
    rsum = torch.empty(rows[0].shape[0], dtype=torch.float32, device="cuda")
    parts = {
        "qgemv": lambda i: tq.qgemv(w.qtype, tiles[i % R], w.K, w.N, q, d, out=y),
        "quantize_act": lambda i: tq.quantize_act(xs[i % X: i % X + 1], q=q, d=d),
        # one weight copy: resident in the 256 MB Infinity Cache after the first step
        "warm": lambda i: tq.qgemv_x(w.qtype, tiles[0], w.K, w.N, xs[i % X: i % X + 1], out=y),
        "read": lambda i: torch.sum(rows[i % R], dim=1, out=rsum),
    }
    return w, R, step, step2, parts


def measure_gemv(torch, tq, synth, args):
    w, R, step, step2, parts = setup_decode(torch, tq, synth)
    for i in range(args.warmup):
        step(i)
        step2(i)
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

    two = capture(torch, step2, 500)
    t1 = time.perf_counter()
    two.replay()
    torch.cuda.synchronize()
    two_us = (time.perf_counter() - t1) / 500 * 1e6

    detail = {
        "qgemv_x_us": kernel_us(torch, step),
        "qgemv_us": kernel_us(torch, parts["qgemv"]),
        "quantize_act_us": kernel_us(torch, parts["quantize_act"]),
        "two_launch_step_us": two_us,
    }
    # references at this size: an (almost) empty launch, and a plain device
    # copy of the same number of bytes (read + write), both graph-replayed
    tiny = torch.zeros(1, device="cuda")
    detail["empty_launch_us"] = kernel_us(torch, lambda i: tiny.add_(1.0))
    src = [torch.ones(w.weight_bytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
    dst = torch.empty_like(src[0])
    cu = kernel_us(torch, lambda i: dst.copy_(src[i % R]))
    del src
    detail["copy_same_bytes_us"] = cu
    detail["copy_same_bytes_GB_s"] = 2 * w.weight_bytes / cu / 1e3

    # per launch: 200 eager launches of the step with a HIP event pair around
    # each, enqueued while the stream is still busy with in-place passes over a
    # 256 MiB buffer, so that the launches run back to back on the GPU and each
    # pair times its kernel rather than the host's launch latency
    pad = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(200)]
    ahead = torch.cuda.Event()
    for passes in (100, 400, 1600):
        for _ in range(passes):
            pad.mul_(1.0)
        ahead.record()
        for i, (e0, e1) in enumerate(evs):
            e0.record()
            step(i)
            e1.record()
        queued = not ahead.query()
        torch.cuda.synchronize()
        if queued:
            break
    del pad
    t = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
    ref = {"per_launch_us": {"median": round(t[100], 3), "p10": round(t[20], 3),
                             "p90": round(t[180], 3), "launches": 200,
                             "queued_behind_busy_stream": queued,
                             "how": "eager launches, a HIP event pair around each"}}
    wu = kernel_us(torch, parts["warm"])
    ref["warm_mall_resident"] = {"us": round(wu, 3), "GB_s": round(w.weight_bytes / wu / 1e3, 1),
                                 "note": "one weight copy, served from the Infinity Cache; "
                                         "not an HBM figure"}
    ru = kernel_us(torch, parts["read"])
    ref["read_same_bytes"] = {"us": round(ru, 3), "GB_s": round(w.weight_bytes / ru / 1e3, 1),
                              "note": "torch row-sum over the same rotating tile copies: "
                                      "what merely reading these bytes costs at this size"}
    return w, R, dt, detail, ref


def setup_gemm(torch, tq, synth):
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
    quant = lambda i: tq.quantize_act(x, q=q, d=d)
    return w, f, quant


def gemm_bytes(w):
    """Algorithmic bytes of one GEMM launch: tiles + int8 q + fp16 d + fp32 y."""
    return w.weight_bytes + w.M * w.K + 2 * w.M * (w.K // 32) + 4 * w.M * w.N


def measure_gemm(torch, tq, synth, n=200):
    w, f, quant = setup_gemm(torch, tq, synth)
    for i in range(20):
        f(i)
    us = kernel_us(torch, f, n)
    quant_us = kernel_us(torch, quant, 50)
    tops = 2.0 * w.M * w.N * w.K / us / 1e6
    tb = traffic_bytes("gemm")
    return {"workload": w.name, "metric": "qgemm int8 TOPS", "value": round(tops, 2),
            "unit": "TOPS", "kernel_us": round(us, 3), "quantize_act_us": round(quant_us, 3),
            "hbm_GB_s": round(gemm_bytes(w) / us / 1e3, 1),
            "roofline": {"bound": "mfma", "achieved": round(tops, 2), "peak": INT8_PEAK_TOPS,
                         "unit": "TOP/s", "frac": round(tops / INT8_PEAK_TOPS, 4),
                         "traffic": tb, "bytes_per_launch": gemm_bytes(w)}}


def setup_mx(torch, tq, synth):
    """MXFP4 M=512 K=N=4096 on the block-scaled matrix cores (MXFP8
    activations from bf16, like the int8 GEMM workload's)."""
    import numpy as np
    w = synth.WORKLOADS["mxfp4_gemm_m512_k4096_n4096"]
    inp = synth.make_inputs(w)
    flat = torch.from_numpy(inp.flat).cuda()
    R = max(2, -(-ROTATE_BYTES // w.weight_bytes))
    tiles = [tq.repack_tiles(w.qtype, flat, w.K, w.N) for _ in range(R)]
    x = torch.from_numpy(inp.x.view(np.int16)).cuda().view(torch.bfloat16)
    q, e = tq.quantize_act_mx(x)
    y = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    f = lambda i: tq.qgemm_mx(tiles[i % R], w.K, w.N, q, e, out=y)
    quant = lambda i: tq.quantize_act_mx(x, q=q, e=e)
    q8, d8 = tq.quantize_act(x)
    f8 = lambda i: tq.qgemm(w.qtype, tiles[i % R], w.K, w.N, q8, d8, out=y)
    return w, f, quant, f8


def measure_mx(torch, tq, synth, n=200):
    w, f, quant, f8 = setup_mx(torch, tq, synth)
    for i in range(20):
        f(i)
        f8(i)
    us = kernel_us(torch, f, n)
    quant_us = kernel_us(torch, quant, 50)
    us8 = kernel_us(torch, f8, n)
    tflops = 2.0 * w.M * w.N * w.K / us / 1e6
    nbytes = w.weight_bytes + w.M * w.K + w.M * (w.K // 32) + 4 * w.M * w.N
    return {"workload": w.name + " (MXFP8 activations, block-scaled MFMA)",
            "metric": "qgemm_mx fp8 x fp4 TFLOP/s", "value": round(tflops, 2), "unit": "TFLOP/s",
            "kernel_us": round(us, 3), "quantize_act_mx_us": round(quant_us, 3),
            "int8_path_same_tiles_us": round(us8, 3),
            "hbm_GB_s": round(nbytes / us / 1e3, 1),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": FP8_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / FP8_PEAK_TFLOPS, 4),
                         "traffic": traffic_bytes("mx"), "bytes_per_launch": nbytes}}


def setup_repack(torch, tq, synth):
    w = synth.WORKLOADS["q4_0_gemv_k4096_n14336_m1"]
    inp = synth.make_inputs(w)
    fb = inp.flat.size
    R = max(2, -(-ROTATE_BYTES // fb))
    flats = [torch.from_numpy(inp.flat).cuda() for _ in range(min(R, 32))]
    out = torch.empty(w.weight_bytes, dtype=torch.uint8, device="cuda")
    f = lambda i: tq.repack_tiles(w.qtype, flats[i % len(flats)], w.K, w.N, out=out)
    return w, f, fb


def measure_repack(torch, tq, synth, n=50):
    w, f, fb = setup_repack(torch, tq, synth)
    for i in range(5):
        f(i)
    us = kernel_us(torch, f, n)
    gbs = (fb + w.weight_bytes) / us / 1e3
    return {"workload": "repack " + w.name, "kernel_us": round(us, 3), "GB_s": round(gbs, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": traffic_bytes("repack"),
                         "bytes_per_launch": fb + w.weight_bytes}}


def measure_others(torch, tq, synth):
    """The other decode / prefill workloads, timed like the roofline kernel
    (graph of 50 steps, HIP events); weights rotate over >= 1 GiB.  Decode
    steps are timed both fused (qgemv_x) and as quantize_act + qgemv; GB/s
    counts tiles + fp32 x + fp32 y over the faster one."""
    import numpy as np
    res = {}
    cases = [("q4_0_gemv_k4096_n14336_m1", 1), ("q4_0_gemv_k4096_n14336_m1", 4),
             ("q4_0_gemv_k4096_n14336_m1", 8), ("q8_0_lmhead_k4096_n128001_m1", 1),
             ("q8_0_lmhead_k4096_n128001_m128", 128), ("mxfp4_gemv_k4096_n14336_m1", 1),
             ("mxfp4_gemv_k4096_n14336_m1", 4), ("mxfp4_gemm_m512_k4096_n4096", 512),
             ("q4_1_gemv_k4096_n14336_m1", 1), ("q4_1_gemv_k4096_n14336_m1", 4),
             ("q4_1_gemm_m512_k4096_n4096", 512), ("q4_k_gemv_k4096_n14336_m1", 1)]
    tiles_cache = {}
    for name, M in cases:
        w = synth.WORKLOADS[name]
        key = (w.qtype, w.K, w.N)
        if key not in tiles_cache:
            inp = synth.make_inputs(w, M=1)
            flat = torch.from_numpy(inp.flat).cuda()
            R = max(2, -(-ROTATE_BYTES // w.weight_bytes))
            tiles_cache.clear()
            tiles_cache[key] = [tq.repack_tiles(w.qtype, flat, w.K, w.N) for _ in range(R)]
            del flat
        tiles = tiles_cache[key]
        R = len(tiles)
        rng = np.random.default_rng(M)
        x = torch.from_numpy(rng.standard_normal((M, w.K), dtype=np.float32)).cuda()
        if M <= 8:
            q = torch.empty((M, w.K), dtype=torch.int8, device="cuda")
            d = torch.empty((M, w.K // 32), dtype=torch.float16, device="cuda")
            y = torch.empty((M, w.N), dtype=torch.float32, device="cuda")
            fused = lambda i: tq.qgemv_x(w.qtype, tiles[i % R], w.K, w.N, x, out=y)

            def two(i):
                tq.quantize_act(x, q=q, d=d)
                tq.qgemv(w.qtype, tiles[i % R], w.K, w.N, q, d, out=y)
            label = f"{name.rsplit('_m', 1)[0]}_m{M}"
            nbytes = w.weight_bytes + 4 * M * w.K + 4 * M * w.N
            for i in range(5):
                fused(i)
                two(i)
            us_f = kernel_us(torch, fused, 50)
            us_2 = kernel_us(torch, two, 50)
            us = min(us_f, us_2)
            res[label] = {"step_us": round(us, 3),
                          "path": "qgemv_x (fused)" if us_f <= us_2 else "quantize_act + qgemv",
                          "qgemv_x_us": round(us_f, 3), "quantize_act_qgemv_us": round(us_2, 3),
                          "GB_s": round(nbytes / us / 1e3, 1),
                          "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
        else:
            q, d = tq.quantize_act(x)
            f = lambda i: tq.qgemm(w.qtype, tiles[i % R], w.K, w.N, q, d)
            nbytes = w.weight_bytes + M * w.K + 2 * M * (w.K // 32) + 4 * M * w.N
            for i in range(5):
                f(i)
            us = kernel_us(torch, f, 50)
            res[f"{name} qgemm"] = {"kernel_us": round(us, 3), "GB_s": round(nbytes / us / 1e3, 1),
                                    "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                                    "TOPS": round(2.0 * M * w.N * w.K / us / 1e6, 2)}
    tiles_cache.clear()
    # repack of every type at the FFN shape (flat copies rotate over >= 1 GiB)
    for qtype in (synth.Q8_0, synth.IQ4_NL, synth.MXFP4, synth.Q4_1, synth.Q4_K):
        w = synth.Workload("repack", qtype, 4096, 14336, 1,
                           {synth.Q8_0: "absnormal", synth.MXFP4: "e8m0", synth.Q4_1: "minmax",
                            synth.Q4_K: "q4k"}.get(qtype, "uniform"))
        inp = synth.make_inputs(w)
        fb = inp.flat.size
        flats = [torch.from_numpy(inp.flat).cuda() for _ in range(min(32, max(2, -(-ROTATE_BYTES // fb))))]
        out = torch.empty(w.weight_bytes, dtype=torch.uint8, device="cuda")
        f = lambda i: tq.repack_tiles(qtype, flats[i % len(flats)], w.K, w.N, out=out)
        for i in range(3):
            f(i)
        us = kernel_us(torch, f, 30)
        gbs = (fb + w.weight_bytes) / us / 1e3
        res[f"repack {synth.TYPE_NAMES[qtype]}_k4096_n14336"] = {
            "kernel_us": round(us, 3), "GB_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        del flats, out
    # flat (un-repacked) weights beside the tiled ones, and the device unpack
    for name, M in (("q4_0_gemv_k4096_n14336_m1", 1), ("q4_0_gemv_k4096_n14336_m1", 8),
                    ("q8_0_gemv_k4096_n4096_m1", 1), ("iq4_nl_gemm_m512_k4096_n4096", 512)):
        w = synth.WORKLOADS[name]
        inp = synth.make_inputs(w, M=1)
        fb = inp.flat.size
        R = min(32, max(2, -(-ROTATE_BYTES // fb)))
        flats = [torch.from_numpy(inp.flat).cuda() for _ in range(R)]
        tiles = [tq.repack_tiles(w.qtype, f, w.K, w.N) for f in flats]
        rng = np.random.default_rng(M)
        x = torch.from_numpy(rng.standard_normal((M, w.K), dtype=np.float32)).cuda()
        q, d = tq.quantize_act(x)
        y = torch.empty((M, w.N), dtype=torch.float32, device="cuda")
        lut = inp.lut
        if M <= 8:
            ft = lambda i: tq.qgemv(w.qtype, tiles[i % R], w.K, w.N, q, d, lut=lut, out=y)
            ff = lambda i: tq.qgemv_flat(w.qtype, flats[i % R], w.K, w.N, q, d, lut=lut, out=y)
        else:
            ft = lambda i: tq.qgemm(w.qtype, tiles[i % R], w.K, w.N, q, d, lut=lut, out=y)
            ff = lambda i: tq.qgemm_flat(w.qtype, flats[i % R], w.K, w.N, q, d, lut=lut, out=y)
        for i in range(3):
            ft(i)
            ff(i)
        ut, uf = kernel_us(torch, ft, 30), kernel_us(torch, ff, 30)
        label = f"flat {name.rsplit('_m', 1)[0]}_m{M}"
        res[label] = {"flat_us": round(uf, 3), "tiled_us": round(ut, 3),
                      "flat_GB_s_of_weights": round(fb / uf / 1e3, 1)}
        if M > 8:
            res[label]["flat_TOPS"] = round(2.0 * M * w.N * w.K / uf / 1e6, 2)
        if name.startswith("q4_0"):
            out = torch.empty(fb, dtype=torch.uint8, device="cuda")
            fu = lambda i: tq.unpack_tiles(w.qtype, tiles[i % R], w.K, w.N, out=out)
            fu(0)
            uu = kernel_us(torch, fu, 30)
            res[f"unpack {name.rsplit('_m', 1)[0]}"] = {
                "kernel_us": round(uu, 3), "GB_s": round((fb + w.weight_bytes) / uu / 1e3, 1)}
        del flats, tiles
    # small-M products through tq_matmul (one decode pass per 8 rows where
    # estimated no slower) beside the GEMM on the same tiles
    w = synth.WORKLOADS["q8_0_gemv_k4096_n4096_m1"]
    for qtype in (synth.Q4_0, synth.IQ4_NL):
        wq = synth.Workload("small_m", qtype, w.K, w.N, 1, "uniform")
        inp = synth.make_inputs(wq)
        flat = torch.from_numpy(inp.flat).cuda()
        R = max(2, -(-ROTATE_BYTES // wq.weight_bytes))
        tiles = [tq.repack_tiles(qtype, flat, w.K, w.N) for _ in range(R)]
        del flat
        for M in (16, 32):
            rng = np.random.default_rng(M)
            x = torch.from_numpy(rng.standard_normal((M, w.K), dtype=np.float32)).cuda()
            q, d = tq.quantize_act(x)
            y = torch.empty((M, w.N), dtype=torch.float32, device="cuda")
            fm = lambda i: tq.matmul(qtype, tiles[i % R], w.K, w.N, q, d, lut=inp.lut, out=y)
            fg = lambda i: tq.qgemm(qtype, tiles[i % R], w.K, w.N, q, d, lut=inp.lut, out=y)
            for i in range(3):
                fm(i)
                fg(i)
            um, ug = kernel_us(torch, fm, 30), kernel_us(torch, fg, 30)
            path = "decode passes" if tq.matmul_path(qtype, w.K, w.N, M) == tq.PATH_GEMV else "qgemm"
            res[f"{synth.TYPE_NAMES[qtype]}_matmul_k4096_n4096_m{M}"] = {
                "matmul_us": round(um, 3), "path": path, "qgemm_us": round(ug, 3)}
        del tiles
    return res


def launch_only(torch, tq, synth, kernel, n):
    """Launch one kernel n times, eagerly, untimed (counter collection)."""
    if kernel == "decode":
        f = setup_decode(torch, tq, synth)[2]
    elif kernel == "gemm":
        f = setup_gemm(torch, tq, synth)[1]
    elif kernel == "repack":
        f = setup_repack(torch, tq, synth)[1]
    elif kernel == "mx":
        f = setup_mx(torch, tq, synth)[1]
    else:                                   # calibration: a plain 256 MiB copy
        a = torch.ones(1 << 28, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        f = lambda i: b.copy_(a)
    for i in range(n):
        f(i)
    torch.cuda.synchronize()
    print(f"launched {kernel} x{n}", flush=True)


def device_info(torch):
    import subprocess
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", ""),
            "compute_units": p.multi_processor_count,
            "memory_GiB": round(p.total_memory / 2**30, 1)}
    # current clocks as rocm-smi reports them (a child process; None if unavailable)
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                           text=True, timeout=30)
        clk = json.loads(r.stdout)
        card = clk.get("card0") or next(iter(clk.values()))
        info["clocks"] = {k: v for k, v in card.items() if "clk" in k.lower() or "clock" in k.lower()}
    except Exception:
        info["clocks"] = None
    return info


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


def host_info():
    """The host CPU the oracle baseline ran on: model name and usable threads."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count()}


def cpu_baseline_threads(synth, w, seconds):
    """The same oracle on every host core: each step's output rows split into
    one contiguous range per thread (the C calls release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    T = len(os.sched_getaffinity(0))
    inp = synth.make_inputs(w)
    tiles = oracle.repack(w.qtype, inp.flat, w.K, w.N)
    cuts = [w.N * i // T for i in range(T + 1)]
    n = 0
    with ThreadPoolExecutor(T) as ex:
        t0 = time.perf_counter()
        while True:
            q, d = oracle.quantize_act(inp.x)
            list(ex.map(lambda j: oracle.matmul(w.qtype, tiles, w.K, w.N, q, d,
                                                n0=cuts[j], n1=cuts[j + 1]), range(T)))
            n += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    return {"value": round(w.weight_bytes * n / dt / 1e9, 4), "unit": "GB/s", "cores": T,
            "kind": "oracle",
            "sample": f"{n} full steps of {w.name} in {dt:.1f} s, output rows split over "
                      f"{T} threads"}


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
    if args.launch_only:
        launch_only(torch, tq, synth, args.launch_only, args.steps)
        return

    w, R, dt, det, ref = measure_gemv(torch, tq, synth, args)
    K = args.steps
    ms = dt / K * 1e3
    value = w.weight_bytes / (dt / K) / 1e9
    achieved = gemv_x_bytes(w) / det["qgemv_x_us"] / 1e3
    line = {
        "metric": "qgemv weight-stream GB/s (% of HBM peak); qgemm int8 TOPS (% MFMA peak)",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": w.name, "qtype": "q8_0", "K": w.K, "N": w.N, "M": w.M,
                   "step": "quantize_act + qgemv fused (tq_qgemv_x)", "weight_copies": R,
                   "launch": "eager" if args.eager else "hip graph",
                   "hbm_frac_of_value": round(value / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_bytes("decode"),
                     "kernel": "k_qgemv (fused quantize, Q8_0, M=1)",
                     "kernel_us": round(det["qgemv_x_us"], 3),
                     "bytes_per_launch": gemv_x_bytes(w)},
        "decode_detail_us": {k: round(v, 3) for k, v in det.items()},
        "decode_reference": ref,
        "device": device_info(torch),
    }
    if not args.no_extra:
        line["qgemm"] = measure_gemm(torch, tq, synth)
        line["qgemm_mx"] = measure_mx(torch, tq, synth)
        line["repack"] = measure_repack(torch, tq, synth)
        line["other_workloads"] = measure_others(torch, tq, synth)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(synth, w, args.cpu_seconds)
        line["cpu_baseline_all_cores"] = cpu_baseline_threads(synth, w, args.cpu_seconds / 2)
        line["host"] = host_info()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
