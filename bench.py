#!/usr/bin/env python
"""Benchmark of the tiled block-32 quantized matmul hot path on one MI355X.

Step (the decode hot path, one token of a vocabulary head): dynamic int8
quantization of the activation row (tq_quantize_act) and the tiled GEMV over
the repacked weights (tq_qgemv) -- on the Q8_0 lm-head K=4096 N=128001 M=1
(4001 row-tiles, the last one with a single valid row; int8 codes uniform in
[-127, 127], fp16 scales |N(0,1)|*0.01, fp32 activations N(0,1), seed 0).
This two-launch form is the faster one at this size (the fused tq_qgemv_x is
timed beside it).  The weights are repacked on the GPU once, at load (as the
pages place repacking), into R = 2 distinct copies (2 x 557 MB >= 1 GiB)
that the steps alternate between, so every step streams its weights from HBM
rather than from the 256 MB Infinity Cache.  All inputs are resident in HBM
before the timed region; the K timed steps are replayed from a HIP graph and
timed with HIP events recorded on the stream that replays it.

Printed: one JSON line.  value = weight-tile bytes per step / step time
(GB/s).  roofline = the GEMV kernel of the step: algorithmic bytes (weight
tiles + int8 activations + fp16 scales + fp32 outputs) per launch over its
average duration, launches replayed back to back from a HIP graph on the
current stream, bracketed by HIP events recorded on that stream.
Also reported: the other decode workloads (Q8_0 K=N=4096 M=1; Q4_0 and
IQ4_NL K=4096 N=14336 M=1/4/8), the int8-MFMA GEMM on IQ4_NL M=512
K=N=4096 (TOPS and fraction of the int8 peak) and on the lm-head at M=128,
the block-scaled MXFP4 GEMM, the load-time repack, and the CPU oracle timed
on this host's cores (the step itself, the GEMM and the repack).
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
HEADLINE = "q8_0_lmhead_k4096_n128001_m1"

# HBM traffic of the kernels, from rocprofv3 --pmc passes (FETCH_SIZE, then
# WRITE_SIZE, each in its own run) of `bench.py --launch-only <kernel>`: KiB
# per dispatch of the named kernel as the counters read them, averaged over
# its dispatches.  The same counters read for a plain 256 MiB device copy
# (`--launch-only copy`) give FETCH_SIZE 131083.55 KiB and WRITE_SIZE 262144
# KiB for 262144 KiB moved each way, so FETCH_SIZE is scaled by
# 262144 / 131083.55 and WRITE_SIZE by 1.  "src" is the SHA-256 of the
# kernel's sources when the counters were taken; once they differ, traffic
# is reported as null.
FETCH_SCALE = 262144.0 / 131083.55
WRITE_SCALE = 1.0
TRAFFIC = {
    "lmhead": {"fetch_kib": 272114.03, "write_kib": 500.03,
               "src": "3a423a43e4d871f6bb6356bd6ea67de6b15fe92051fa5175fcce1628c83275ea"},
    "decode": {"fetch_kib": 8765.57, "write_kib": 112.00,
               "src": "3a423a43e4d871f6bb6356bd6ea67de6b15fe92051fa5175fcce1628c83275ea"},
    "gemm": {"fetch_kib": 13370.22, "write_kib": 8192.00,
             "src": "85eea73c90c07c699538e430d7765b8606d76769b19020a9682e93b45cb58ec0"},
    "repack": {"fetch_kib": 16144.35, "write_kib": 32256.00,
               "src": "13ee865d5b5d1480aafc1f034eaad5446734deecedae01956acf64171bf07d6e"},
    "mx": {"fetch_kib": 12897.43, "write_kib": 8192.00,
           "src": "4413a56d8387d2cf011c0fb2982931b0ad3d4c460d439b67a01c5f4de04f9923"},
}
KERNEL_SOURCES = {
    "lmhead": ("qgemv.hip", "tq_internal.h"),
    "decode": ("qgemv.hip", "tq_internal.h"),
    "gemm": ("qgemm.hip", "tq_internal.h"),
    "repack": ("repack.hip", "tq_internal.h"),
    "mx": ("mx.hip", "tq_internal.h"),
}
LAUNCH_ONLY = ("lmhead", "decode", "gemm", "repack", "mx", "copy")


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
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="bounded CPU work per oracle baseline leg")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="only the headline step (no other workloads)")
    p.add_argument("--launch-only", default=None,
                   help="no timing: launch one kernel --steps times on the bench's inputs "
                        "(for rocprofv3 --pmc counter passes) and exit: one of "
                        + ", ".join(LAUNCH_ONLY) + ", or ffn-<type>-m<M> (the decode GEMV, "
                        "int8 activations, on the K=4096 N=14336 weights of <type>)")
    return p.parse_args()


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


def replay_us(torch, g, n):
    """Average time per item of a graph of n items: the graph replayed on the
    current stream between two HIP events recorded on that stream."""
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n * 1e3


def kernel_us(torch, fn, n=200):
    """Average duration of the kernel(s) fn(i) launches: n launches replayed
    back to back from a HIP graph, timed by HIP events on the replaying
    stream."""
    return replay_us(torch, capture(torch, fn, n), n)


def launch_stats(torch, fn, n=200):
    """Per-launch durations: n launches enqueued one by one (no graph), a HIP
    event recorded on the stream between consecutive launches; median, p10
    and p90 of the n intervals."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(n):
        fn(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    t = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n))
    return {"launches": n, "median_us": round(t[n // 2], 3), "p10_us": round(t[n // 10], 3),
            "p90_us": round(t[(9 * n) // 10], 3),
            "timing": "HIP event pair around each launch, launches enqueued one by one"}


def launch_floor_us(torch):
    """A one-element fill kernel, graph-replayed: the cost of a launch that
    does no work."""
    z = torch.zeros(1, dtype=torch.float32, device="cuda")
    return round(kernel_us(torch, lambda i: z.fill_(float(i)), 200), 3)


def stream_read_ref(torch, tq, tiles, nbytes, decode_us=None, n=100):
    """The library's streaming-read instrument (tq_stream_read: 16-byte
    nontemporal loads, one pass, nothing else) over the same rotating tile
    copies, graph-replayed: what merely reading these bytes costs, and the
    decode kernel's time as a fraction of it."""
    R = len(tiles)
    sink = torch.empty(tq.ops.STREAM_READ_BLOCKS, dtype=torch.int32, device="cuda")
    f = lambda i: tq.stream_read(tiles[i % R], nbytes, sink=sink)
    for i in range(3):
        f(i)
    us = min(kernel_us(torch, f, n) for _ in range(2))
    out = {"us": round(us, 3), "GB_s": round(nbytes / us / 1e3, 1),
           "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
    if decode_us:
        out["decode_rate_over_read_rate"] = round(us / decode_us, 4)
    out["note"] = "tq_stream_read over the same rotating tile copies"
    return out


def rotating_tiles(torch, tq, w, flat):
    R = max(2, -(-ROTATE_BYTES // w.weight_bytes))
    return [tq.repack_tiles(w.qtype, flat, w.K, w.N) for _ in range(R)]


def decode_bytes(w, M, fused):
    """Algorithmic bytes of one decode step: tiles, the activations as the
    kernel reads them (fp32 x when fused, else int8 q + fp16 d), fp32 y."""
    act = 4 * M * w.K if fused else M * w.K + 2 * M * (w.K // 32)
    return w.weight_bytes + act + 4 * M * w.N


# ---------------------------------------------------------------------------
# The headline: the lm-head decode step

def setup_headline(torch, tq, synth):
    import numpy as np
    w = synth.WORKLOADS[HEADLINE]
    inp = synth.make_inputs(w)
    flat = torch.from_numpy(inp.flat).cuda()
    tiles = rotating_tiles(torch, tq, w, flat)
    R = len(tiles)
    del flat
    X = 64
    rng = np.random.default_rng(1)
    xs = torch.from_numpy(np.concatenate(
        [inp.x, rng.standard_normal((X - 1, w.K), dtype=np.float32)])).cuda()
    q = torch.empty((1, w.K), dtype=torch.int8, device="cuda")
    d = torch.empty((1, w.K // 32), dtype=torch.float16, device="cuda")
    y = torch.empty((1, w.N), dtype=torch.float32, device="cuda")

    def step(i):                 # one decode token: quantize, then the GEMV
        tq.quantize_act(xs[i % X: i % X + 1], q=q, d=d)
        tq.qgemv(w.qtype, tiles[i % R], w.K, w.N, q, d, out=y)

    parts = {
        "qgemv": lambda i: tq.qgemv(w.qtype, tiles[i % R], w.K, w.N, q, d, out=y),
        "quantize_act": lambda i: tq.quantize_act(xs[i % X: i % X + 1], q=q, d=d),
        "fused": lambda i: tq.qgemv_x(w.qtype, tiles[i % R], w.K, w.N, xs[i % X: i % X + 1],
                                      out=y),
    }
    return w, R, step, parts, tiles


def measure_headline(torch, tq, synth, args):
    w, R, step, parts, tiles = setup_headline(torch, tq, synth)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    g = capture(torch, step, K)
    # the timed region: K steps, synchronized on both sides, HIP events on
    # the replaying stream; the host clock around it is kept as a cross-check
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    us_step = replay_us(torch, g, K)
    host_s = time.perf_counter() - t0
    del g
    stats = launch_stats(torch, parts["qgemv"], 200)
    detail = {
        "qgemv_us": kernel_us(torch, parts["qgemv"], 100),
        "quantize_act_us": kernel_us(torch, parts["quantize_act"], 100),
        "fused_qgemv_x_step_us": kernel_us(torch, parts["fused"], 100),
        "host_clock_us_per_step": host_s / K * 1e6,
    }
    ref = {"read_same_bytes": stream_read_ref(torch, tq, tiles, w.weight_bytes, detail["qgemv_us"])}
    ref["empty_launch_floor_us"] = launch_floor_us(torch)
    del tiles
    return w, R, us_step, detail, ref, stats


# ---------------------------------------------------------------------------
# Other decode workloads

def measure_decodes(torch, tq, synth):
    """Decode steps timed fused (qgemv_x) and as quantize_act + qgemv; GB/s
    counts what the faster form reads and writes.  Config 2 (Q8_0
    K=N=4096 M=1, fused) also gets a roofline object of its own."""
    import numpy as np
    res = {}
    cases = [("q8_0_gemv_k4096_n4096_m1", synth.Q8_0, 4096, 4096, "absnormal", (1,)),
             ("q4_0_gemv_k4096_n14336", synth.Q4_0, 4096, 14336, "uniform", (1, 4, 8)),
             ("iq4_nl_gemv_k4096_n14336", synth.IQ4_NL, 4096, 14336, "uniform", (1, 4, 8))]
    for name, qtype, K, N, dist, Ms in cases:
        w = synth.Workload(name, qtype, K, N, 1, dist)
        inp = synth.make_inputs(w)
        tiles = rotating_tiles(torch, tq, w, torch.from_numpy(inp.flat).cuda())
        R = len(tiles)
        lut = inp.lut if qtype == synth.IQ4_NL else None
        for M in Ms:
            rng = np.random.default_rng(M)
            X = 16
            xs = torch.from_numpy(rng.standard_normal((X * M, K), dtype=np.float32)).cuda()
            q = torch.empty((M, K), dtype=torch.int8, device="cuda")
            d = torch.empty((M, K // 32), dtype=torch.float16, device="cuda")
            y = torch.empty((M, N), dtype=torch.float32, device="cuda")
            xi = lambda i: xs[(i % X) * M:(i % X + 1) * M]
            fused = lambda i: tq.qgemv_x(qtype, tiles[i % R], K, N, xi(i), lut=lut, out=y)

            def two(i):
                tq.quantize_act(xi(i), q=q, d=d)
                tq.qgemv(qtype, tiles[i % R], K, N, q, d, lut=lut, out=y)
            for i in range(5):
                fused(i)
                two(i)
            us_f = kernel_us(torch, fused, 100)
            us_2 = kernel_us(torch, two, 100)
            f = us_f <= us_2
            us = min(us_f, us_2)
            nbytes = decode_bytes(w, M, f)
            label = name if name.endswith("_m1") else f"{name}_m{M}"
            res[label] = {"step_us": round(us, 3),
                          "path": "qgemv_x (fused)" if f else "quantize_act + qgemv",
                          "qgemv_x_us": round(us_f, 3), "quantize_act_qgemv_us": round(us_2, 3),
                          "GB_s": round(nbytes / us / 1e3, 1),
                          "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                          "bytes_per_step": nbytes}
            if name == "q8_0_gemv_k4096_n4096_m1":
                warm = lambda i: tq.qgemv_x(qtype, tiles[0], K, N, xi(i), lut=lut, out=y)
                res[label]["warm_us"] = round(kernel_us(torch, warm, 200), 3)
                res[label]["warm_note"] = ("fused, one weight copy only (17.8 MB, resident in "
                                           "the 256 MB MALL): not an HBM figure")
                ku = kernel_us(torch, fused, 200)
                nb = decode_bytes(w, M, True)
                res[label]["roofline"] = {
                    "bound": "hbm", "achieved": round(nb / ku / 1e3, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(nb / ku / 1e3 / HBM_PEAK_GBS, 4),
                    "traffic": traffic_bytes("decode"),
                    "kernel": "k_qgemv (fused quantize, Q8_0, M=1)", "kernel_us": round(ku, 3),
                    "bytes_per_launch": nb}
        if name != "iq4_nl_gemv_k4096_n14336":
            label = name if name.endswith("_m1") else f"{name}_m1"
            res[label]["read_same_bytes"] = stream_read_ref(
                torch, tq, tiles, w.weight_bytes, res[label]["step_us"])
        del tiles
    res["q4_0_gemv_n_sweep"] = decode_n_sweep(torch, tq, synth)
    return res


def decode_n_sweep(torch, tq, synth):
    """The Q4_0 decode GEMV (M = 1, K = 4096) over N = 4096 .. 32768 (128 to
    1024 stripes on 256 compute units): the line through 256 and 512
    stripes separates a fixed cost per launch from the marginal streaming
    rate, which is what holds a 33 MB decode well below the HBM peak.  The
    streaming-read instrument over the same bytes gets the same fit: the
    fixed cost a plain read of these sizes pays too."""
    import numpy as np
    K = 4096
    out = {}
    for N in (4096, 8192, 14336, 16384, 32768):
        w = synth.Workload("sweep", synth.Q4_0, K, N, 1, "uniform")
        inp = synth.make_inputs(w)
        tiles = rotating_tiles(torch, tq, w, torch.from_numpy(inp.flat).cuda())
        R = len(tiles)
        x = torch.from_numpy(np.random.default_rng(1).standard_normal((1, K), dtype=np.float32)).cuda()
        q, d = tq.quantize_act(x)
        y = torch.empty((1, N), dtype=torch.float32, device="cuda")
        f = lambda i: tq.qgemv(w.qtype, tiles[i % R], K, N, q, d, out=y)
        for i in range(3):
            f(i)
        us = min(kernel_us(torch, f, 100) for _ in range(2))
        rd = stream_read_ref(torch, tq, tiles, w.weight_bytes)
        out[f"n{N}"] = {"stripes": w.n_col_tiles, "kernel_us": round(us, 3),
                        "GB_s": round(w.weight_bytes / us / 1e3, 1),
                        "read_same_bytes_us": rd["us"], "read_GB_s": rd["GB_s"]}
        del tiles
    stripe_bytes = (K // 32) * 576

    def fit(key):
        per = (out["n16384"][key] - out["n8192"][key]) / 256     # us per stripe
        return {"fixed_us": round(out["n8192"][key] - 256 * per, 3),
                "marginal_GB_s": round(stripe_bytes / per / 1e3, 1) if per > 0 else None}
    out["fit_256_to_512_stripes"] = fit("kernel_us")
    out["read_fit_256_to_512_stripes"] = fit("read_same_bytes_us")
    return out


# ---------------------------------------------------------------------------
# GEMMs, repack

def setup_gemm(torch, tq, synth):
    import numpy as np
    w = synth.WORKLOADS["iq4_nl_gemm_m512_k4096_n4096"]
    inp = synth.make_inputs(w)
    tiles = rotating_tiles(torch, tq, w, torch.from_numpy(inp.flat).cuda())
    R = len(tiles)
    x = torch.from_numpy(inp.x.view(np.int16)).cuda().view(torch.bfloat16)
    q, d = tq.quantize_act(x)
    y = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    f = lambda i: tq.qgemm(w.qtype, tiles[i % R], w.K, w.N, q, d, lut=inp.lut, out=y)
    quant = lambda i: tq.quantize_act(x, q=q, d=d)
    return w, f, quant


def gemm_bytes(w, M=None):
    """Algorithmic bytes of one GEMM launch: tiles + int8 q + fp16 d + fp32 y."""
    M = w.M if M is None else M
    return w.weight_bytes + M * w.K + 2 * M * (w.K // 32) + 4 * M * w.N


def measure_gemm(torch, tq, synth, n=200):
    w, f, quant = setup_gemm(torch, tq, synth)
    for i in range(20):
        f(i)
    us = kernel_us(torch, f, n)
    quant_us = kernel_us(torch, quant, 50)
    tops = 2.0 * w.M * w.N * w.K / us / 1e6
    return {"workload": w.name, "metric": "qgemm int8 TOPS", "value": round(tops, 2),
            "unit": "TOPS", "kernel_us": round(us, 3), "quantize_act_us": round(quant_us, 3),
            "hbm_GB_s": round(gemm_bytes(w) / us / 1e3, 1),
            "roofline": {"bound": "mfma", "achieved": round(tops, 2), "peak": INT8_PEAK_TOPS,
                         "unit": "TOP/s", "frac": round(tops / INT8_PEAK_TOPS, 4),
                         "traffic": traffic_bytes("gemm"), "bytes_per_launch": gemm_bytes(w)}}


def measure_lmhead_gemm(torch, tq, synth):
    """The lm-head at M=128 (config 5's prefill side): below the int8 ridge,
    so both its HBM and its MFMA fractions are reported."""
    import numpy as np
    w = synth.WORKLOADS["q8_0_lmhead_k4096_n128001_m128"]
    inp = synth.make_inputs(w, M=1)
    tiles = rotating_tiles(torch, tq, w, torch.from_numpy(inp.flat).cuda())
    R = len(tiles)
    x = torch.from_numpy(np.random.default_rng(128).standard_normal(
        (w.M, w.K), dtype=np.float32)).cuda()
    q, d = tq.quantize_act(x)
    y = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    f = lambda i: tq.qgemm(w.qtype, tiles[i % R], w.K, w.N, q, d, out=y)
    for i in range(3):
        f(i)
    us = kernel_us(torch, f, 30)
    nb = gemm_bytes(w)
    tops = 2.0 * w.M * w.N * w.K / us / 1e6
    del tiles
    return {"workload": w.name, "kernel_us": round(us, 3), "TOPS": round(tops, 2),
            "int8_frac": round(tops / INT8_PEAK_TOPS, 4), "GB_s": round(nb / us / 1e3, 1),
            "hbm_frac": round(nb / us / 1e3 / HBM_PEAK_GBS, 4), "bytes_per_launch": nb}


def setup_mx(torch, tq, synth):
    """MXFP4 M=512 K=N=4096 on the block-scaled matrix cores (MXFP8
    activations from bf16, like the int8 GEMM workload's)."""
    import numpy as np
    w = synth.WORKLOADS["mxfp4_gemm_m512_k4096_n4096"]
    inp = synth.make_inputs(w)
    tiles = rotating_tiles(torch, tq, w, torch.from_numpy(inp.flat).cuda())
    R = len(tiles)
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
    """The widened formats and paths, timed like the rest (graph of steps,
    HIP events); weights rotate over >= 1 GiB."""
    import numpy as np
    res = {}
    cases = [("mxfp4_gemv_k4096_n14336_m1", 1), ("mxfp4_gemv_k4096_n14336_m1", 4),
             ("mxfp4_gemm_m512_k4096_n4096", 512), ("q4_1_gemv_k4096_n14336_m1", 1),
             ("q4_1_gemv_k4096_n14336_m1", 4), ("q4_1_gemm_m512_k4096_n4096", 512),
             ("q4_k_gemv_k4096_n14336_m1", 1)]
    tiles_cache = {}
    for name, M in cases:
        w = synth.WORKLOADS[name]
        key = (w.qtype, w.K, w.N)
        if key not in tiles_cache:
            inp = synth.make_inputs(w, M=1)
            tiles_cache.clear()
            tiles_cache[key] = rotating_tiles(torch, tq, w, torch.from_numpy(inp.flat).cuda())
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
            for i in range(5):
                fused(i)
                two(i)
            us_f = kernel_us(torch, fused, 50)
            us_2 = kernel_us(torch, two, 50)
            us = min(us_f, us_2)
            nbytes = decode_bytes(w, M, us_f <= us_2)
            res[f"{name.rsplit('_m', 1)[0]}_m{M}"] = {
                "step_us": round(us, 3),
                "path": "qgemv_x (fused)" if us_f <= us_2 else "quantize_act + qgemv",
                "qgemv_x_us": round(us_f, 3), "quantize_act_qgemv_us": round(us_2, 3),
                "GB_s": round(nbytes / us / 1e3, 1),
                "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
        else:
            q, d = tq.quantize_act(x)
            f = lambda i: tq.qgemm(w.qtype, tiles[i % R], w.K, w.N, q, d)
            for i in range(5):
                f(i)
            us = kernel_us(torch, f, 50)
            nbytes = gemm_bytes(w, M)
            res[f"{name} qgemm"] = {"kernel_us": round(us, 3), "GB_s": round(nbytes / us / 1e3, 1),
                                    "TOPS": round(2.0 * M * w.N * w.K / us / 1e6, 2)}
    tiles_cache.clear()
    # repack of every type at the FFN shape (flat copies rotate over >= 1 GiB)
    for qtype in (synth.Q8_0, synth.IQ4_NL, synth.MXFP4, synth.Q4_1, synth.Q4_K):
        w = synth.Workload("repack", qtype, 4096, 14336, 1,
                           {synth.Q8_0: "absnormal", synth.MXFP4: "e8m0", synth.Q4_1: "minmax",
                            synth.Q4_K: "q4k"}.get(qtype, "uniform"))
        inp = synth.make_inputs(w)
        fb = inp.flat.size
        flats = [torch.from_numpy(inp.flat).cuda()
                 for _ in range(min(32, max(2, -(-ROTATE_BYTES // fb))))]
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
        if name.startswith("q4_0") and M == 1:
            out = torch.empty(fb, dtype=torch.uint8, device="cuda")
            fu = lambda i: tq.unpack_tiles(w.qtype, tiles[i % R], w.K, w.N, out=out)
            fu(0)
            uu = kernel_us(torch, fu, 30)
            res[f"unpack {name.rsplit('_m', 1)[0]}"] = {
                "kernel_us": round(uu, 3), "GB_s": round((fb + w.weight_bytes) / uu / 1e3, 1)}
        del flats, tiles
    # small-M products through tq_matmul beside the GEMM on the same tiles
    for qtype in (synth.Q4_0, synth.IQ4_NL, synth.Q8_0):
        wq = synth.Workload("small_m", qtype, 4096, 4096, 1,
                            "absnormal" if qtype == synth.Q8_0 else "uniform")
        inp = synth.make_inputs(wq)
        tiles = rotating_tiles(torch, tq, wq, torch.from_numpy(inp.flat).cuda())
        R = len(tiles)
        lut = inp.lut if qtype == synth.IQ4_NL else None
        for M in (16, 32, 64, 128):
            rng = np.random.default_rng(M)
            x = torch.from_numpy(rng.standard_normal((M, wq.K), dtype=np.float32)).cuda()
            q, d = tq.quantize_act(x)
            y = torch.empty((M, wq.N), dtype=torch.float32, device="cuda")
            fm = lambda i: tq.matmul(qtype, tiles[i % R], wq.K, wq.N, q, d, lut=lut, out=y)
            fg = lambda i: tq.qgemm(qtype, tiles[i % R], wq.K, wq.N, q, d, lut=lut, out=y)
            for i in range(3):
                fm(i)
                fg(i)
            um, ug = kernel_us(torch, fm, 30), kernel_us(torch, fg, 30)
            path = {tq.PATH_GEMV: "decode passes", tq.PATH_GEMM: "qgemm",
                    tq.PATH_GEMM_SPLIT: "qgemm, K split"}[tq.matmul_path(qtype, wq.K, wq.N, M)]
            res[f"{synth.TYPE_NAMES[qtype]}_matmul_k4096_n4096_m{M}"] = {
                "matmul_us": round(um, 3), "path": path, "qgemm_us": round(ug, 3),
                "TOPS": round(2.0 * M * wq.N * wq.K / um / 1e6, 2)}
        del tiles
    # the block-scaled GEMM at small M: tq_matmul_mx (K split where its cost
    # model says faster) beside the unsplit tq_qgemm_mx
    for K, Ms in ((4096, (8, 64, 128)), (8192, (128,))):
        wm = synth.Workload("mx_small_m", synth.MXFP4, K, 4096, 1, "e8m0")
        inp = synth.make_inputs(wm)
        tiles = rotating_tiles(torch, tq, wm, torch.from_numpy(inp.flat).cuda())
        R = len(tiles)
        for M in Ms:
            x = torch.from_numpy(np.random.default_rng(M).standard_normal(
                (M, K), dtype=np.float32)).cuda()
            q, e = tq.quantize_act_mx(x)
            y = torch.empty((M, wm.N), dtype=torch.float32, device="cuda")
            fm = lambda i: tq.matmul_mx(tiles[i % R], K, wm.N, q, e, out=y)
            fg = lambda i: tq.qgemm_mx(tiles[i % R], K, wm.N, q, e, out=y)
            for i in range(3):
                fm(i)
                fg(i)
            um, ug = kernel_us(torch, fm, 30), kernel_us(torch, fg, 30)
            need = tq.lib().tq_matmul_mx_workspace_bytes(K, wm.N, M)
            S = (need - (1 << 20)) // (M * wm.N * 4) if need else 1
            res[f"mxfp4_matmul_mx_k{K}_n4096_m{M}"] = {
                "matmul_mx_us": round(um, 3), "k_split": int(S), "qgemm_mx_us": round(ug, 3),
                "TFLOPS": round(2.0 * M * wm.N * K / um / 1e6, 2)}
        del tiles
    return res


def launch_only(torch, tq, synth, kernel, n):
    """Launch one kernel n times, eagerly, untimed (counter collection)."""
    if kernel.startswith("ffn-"):
        import numpy as np
        _, tname, m = kernel.split("-")
        qtype = {v: k for k, v in synth.TYPE_NAMES.items()}[tname]
        M = int(m[1:])
        w = synth.Workload("ffn", qtype, 4096, 14336, 1, "uniform")
        inp = synth.make_inputs(w)
        tiles = rotating_tiles(torch, tq, w, torch.from_numpy(inp.flat).cuda())
        x = torch.from_numpy(np.random.default_rng(M).standard_normal((M, 4096), dtype=np.float32)).cuda()
        q, d = tq.quantize_act(x)
        y = torch.empty((M, w.N), dtype=torch.float32, device="cuda")
        lut = inp.lut if qtype == synth.IQ4_NL else None
        f = lambda i: tq.qgemv(qtype, tiles[i % len(tiles)], w.K, w.N, q, d, lut=lut, out=y)
    elif kernel == "lmhead":
        _, _, _, parts, _ = setup_headline(torch, tq, synth)
        parts["quantize_act"](0)
        f = parts["qgemv"]
    elif kernel == "decode":
        w = synth.WORKLOADS["q8_0_gemv_k4096_n4096_m1"]
        inp = synth.make_inputs(w)
        tiles = rotating_tiles(torch, tq, w, torch.from_numpy(inp.flat).cuda())
        x = torch.from_numpy(inp.x).cuda()
        y = torch.empty((1, w.N), dtype=torch.float32, device="cuda")
        f = lambda i: tq.qgemv_x(w.qtype, tiles[i % len(tiles)], w.K, w.N, x, out=y)
    elif kernel == "gemm":
        f = setup_gemm(torch, tq, synth)[1]
    elif kernel == "repack":
        f = setup_repack(torch, tq, synth)[1]
    elif kernel == "mx":
        f = setup_mx(torch, tq, synth)[1]
    elif kernel == "copy":                  # calibration: a plain 256 MiB copy
        a = torch.ones(1 << 28, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        f = lambda i: b.copy_(a)
    else:
        raise SystemExit(f"unknown --launch-only kernel {kernel!r}")
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


# ---------------------------------------------------------------------------
# The CPU oracle, timed on this host (bounded samples of the same workloads)

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


def _threads():
    return len(os.sched_getaffinity(0))


def _split_matmul(ex, T, oracle, w, tiles, q, d, lut, n0, n1):
    cuts = [n0 + (n1 - n0) * i // T for i in range(T + 1)]
    list(ex.map(lambda j: oracle.matmul(w.qtype, tiles, w.K, w.N, q, d, lut,
                                        n0=cuts[j], n1=cuts[j + 1]), range(T)))


def cpu_baselines(synth, seconds):
    """The oracle as it stands (plain C, fp64), on the same workloads:
    - the headline step (quantize_act + matmul of the lm-head, M=1): full
      steps on 1 thread for about `seconds`, and with the output rows split
      over every host thread;
    - the lm-head at M=128: 1/32 of its row-stripes on 1 thread, scaled,
      and the whole product over every host thread;
    - the IQ4_NL M=512 GEMM: a stated subset of the 128 row-stripes on 1
      thread, scaled to the whole product, and the whole product split over
      every host thread;
    - the repack of the Q4_0 FFN weights (K=4096 N=14336), 1 thread."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    T = _threads()
    out = {}
    w = synth.WORKLOADS[HEADLINE]
    inp = synth.make_inputs(w)
    tiles = oracle.repack(w.qtype, inp.flat, w.K, w.N)
    inp.flat = inp.codes = None
    n, t0 = 0, time.perf_counter()
    while True:
        q, d = oracle.quantize_act(inp.x)
        oracle.matmul(w.qtype, tiles, w.K, w.N, q, d)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    out["cpu_baseline"] = {
        "value": round(w.weight_bytes * n / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
        "kind": "oracle", "ms_per_step": round(dt / n * 1e3, 1),
        "sample": f"{n} full steps (quantize_act + fp64 matmul) of {w.name} in {dt:.1f} s, "
                  "1 thread; GB/s of weight tiles, as value"}
    with ThreadPoolExecutor(T) as ex:
        n, t0 = 0, time.perf_counter()
        while True:
            q, d = oracle.quantize_act(inp.x)
            _split_matmul(ex, T, oracle, w, tiles, q, d, None, 0, w.N)
            n += 1
            if time.perf_counter() - t0 >= seconds / 2:
                break
        dt = time.perf_counter() - t0
    out["cpu_baseline_all_cores"] = {
        "value": round(w.weight_bytes * n / dt / 1e9, 4), "unit": "GB/s", "cores": T,
        "kind": "oracle", "ms_per_step": round(dt / n * 1e3, 1),
        "sample": f"{n} full steps of {w.name} in {dt:.1f} s, output rows split over "
                  f"{T} threads"}

    # the lm-head at M = 128 (the prefill side of config 5), on the same
    # weights: 1/32 of the stripes on 1 thread, scaled, and the whole
    # product over every host thread
    import numpy as np
    M5 = 128
    x5 = np.random.default_rng(128).standard_normal((M5, w.K), dtype=np.float32)
    q5, d5 = oracle.quantize_act(x5)
    sub = -(-w.n_col_tiles // 32)
    t0 = time.perf_counter()
    oracle.matmul(w.qtype, tiles, w.K, w.N, q5, d5, None, n0=0, n1=32 * sub)
    dt1 = time.perf_counter() - t0
    with ThreadPoolExecutor(T) as ex:
        t0 = time.perf_counter()
        _split_matmul(ex, T, oracle, w, tiles, q5, d5, None, 0, w.N)
        dtT = time.perf_counter() - t0
    ops5 = 2.0 * M5 * w.N * w.K
    out["cpu_baseline_lmhead_m128"] = {
        "value": round(2.0 * M5 * 32 * sub * w.K / dt1 / 1e9, 3), "unit": "GOPS", "cores": 1,
        "kind": "oracle", "scaled_full_product_s": round(dt1 * w.N / (32 * sub), 1),
        "sample": f"{w.name} at M={M5}: {sub} of {w.n_col_tiles} row-stripes in {dt1:.1f} s "
                  "on 1 thread, scaled by ops"}
    out["cpu_baseline_lmhead_m128_all_cores"] = {
        "value": round(ops5 / dtT / 1e9, 3), "unit": "GOPS", "cores": T, "kind": "oracle",
        "sample": f"{w.name} at M={M5}: the whole product in {dtT:.1f} s, output rows split "
                  f"over {T} threads"}
    del tiles, inp

    # the GEMM (config 4): GOPS = 2 M N K / time, same formula as the GPU's
    wg = synth.WORKLOADS["iq4_nl_gemm_m512_k4096_n4096"]
    inp = synth.make_inputs(wg)
    tiles = oracle.repack(wg.qtype, inp.flat, wg.K, wg.N)
    q, d = oracle.quantize_act(inp.x, oracle.BF16)
    stripes = 8
    t0 = time.perf_counter()
    oracle.matmul(wg.qtype, tiles, wg.K, wg.N, q, d, inp.lut, n0=0, n1=32 * stripes)
    dt1 = time.perf_counter() - t0
    ops_sub = 2.0 * wg.M * 32 * stripes * wg.K
    with ThreadPoolExecutor(T) as ex:
        t0 = time.perf_counter()
        _split_matmul(ex, T, oracle, wg, tiles, q, d, inp.lut, 0, wg.N)
        dtT = time.perf_counter() - t0
    ops = 2.0 * wg.M * wg.N * wg.K
    out["cpu_baseline_qgemm"] = {
        "value": round(ops_sub / dt1 / 1e9, 3), "unit": "GOPS", "cores": 1, "kind": "oracle",
        "scaled_full_product_s": round(dt1 * wg.N / (32 * stripes), 1),
        "sample": f"{wg.name}: {stripes} of {wg.n_col_tiles} row-stripes (all 512 activation "
                  f"rows) in {dt1:.1f} s on 1 thread, scaled by ops"}
    out["cpu_baseline_qgemm_all_cores"] = {
        "value": round(ops / dtT / 1e9, 3), "unit": "GOPS", "cores": T, "kind": "oracle",
        "sample": f"{wg.name}: the whole product in {dtT:.1f} s, output rows split over "
                  f"{T} threads"}
    del tiles, inp

    # the repack of config 3's weights: bytes read + written per second
    wr = synth.WORKLOADS["q4_0_gemv_k4096_n14336_m1"]
    inp = synth.make_inputs(wr)
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.repack(wr.qtype, inp.flat, wr.K, wr.N)
        n += 1
        if time.perf_counter() - t0 >= seconds / 2:
            break
    dt = time.perf_counter() - t0
    out["cpu_baseline_repack"] = {
        "value": round((inp.flat.size + wr.weight_bytes) * n / dt / 1e9, 4), "unit": "GB/s",
        "cores": 1, "kind": "oracle",
        "sample": f"{n} repacks of {wr.name}'s Q4_0 weights in {dt:.1f} s, 1 thread "
                  "(flat bytes read + tile bytes written)"}
    return out


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

    w, R, us_step, det, ref, stats = measure_headline(torch, tq, synth, args)
    K = args.steps
    value = w.weight_bytes / us_step / 1e3
    kb = decode_bytes(w, 1, False)          # tiles + int8 q + fp16 d + fp32 y
    achieved = kb / det["qgemv_us"] / 1e3
    line = {
        "metric": "qgemv weight-stream GB/s (% of HBM peak); qgemm int8 TOPS (% MFMA peak)",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(us_step / 1e3, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": w.name, "qtype": "q8_0", "K": w.K, "N": w.N, "M": 1,
                   "step": "quantize_act + qgemv (two launches)", "weight_copies": R,
                   "launch": "hip graph, HIP events on the replaying stream",
                   "hbm_frac_of_value": round(value / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_bytes("lmhead"),
                     "kernel": "k_qgemv (Q8_0, M=1, int8 activations)",
                     "kernel_us": round(det["qgemv_us"], 3), "bytes_per_launch": kb},
        "step_detail_us": {k: round(v, 3) for k, v in det.items()},
        "qgemv_launch_stats": stats,
        "step_reference": ref,
        "device": device_info(torch),
    }
    torch.cuda.empty_cache()
    if not args.no_extra:
        line["decode"] = measure_decodes(torch, tq, synth)
        line["qgemm"] = measure_gemm(torch, tq, synth)
        line["qgemm_lmhead_m128"] = measure_lmhead_gemm(torch, tq, synth)
        torch.cuda.empty_cache()
        line["qgemm_mx"] = measure_mx(torch, tq, synth)
        line["repack"] = measure_repack(torch, tq, synth)
        line["other_workloads"] = measure_others(torch, tq, synth)
    if not args.no_cpu_baseline:
        cb = cpu_baselines(synth, args.cpu_seconds)
        line["cpu_baseline"] = cb.pop("cpu_baseline")
        line["cpu_baselines_more"] = cb
        line["host"] = host_info()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
