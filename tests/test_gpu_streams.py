"""Stream and graph semantics of the entry points: every call runs on the
stream it is given (a side stream gives the same bits as the default one),
calls replayed from a captured HIP graph give the bits of the same calls made
eagerly, replay after replay with eager work in between, and the K-split
workspace of the decode product is all zero after every call (the next call
on that stream relies on it).  All kernels here are deterministic, so the
comparisons are bit for bit; one eager result per product is also checked
against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import check_mx, check_y, make

pytestmark = pytest.mark.gpu

K, N = 1024, 300          # 10 column tiles, the last one ragged: the decode splits K 8 ways
MG = 130                  # GEMM rows: two row blocks, the second ragged
MX_M = 64
LUT = synth.IQ4_NL_STANDIN_LUT


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_matmul_repack_amd as tq
    tq.lib()
    return tq


@pytest.fixture(scope="module")
def weights(tq):
    """Tiles of four formats (repacked on the device) and their inputs."""
    out = {}
    for qt in (synth.Q4_0, synth.Q8_0, synth.IQ4_NL, synth.MXFP4):
        inp = make(qt, K, N, 1, seed=20 + qt)
        flat = torch.from_numpy(inp.flat).cuda()
        out[qt] = (inp, flat, tq.repack_tiles(qt, flat, K, N))
    return out


def activations(seed, M):
    return torch.from_numpy(
        synth.draw_activations(np.random.default_rng(seed), M, K)).cuda()


def run_all(tq, w, x4, xg, outs):
    """The calls under test, writing into the tensors of outs."""
    tq.quantize_act(x4, q=outs["q4"], d=outs["d4"])
    tq.qgemv(synth.Q4_0, w[synth.Q4_0][2], K, N, outs["q4"], outs["d4"], out=outs["gemv"])
    tq.qgemv_x(synth.Q8_0, w[synth.Q8_0][2], K, N, x4[:1], out=outs["gemv_x"])
    tq.quantize_act(xg, q=outs["qg"], d=outs["dg"])
    tq.qgemm(synth.IQ4_NL, w[synth.IQ4_NL][2], K, N, outs["qg"], outs["dg"], lut=LUT,
             out=outs["gemm"])
    tq.quantize_act_mx(xg[:MX_M], q=outs["qm"], e=outs["em"])
    tq.qgemm_mx(w[synth.MXFP4][2], K, N, outs["qm"], outs["em"], out=outs["mx"])
    tq.repack_tiles(synth.Q4_0, w[synth.Q4_0][1], K, N, out=outs["tiles"])


def new_outs(tq):
    dev = "cuda"
    return {
        "q4": torch.empty((4, K), dtype=torch.int8, device=dev),
        "d4": torch.empty((4, K // 32), dtype=torch.float16, device=dev),
        "gemv": torch.empty((4, N), dtype=torch.float32, device=dev),
        "gemv_x": torch.empty((1, N), dtype=torch.float32, device=dev),
        "qg": torch.empty((MG, K), dtype=torch.int8, device=dev),
        "dg": torch.empty((MG, K // 32), dtype=torch.float16, device=dev),
        "gemm": torch.empty((MG, N), dtype=torch.float32, device=dev),
        "qm": torch.empty((MX_M, K), dtype=torch.uint8, device=dev),
        "em": torch.empty((MX_M, K // 32), dtype=torch.uint8, device=dev),
        "mx": torch.empty((MX_M, N), dtype=torch.float32, device=dev),
        "tiles": torch.empty(tq.tiled_bytes(synth.Q4_0, K, N), dtype=torch.uint8, device=dev),
    }


def assert_same(a, b, what):
    for k in a:
        assert torch.equal(a[k], b[k]), (what, k)


def workspaces_zero(tq):
    """The binding's workspaces keep their slot region (the first
    TQ_NOALLOC_SCRATCH_BYTES = 1 MiB, where the decode split's slots lie)
    zero; what follows is scratch (activation codes, partial planes)."""
    from block_quantized_matmul_repack_amd import ops
    torch.cuda.synchronize()
    return all(bool((ws[: 1 << 20] == 0).all()) for ws in ops._workspaces.values())


def test_eager_results_match_oracle(tq, weights):
    x4, xg = activations(1, 4), activations(2, MG)
    o = new_outs(tq)
    run_all(tq, weights, x4, xg, o)
    torch.cuda.synchronize()
    inp, _, tiles = weights[synth.Q4_0]
    q, d = oracle.quantize_act(x4.cpu().numpy())
    y, a = oracle.matmul(synth.Q4_0, tiles.cpu().numpy(), K, N, q, d)
    check_y(o["gemv"].cpu().numpy(), y, a, "gemv")
    assert np.array_equal(o["tiles"].cpu().numpy(), tiles.cpu().numpy())
    t8 = weights[synth.Q8_0][2].cpu().numpy()
    y, a = oracle.matmul(synth.Q8_0, t8, K, N, q[:1], d[:1])
    check_y(o["gemv_x"].cpu().numpy(), y, a, "gemv_x")
    qg, dg = oracle.quantize_act(xg.cpu().numpy())
    y, a = oracle.matmul(synth.IQ4_NL, weights[synth.IQ4_NL][2].cpu().numpy(), K, N, qg, dg, LUT)
    check_y(o["gemm"].cpu().numpy(), y, a, "gemm")
    qm, em = oracle.quantize_act_mx(xg[:MX_M].cpu().numpy())
    assert np.array_equal(o["qm"].cpu().numpy(), qm) and np.array_equal(o["em"].cpu().numpy(), em)
    y, a = oracle.matmul_mx(weights[synth.MXFP4][2].cpu().numpy(), K, N, qm, em)
    check_mx(o["mx"].cpu().numpy(), y, a, "mx", K)    # the block-scaled path's bound
    assert workspaces_zero(tq)


def test_side_stream_matches_default(tq, weights):
    x4, xg = activations(3, 4), activations(4, MG)
    ref = new_outs(tq)
    run_all(tq, weights, x4, xg, ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = new_outs(tq)
        run_all(tq, weights, x4, xg, got)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert_same(got, ref, "side stream")
    assert workspaces_zero(tq)


def test_graph_replays_match_eager(tq, weights):
    x4 = torch.empty((4, K), dtype=torch.float32, device="cuda")
    xg = torch.empty((MG, K), dtype=torch.float32, device="cuda")
    x4.copy_(activations(5, 4))
    xg.copy_(activations(6, MG))
    static = new_outs(tq)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_all(tq, weights, x4, xg, static)        # warm-up: the stream's workspace exists
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run_all(tq, weights, x4, xg, static)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for it in range(4):
        x4.copy_(activations(10 + it, 4))
        xg.copy_(activations(20 + it, MG))
        ref = new_outs(tq)
        run_all(tq, weights, x4, xg, ref)           # eager, default stream
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same(static, ref, ("replay", it))
        assert workspaces_zero(tq)
        # unrelated eager work between replays
        run_all(tq, weights, xg[:4], x4.repeat(33, 1)[:MG], new_outs(tq))
        torch.cuda.synchronize()
