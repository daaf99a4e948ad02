"""The largest shapes the entry points accept, against the oracle:
N = 2^27 weight rows (2^22 column tiles: the largest repack, decode and GEMM
grids) and K = 2^20 (the longest k-loops and the deepest decode K split).

The N = 2^27 weights (2.4 GB of flat Q4_0 blocks) are drawn on the device;
sampled stripes (first, second, middle, last two) are copied back and checked
-- repack bit for bit, products within the fp32 bound -- against the oracle
run on just those rows."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import check_mx, check_y, make

pytestmark = pytest.mark.gpu
Q4_0, Q8_0, MXFP4 = synth.Q4_0, synth.Q8_0, synth.MXFP4


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_matmul_repack_amd as tq
    tq.lib()
    return tq


def test_max_n_q4_0(tq):
    K, N = 32, 2 ** 27
    nct = N // 32
    assert tq.supported(Q4_0, K, N, 1) and not tq.supported(Q4_0, K, N + 1, 1)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    flat = torch.randint(0, 256, (N, 18), dtype=torch.uint8, device="cuda", generator=g)
    # fp16 row scales: positive normals 2^-14 .. 2^-6 (bit patterns 0x0400 .. 0x2400)
    sc = torch.randint(0x0400, 0x2400, (N,), dtype=torch.int32, device="cuda", generator=g)
    flat[:, 0] = (sc & 0xFF).to(torch.uint8)
    flat[:, 1] = (sc >> 8).to(torch.uint8)
    flat = flat.reshape(-1)
    tiles = tq.repack_tiles(Q4_0, flat, K, N)
    x = torch.from_numpy(synth.draw_activations(np.random.default_rng(3), 1, K)).cuda()
    q, d = tq.quantize_act(x)
    y_gemv = tq.qgemv(Q4_0, tiles, K, N, q, d)
    y_gemm = tq.qgemm(Q4_0, tiles, K, N, q, d)
    torch.cuda.synchronize()
    qh, dh = oracle.quantize_act(x.cpu().numpy())
    assert np.array_equal(q.cpu().numpy(), qh) and np.array_equal(d.cpu().numpy().view(np.uint16), dh)
    ts = oracle.tile_bytes(Q4_0)
    for ct in (0, 1, nct // 2 + 5, nct - 2, nct - 1):
        rows = slice(32 * ct, 32 * ct + 32)
        fl = flat[32 * ct * 18:(32 * ct + 32) * 18].cpu().numpy()
        t_ref = oracle.repack(Q4_0, fl, K, 32)
        assert np.array_equal(tiles[ct * ts:(ct + 1) * ts].cpu().numpy(), t_ref), ct
        y_ref, acond = oracle.matmul(Q4_0, t_ref, K, 32, qh, dh)
        check_y(y_gemv[:, rows].cpu().numpy(), y_ref, acond, ("gemv", ct))
        check_y(y_gemm[:, rows].cpu().numpy(), y_ref, acond, ("gemm", ct))
    del flat, tiles, y_gemv, y_gemm
    torch.cuda.empty_cache()


@pytest.mark.parametrize("qtype", [Q8_0, synth.IQ4_NL])
def test_max_k(tq, qtype):
    K, N = 2 ** 20, 40
    inp = make(qtype, K, N, 33, seed=11)
    tiles = oracle.repack(qtype, inp.flat, K, N)
    td = tq.repack_tiles(qtype, torch.from_numpy(inp.flat).cuda(), K, N)
    assert np.array_equal(td.cpu().numpy(), tiles)
    x = torch.from_numpy(inp.x).cuda()
    q, d = tq.quantize_act(x)
    qh, dh = oracle.quantize_act(inp.x)
    assert np.array_equal(q.cpu().numpy(), qh)
    lut = synth.IQ4_NL_STANDIN_LUT if qtype == synth.IQ4_NL else None
    y_ref, acond = oracle.matmul(qtype, tiles, K, N, qh, dh, lut)
    for M in (1, 8):
        y = tq.qgemv(qtype, td, K, N, q[:M], d[:M], lut=lut)
        check_y(y.cpu().numpy(), y_ref[:M], acond[:M], ("gemv", M))
    y = tq.qgemm(qtype, td, K, N, q, d, lut=lut)
    check_y(y.cpu().numpy(), y_ref, acond, "gemm")


def test_max_k_mx(tq):
    K, N, M = 2 ** 20, 40, 17
    inp = make(MXFP4, K, N, M, seed=12)
    tiles = oracle.repack(MXFP4, inp.flat, K, N)
    qh, eh = oracle.quantize_act_mx(inp.x)
    y_ref, acond = oracle.matmul_mx(tiles, K, N, qh, eh)
    q, e = tq.quantize_act_mx(torch.from_numpy(inp.x).cuda())
    assert np.array_equal(q.cpu().numpy(), qh) and np.array_equal(e.cpu().numpy(), eh)
    y = tq.qgemm_mx(torch.from_numpy(tiles).cuda(), K, N, q, e).cpu().numpy()
    check_mx(y, y_ref, acond, "mx", K)
