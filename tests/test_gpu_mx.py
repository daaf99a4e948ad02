"""MXFP4 tiles x MXFP8 activations on the block-scaled matrix cores, against
the oracle: the MXFP8 quantizer bit-exact, the product elementwise within a
bound derived beforehand from how the instruction adds, and normwise within
1e-4.

Bound.  One v_mfma_scale_f32_32x32x64_f8f6f4 forms 64 products of E4M3 and
E2M1 values, each scaled by a power of two: every product is exact (3 + 1
significant bits).  The instruction adds its 64 products with a limited
internal precision rather than in exact or fp32 arithmetic; taking it to keep
at least 15 significant bits of the magnitude sum of its products (twice the
error of the 16 bits the instruction was observed to keep), its error is at
most 2^-14 * sum_i |p_i| over that instruction's products.  The kernel adds
the K/64 instruction results of an output in fp32 (the matrix core's
accumulator), one rounding of at most 2^-24 * A each, and the two wave
groups' partial sums once more.  Summed over the K/64 instructions:

    |y - y_ref| <= 2^-14 * A + (K/64 + 1) * 2^-24 * A,

A = sum_k |W * A| (the oracle's conditioning sum).  An element passes if it
is within that bound or within the stated 1e-3 relative bound.  At K = 4096
the bound is 6.5e-5 * A; a layout, scale or indexing mistake gives errors of
the order of A itself."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import check_mx, check_y, make, to_dev_act

pytestmark = pytest.mark.gpu
MXFP4 = synth.MXFP4


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_matmul_repack_amd as tq
    tq.lib()
    return tq


def specials(x):
    """Blocks that exercise the scale rule, ties, saturation and signs."""
    K = x.shape[1]
    x[0, :32] = 0.0                                  # all-zero block: e = 0
    if K >= 128:
        x[0, 32:64] = 1.5                            # constant block
        x[0, 64:96] = np.float32(2.0 ** -120)        # scale clamped to e = 0
        x[0, 96] = 511.0                             # X = 1 for the rest of the block
        x[0, 97:106] = [448.0, 460.0, 479.0, -490.0, -0.0, 0.0029296875, 0.0009765625,
                        9.0, 13.0]                   # saturation, signed zero, ties
    return x


@pytest.mark.parametrize("act", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("M,K", [(1, 32), (3, 256), (8, 4096), (37, 1024), (130, 96)])
def test_quantize_mx_bitexact(tq, act, M, K):
    inp = make(MXFP4, K, 1, M, seed=M * 100 + K, act=act)
    x = inp.x.copy()
    if act == "f32":
        x = specials(x)
    dt = {"f32": oracle.F32, "bf16": oracle.BF16, "f16": oracle.F16}[act]
    qr, er = oracle.quantize_act_mx(x, dt)
    q, e = tq.quantize_act_mx(to_dev_act(x, act))
    assert np.array_equal(q.cpu().numpy(), qr)
    assert np.array_equal(e.cpu().numpy(), er)


def test_quantize_mx_row_stride(tq):
    inp = make(MXFP4, 256, 1, 5, seed=3)
    wide = np.concatenate([inp.x, np.full((5, 64), 9e5, np.float32)], axis=1)
    qr, er = oracle.quantize_act_mx(wide, oracle.F32, K=256)
    q, e = tq.quantize_act_mx(torch.from_numpy(wide).cuda(), K=256)
    assert np.array_equal(q.cpu().numpy(), qr)
    assert np.array_equal(e.cpu().numpy(), er)


def mx_case(tq, M, K, N, seed, ebytes=None):
    inp = make(MXFP4, K, N, M, seed=seed)
    flat = inp.flat
    if ebytes is not None:
        flat = synth.pack_flat(MXFP4, inp.codes, ebytes.astype(np.uint16))
    tiles = oracle.repack(MXFP4, flat, K, N)
    q, e = oracle.quantize_act_mx(inp.x)
    y_ref, acond = oracle.matmul_mx(tiles, K, N, q, e)
    qd, ed = tq.quantize_act_mx(torch.from_numpy(inp.x).cuda())
    out = torch.full((M, N + 16), 7.0, dtype=torch.float32, device="cuda")
    tq.qgemm_mx(torch.from_numpy(tiles).cuda(), K, N, qd, ed, out=out)
    got = out.cpu().numpy()
    assert (got[:, N:] == 7.0).all()                 # columns beyond N untouched
    return got[:, :N], y_ref, acond


@pytest.mark.parametrize("M", [1, 5, 128, 130, 300])
@pytest.mark.parametrize("K,N", [(32, 1), (96, 33), (256, 64), (1024, 97), (2048, 300),
                                 (4064, 65)])
def test_qgemm_mx_y(tq, M, K, N):
    got, y_ref, acond = mx_case(tq, M, K, N, seed=M * 7 + K + N)
    check_mx(got, y_ref, acond, ("mx", M, K, N), K)


def test_qgemm_mx_scale_edges(tq):
    """Rows whose E8M0 byte the page maps to 0 (e <= 112) contribute exactly
    nothing; e >= 142 saturates at 2^15 -- mixed with ordinary rows."""
    K, N, M = 256, 70, 40
    rng = np.random.default_rng(9)
    e = rng.integers(118, 125, (N, K // 32)).astype(np.uint8)
    e[0, :] = 0
    e[1, :] = 112
    e[2, ::2] = 113
    e[3, :] = 142
    e[4, :] = 200
    e[5, 1::3] = 255
    e[69, :] = 100
    got, y_ref, acond = mx_case(tq, M, K, N, seed=5, ebytes=e)
    assert (got[:, 0] == 0).all() and (got[:, 1] == 0).all() and (got[:, 69] == 0).all()
    check_mx(got, y_ref, acond, "mx scale edges", K)


def test_qgemm_mx_deterministic(tq):
    K, N, M = 1024, 200, 130
    inp = make(MXFP4, K, N, M, seed=1)
    tiles = torch.from_numpy(oracle.repack(MXFP4, inp.flat, K, N)).cuda()
    q, e = tq.quantize_act_mx(torch.from_numpy(inp.x).cuda())
    a = tq.qgemm_mx(tiles, K, N, q, e)
    b = tq.qgemm_mx(tiles, K, N, q, e)
    assert torch.equal(a, b)


def test_qgemm_mx_close_to_int8_path(tq):
    """The same MXFP4 tiles through the page's Q8_0 activations (tq_qgemm):
    both approximate the same real product, each within its activation
    rounding (E4M3 keeps 3 mantissa bits, so this is loose)."""
    K, N, M = 1024, 96, 64
    inp = make(MXFP4, K, N, M, seed=4)
    tiles = torch.from_numpy(oracle.repack(MXFP4, inp.flat, K, N)).cuda()
    x = torch.from_numpy(inp.x).cuda()
    q, e = tq.quantize_act_mx(x)
    y_mx = tq.qgemm_mx(tiles, K, N, q, e).cpu().numpy().astype(np.float64)
    q8, d8 = tq.quantize_act(x)
    y_i8 = tq.qgemm(MXFP4, tiles, K, N, q8, d8).cpu().numpy().astype(np.float64)
    assert np.linalg.norm(y_mx - y_i8) / np.linalg.norm(y_i8) < 0.1


# (K, N, M) with a small output grid: tq_matmul_mx splits K over 2 .. 8
# workgroups per output block (partial planes summed in a fixed order);
# K = 4160 (130 k-tiles) with S = 8 ranges of 24 leaves two ranges empty
SPLIT_SHAPES = [(4096, 4096, 128), (4096, 4096, 64), (1024, 300, 40), (2048, 1000, 130),
                (8192, 512, 200), (4096, 1000, 8), (512, 4096, 300), (4160, 4096, 8)]


@pytest.mark.parametrize("K,N,M", SPLIT_SHAPES)
def test_matmul_mx_split(tq, K, N, M):
    """tq_matmul_mx on its K split: within the bound (the split adds at most
    2 S fp32 additions of partial sums: S = 8 at most), bitwise repeatable,
    close to the unsplit tq_qgemm_mx, and the workspace's first 1 MiB (the
    decode split's zero-kept slots, shared through the per-stream
    workspace) still zero."""
    from block_quantized_matmul_repack_amd import ops
    inp = make(MXFP4, K, N, M, seed=K + N + M)
    tiles_ref = oracle.repack(MXFP4, inp.flat, K, N)
    qr, er = oracle.quantize_act_mx(inp.x)
    y_ref, acond = oracle.matmul_mx(tiles_ref, K, N, qr, er)
    tiles = torch.from_numpy(tiles_ref).cuda()
    q, e = tq.quantize_act_mx(torch.from_numpy(inp.x).cuda())
    need = tq.lib().tq_matmul_mx_workspace_bytes(K, N, M)
    out = torch.full((M, N + 8), 7.0, dtype=torch.float32, device="cuda")
    y = tq.matmul_mx(tiles, K, N, q, e, out=out[:, :N])
    got = out.cpu().numpy()
    assert (got[:, N:] == 7.0).all()
    check_mx(got[:, :N], y_ref, acond, ("matmul_mx", K, N, M, need), K, adds=16)
    y2 = tq.matmul_mx(tiles, K, N, q, e)
    assert torch.equal(y, y2), "not bitwise repeatable"
    y1 = tq.qgemm_mx(tiles, K, N, q, e)
    check_mx(y1.cpu().numpy(), y_ref, acond, ("qgemm_mx", K, N, M), K)
    torch.cuda.synchronize()
    assert all(int(torch.count_nonzero(ws[: 1 << 20])) == 0 for ws in ops._workspaces.values())


def test_matmul_mx_short_workspace_runs_unsplit(tq):
    """With less workspace than the split needs (or none), tq_matmul_mx runs
    the unsplit product: the same bits as tq_qgemm_mx."""
    import ctypes
    K, N, M = 4096, 4096, 64
    inp = make(MXFP4, K, N, M, seed=2)
    tiles = torch.from_numpy(oracle.repack(MXFP4, inp.flat, K, N)).cuda()
    q, e = tq.quantize_act_mx(torch.from_numpy(inp.x).cuda())
    need = tq.lib().tq_matmul_mx_workspace_bytes(K, N, M)
    assert need > (1 << 20)
    ref = tq.qgemm_mx(tiles, K, N, q, e)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    for ws_bytes in (need - 256, 0):
        ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
        y = torch.zeros((M, N), dtype=torch.float32, device="cuda")
        st = tq.lib().tq_matmul_mx(P(tiles), K, N, P(q), P(e), M, P(y), N,
                                   P(ws) if ws_bytes else None, ws_bytes, None)
        assert st == 0
        torch.cuda.synchronize()
        assert torch.equal(y, ref), ws_bytes


def test_matmul_mx_split_taken(tq):
    L = tq.lib()
    assert L.tq_matmul_mx_workspace_bytes(4096, 4096, 128) == (1 << 20) + 4 * 128 * 4096 * 4
    assert L.tq_matmul_mx_workspace_bytes(4096, 4096, 64) == (1 << 20) + 4 * 64 * 4096 * 4
    assert L.tq_matmul_mx_workspace_bytes(4096, 1000, 8) == (1 << 20) + 8 * 8 * 1000 * 4
    assert L.tq_matmul_mx_workspace_bytes(4096, 4096, 256) == 0
    assert L.tq_matmul_mx_workspace_bytes(4096, 4096, 512) == 0


def test_mx_empty_shapes(tq):
    t = torch.zeros(1088, dtype=torch.uint8, device="cuda")
    q = torch.zeros((0, 64), dtype=torch.uint8, device="cuda")
    e = torch.zeros((0, 2), dtype=torch.uint8, device="cuda")
    out = tq.qgemm_mx(t, 64, 32, q, e)
    assert out.shape == (0, 32)
    qq, ee = tq.quantize_act_mx(torch.zeros((0, 64), device="cuda"))
    assert qq.shape == (0, 64) and ee.shape == (0, 2)
