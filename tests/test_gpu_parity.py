"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bit-exact: repack bytes, quantized activations and scales, per-block integer
dots of both the GEMV and the GEMM kernel.  fp32 outputs: within the
tolerance stated in gpu_helpers (1e-3 relative with a cancellation floor).
Shapes span several tiles and ragged tails; all inputs are seeded.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import check_y, make, tiles_slice, to_dev_act

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

Q4_0, Q8_0, IQ4_NL, MXFP4, Q4_1 = synth.Q4_0, synth.Q8_0, synth.IQ4_NL, synth.MXFP4, synth.Q4_1
Q4_K = synth.Q4_K
TYPES = [Q4_0, Q8_0, IQ4_NL, MXFP4, Q4_1]
LUT = synth.IQ4_NL_STANDIN_LUT


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_matmul_repack_amd as tq
    tq.lib()
    return tq


SHAPES = [(32, 1), (64, 31), (96, 33), (256, 64), (512, 65), (1024, 100), (4096, 97)]


@pytest.mark.parametrize("qtype", TYPES)
@pytest.mark.parametrize("K,N", SHAPES)
def test_repack_bitexact(tq, qtype, K, N):
    inp = make(qtype, K, N, 1, seed=K * 7 + N)
    ref = oracle.repack(qtype, inp.flat, K, N)
    flat = torch.from_numpy(inp.flat).cuda()
    out = torch.full((ref.size + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    tq.repack_tiles(qtype, flat, K, N, out=out[:ref.size])
    got = out.cpu().numpy()
    assert np.array_equal(got[:ref.size], ref)
    assert (got[ref.size:] == 0xA5).all()          # guard band untouched


@pytest.mark.parametrize("act", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("M,K", [(1, 32), (3, 256), (8, 4096), (37, 1024)])
def test_quantize_bitexact(tq, act, M, K):
    inp = make(Q8_0, K, 1, M, seed=M * 1000 + K, act=act)
    x = inp.x.copy()
    if act == "f32":
        x[0, :32] = 0.0
        if K >= 64:
            x[0, 32:64] = 0.25
            x[0, 32] = 127.0
            x[0, 33:40] = [2.5, -2.5, 0.5, -0.5, 1.5, 126.5, -126.5]
    dt = {"f32": oracle.F32, "bf16": oracle.BF16, "f16": oracle.F16}[act]
    qr, dr = oracle.quantize_act(x, dt)
    q, d = tq.quantize_act(to_dev_act(x, act))
    assert np.array_equal(q.cpu().numpy(), qr)
    assert np.array_equal(d.cpu().view(torch.int16).numpy().view(np.uint16), dr)


def test_quantize_row_stride(tq):
    inp = make(Q8_0, 256, 1, 5, seed=3)
    wide = np.concatenate([inp.x, np.full((5, 64), 9e5, np.float32)], axis=1)
    qr, dr = oracle.quantize_act(wide, oracle.F32, K=256)
    q, d = tq.quantize_act(torch.from_numpy(wide).cuda(), K=256)
    assert np.array_equal(q.cpu().numpy(), qr)
    assert np.array_equal(d.cpu().view(torch.int16).numpy().view(np.uint16), dr)


def _dev(inp, qtype, K, N):
    tiles = oracle.repack(qtype, inp.flat, K, N)
    return tiles, torch.from_numpy(tiles).cuda()


@pytest.mark.parametrize("qtype", TYPES)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("K,N", [(64, 33), (512, 100), (4096, 64)])
def test_block_dots_gemv(tq, qtype, M, K, N):
    inp = make(qtype, K, N, M, seed=M + 10 * K + N)
    tiles, tdev = _dev(inp, qtype, K, N)
    q, _ = oracle.quantize_act(inp.x)
    ref = oracle.block_dots(qtype, tiles, K, N, q, LUT)
    got = tq.block_dots(qtype, tdev, K, N, torch.from_numpy(q).cuda(), lut=LUT,
                        path=tq.PATH_GEMV).cpu().numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("qtype", TYPES)
@pytest.mark.parametrize("M", [1, 8, 33, 130])
@pytest.mark.parametrize("K,N", [(64, 33), (512, 100), (1024, 129)])
def test_block_dots_gemm(tq, qtype, M, K, N):
    inp = make(qtype, K, N, M, seed=M + 10 * K + N + 1)
    tiles, tdev = _dev(inp, qtype, K, N)
    q, _ = oracle.quantize_act(inp.x)
    ref = oracle.block_dots(qtype, tiles, K, N, q, LUT)
    got = tq.block_dots(qtype, tdev, K, N, torch.from_numpy(q).cuda(), lut=LUT,
                        path=tq.PATH_GEMM).cpu().numpy()
    assert np.array_equal(got, ref)


def _y_case(tq, fn, qtype, M, K, N, seed):
    inp = make(qtype, K, N, M, seed=seed)
    tiles, tdev = _dev(inp, qtype, K, N)
    q, d = oracle.quantize_act(inp.x)
    y_ref, acond = oracle.matmul(qtype, tiles, K, N, q, d, LUT)
    qd, dd = tq.quantize_act(torch.from_numpy(inp.x).cuda())
    out = torch.full((M, N + 16), 7.0, dtype=torch.float32, device="cuda")
    fn(qtype, tdev, K, N, qd, dd, lut=LUT, out=out)
    got = out.cpu().numpy()
    assert (got[:, N:] == 7.0).all()               # columns beyond N untouched
    return check_y(got[:, :N], y_ref, acond, (qtype, M, K, N))


@pytest.mark.parametrize("qtype", TYPES)
@pytest.mark.parametrize("M", [1, 4, 8])
@pytest.mark.parametrize("K,N", [(256, 64), (1024, 97), (4096, 300)])
def test_qgemv_y(tq, qtype, M, K, N):
    _y_case(tq, tq.qgemv, qtype, M, K, N, seed=M * 3 + K + N)


@pytest.mark.parametrize("qtype", TYPES)
@pytest.mark.parametrize("M", [1, 9, 128, 200])
@pytest.mark.parametrize("K,N", [(256, 64), (1024, 97), (2048, 300)])
def test_qgemm_y(tq, qtype, M, K, N):
    _y_case(tq, tq.qgemm, qtype, M, K, N, seed=M * 5 + K + N)


# K whose k-blocks do not fill the GEMM's 4-block steps (5, 12 and 13
# blocks: an odd step count, a padded last step, a last step of one block),
# with row counts that end inside a 32-row sub-block and inside a 128-row
# block; y and the block dots of the GEMM.
@pytest.mark.parametrize("qtype", TYPES)
@pytest.mark.parametrize("M", [7, 129])
@pytest.mark.parametrize("K,N", [(160, 40), (384, 96), (416, 65)])
def test_qgemm_y_partial_steps(tq, qtype, M, K, N):
    _y_case(tq, tq.qgemm, qtype, M, K, N, seed=M * 11 + K + N)


@pytest.mark.parametrize("qtype", TYPES)
@pytest.mark.parametrize("M", [7, 129])
@pytest.mark.parametrize("K,N", [(160, 40), (416, 65)])
def test_block_dots_gemm_partial_steps(tq, qtype, M, K, N):
    inp = make(qtype, K, N, M, seed=M * 13 + K + N)
    tiles, tdev = _dev(inp, qtype, K, N)
    q, _ = oracle.quantize_act(inp.x)
    ref = oracle.block_dots(qtype, tiles, K, N, q, LUT)
    got = tq.block_dots(qtype, tdev, K, N, torch.from_numpy(q).cuda(), lut=LUT,
                        path=tq.PATH_GEMM).cpu().numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("qtype", TYPES)
def test_gemv_gemm_agree(tq, qtype):
    K, N, M = 1024, 130, 8
    inp = make(qtype, K, N, M, seed=99)
    _, tdev = _dev(inp, qtype, K, N)
    qd, dd = tq.quantize_act(torch.from_numpy(inp.x).cuda())
    b1 = tq.block_dots(qtype, tdev, K, N, qd, lut=LUT, path=tq.PATH_GEMV)
    b2 = tq.block_dots(qtype, tdev, K, N, qd, lut=LUT, path=tq.PATH_GEMM)
    assert torch.equal(b1, b2)
    y1 = tq.qgemv(qtype, tdev, K, N, qd, dd, lut=LUT)
    y2 = tq.qgemm(qtype, tdev, K, N, qd, dd, lut=LUT)
    assert torch.allclose(y1, y2, rtol=1e-5, atol=1e-6 * float(y1.abs().max()))


@pytest.mark.parametrize("fn", ["qgemv", "qgemm"])
def test_deterministic(tq, fn):
    K, N, M = 2048, 200, 4
    inp = make(Q4_0, K, N, M, seed=5)
    _, tdev = _dev(inp, Q4_0, K, N)
    qd, dd = tq.quantize_act(torch.from_numpy(inp.x).cuda())
    f = getattr(tq, fn)
    y1 = f(Q4_0, tdev, K, N, qd, dd)
    y2 = f(Q4_0, tdev, K, N, qd, dd)
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


def test_iq4_identity_table_equals_q4_0(tq):
    K, N, M = 512, 70, 3
    inp = make(Q4_0, K, N, M, seed=8)
    _, tdev = _dev(inp, Q4_0, K, N)
    qd, dd = tq.quantize_act(torch.from_numpy(inp.x).cuda())
    ident = np.arange(16, dtype=np.int8) - 8
    for f in (tq.qgemv, tq.qgemm):
        assert torch.equal(f(Q4_0, tdev, K, N, qd, dd), f(IQ4_NL, tdev, K, N, qd, dd, lut=ident))


def test_empty_shapes_are_noops(tq):
    q = torch.zeros((1, 64), dtype=torch.int8, device="cuda")
    d = torch.zeros((1, 2), dtype=torch.float16, device="cuda")
    t = torch.zeros(0, dtype=torch.uint8, device="cuda")
    y = tq.qgemv(Q4_0, t, 64, 0, q, d)
    assert y.shape == (1, 0)
    y = tq.qgemm(Q4_0, t, 64, 0, q, d)
    assert y.shape == (1, 0)
    torch.cuda.synchronize()


@pytest.mark.parametrize("qtype", TYPES)
@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("K,N", [(96, 40), (160, 300), (4064, 33), (2048, 1), (4096, 4096)])
def test_qgemv_split_and_unsplit(tq, qtype, M, K, N):
    """K split across workgroups (workspace) and one workgroup per stripe both
    meet the tolerance and are each bitwise repeatable."""
    inp = make(qtype, K, N, M, seed=M * 7 + K + N)
    tiles, tdev = _dev(inp, qtype, K, N)
    q, d = oracle.quantize_act(inp.x)
    y_ref, acond = oracle.matmul(qtype, tiles, K, N, q, d, LUT)
    qd, dd = tq.quantize_act(torch.from_numpy(inp.x).cuda())
    for split in (True, False):
        y1 = tq.qgemv(qtype, tdev, K, N, qd, dd, lut=LUT, split=split)
        y2 = tq.qgemv(qtype, tdev, K, N, qd, dd, lut=LUT, split=split)
        assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
        check_y(y1.cpu().numpy(), y_ref, acond, (qtype, M, K, N, split))
    ref = oracle.block_dots(qtype, tiles, K, N, q, LUT)
    got = tq.block_dots(qtype, tdev, K, N, qd, lut=LUT, path=tq.PATH_GEMV).cpu().numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("qtype", TYPES)
@pytest.mark.parametrize("M", [2, 5, 6, 7])
@pytest.mark.parametrize("K,N", [(2048, 96), (4064, 33)])
def test_qgemv_every_row_count(tq, qtype, M, K, N):
    """Row counts between the ones above, with many tiles per workgroup
    (split and unsplit): for 4-bit tiles these take the matrix-core path,
    where rows 4..7 come from the second half of the wave."""
    inp = make(qtype, K, N, M, seed=M * 11 + K + N)
    tiles, tdev = _dev(inp, qtype, K, N)
    q, d = oracle.quantize_act(inp.x)
    y_ref, acond = oracle.matmul(qtype, tiles, K, N, q, d, LUT)
    qd, dd = tq.quantize_act(torch.from_numpy(inp.x).cuda())
    for split in (True, False):
        y = tq.qgemv(qtype, tdev, K, N, qd, dd, lut=LUT, split=split)
        check_y(y.cpu().numpy(), y_ref, acond, (qtype, M, K, N, split))
    yx = tq.qgemv_x(qtype, tdev, K, N, torch.from_numpy(inp.x).cuda(), lut=LUT)
    check_y(yx.cpu().numpy(), y_ref, acond, (qtype, M, K, N, "fused"))


@pytest.mark.parametrize("qtype", TYPES)
@pytest.mark.parametrize("M,K", [(1, 20480), (2, 9216), (4, 9216), (5, 9216), (8, 9216),
                                 (8, 4544)])
def test_qgemv_long_passes(tq, qtype, M, K):
    """One workgroup per stripe over 142 to 640 k-tiles: a staging pass of
    the int8 activations then holds more chunks and scales than the loads
    issued ahead of the weight stream cover (128 tiles at M = 4 and 8, 256
    at M = 1 and 512 for M = 1's scales), so the trailing staging loops run,
    and at M >= 2 several passes follow each other.  Block dots bit for bit;
    y unsplit, split and fused within tolerance."""
    N = 40
    inp = make(qtype, K, N, M, seed=M * 13 + K)
    tiles, tdev = _dev(inp, qtype, K, N)
    q, d = oracle.quantize_act(inp.x)
    y_ref, acond = oracle.matmul(qtype, tiles, K, N, q, d, LUT)
    qd, dd = tq.quantize_act(torch.from_numpy(inp.x).cuda())
    for split in (False, True):
        y = tq.qgemv(qtype, tdev, K, N, qd, dd, lut=LUT, split=split)
        check_y(y.cpu().numpy(), y_ref, acond, (qtype, M, K, N, split))
    yx = tq.qgemv_x(qtype, tdev, K, N, torch.from_numpy(inp.x).cuda(), lut=LUT, split=False)
    check_y(yx.cpu().numpy(), y_ref, acond, (qtype, M, K, N, "fused"))
    ref = oracle.block_dots(qtype, tiles, K, N, q, LUT)
    got = tq.block_dots(qtype, tdev, K, N, qd, lut=LUT, path=tq.PATH_GEMV).cpu().numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("qtype", TYPES)
@pytest.mark.parametrize("M", [1, 8, 9, 13, 16, 17, 40, 49])
@pytest.mark.parametrize("K,N", [(512, 100), (4096, 300)])
def test_matmul_dispatch(tq, qtype, M, K, N):
    """tq_matmul is bitwise the GEMV for M <= 8, one GEMV pass per 8 rows
    where matmul_path picks the decode passes, bitwise the GEMM where it picks
    the GEMM, and bitwise repeatable on the split GEMM (whose fp32 sums run in
    another order than the unsplit GEMM's); each within the tolerance of the
    oracle."""
    inp = make(qtype, K, N, M, seed=M + 3 + K)
    tiles, tdev = _dev(inp, qtype, K, N)
    q, d = oracle.quantize_act(inp.x)
    qd, dd = tq.quantize_act(torch.from_numpy(inp.x).cuda())
    y = tq.matmul(qtype, tdev, K, N, qd, dd, lut=LUT)
    path = tq.matmul_path(qtype, K, N, M)
    assert path in (tq.PATH_GEMV, tq.PATH_GEMM, tq.PATH_GEMM_SPLIT)
    assert (path == tq.PATH_GEMV) if M <= 8 else True
    if path == tq.PATH_GEMV:
        ref = torch.cat([tq.qgemv(qtype, tdev, K, N, qd[i:i + 8], dd[i:i + 8], lut=LUT)
                         for i in range(0, M, 8)])
    elif path == tq.PATH_GEMM:
        ref = tq.qgemm(qtype, tdev, K, N, qd, dd, lut=LUT)
    else:
        ref = tq.matmul(qtype, tdev, K, N, qd, dd, lut=LUT)
    assert torch.equal(y.view(torch.int32), ref.view(torch.int32))
    y_ref, acond = oracle.matmul(qtype, tiles, K, N, q, d, LUT)
    check_y(y.cpu().numpy(), y_ref, acond, (qtype, M, K, N))


def test_qgemv_workspace_reused_across_shapes(tq):
    """One workspace serves calls of different shapes in a row (its counter
    and partial offsets depend on the shape): every call must leave it zero."""
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    L = tq.lib()
    import ctypes
    for (K, N) in [(4096, 2048), (2048, 4096), (4096, 4096), (1024, 100), (4096, 4096)]:
        inp = make(Q4_0, K, N, 1, seed=K + N)
        tiles, tdev = _dev(inp, Q4_0, K, N)
        q, d = oracle.quantize_act(inp.x)
        y_ref, acond = oracle.matmul(Q4_0, tiles, K, N, q, d)
        qd, dd = tq.quantize_act(torch.from_numpy(inp.x).cuda())
        y = torch.full((1, N), float("nan"), device="cuda")
        need = L.tq_qgemv_workspace_bytes(Q4_0, K, N, 1)
        assert 0 < need <= ws.numel()
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        assert L.tq_qgemv(Q4_0, ctypes.c_void_p(tdev.data_ptr()), K, N, ctypes.c_void_p(qd.data_ptr()),
                          ctypes.c_void_p(dd.data_ptr()), 1, None, ctypes.c_void_p(y.data_ptr()), N,
                          ctypes.c_void_p(ws.data_ptr()), ws.numel(), st) == 0
        check_y(y.cpu().numpy(), y_ref, acond, (K, N))
        assert int(ws.count_nonzero()) == 0


@pytest.mark.parametrize("qtype", TYPES)
@pytest.mark.parametrize("act", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("M,K,N", [(1, 4096, 4096), (3, 96, 40), (8, 1024, 300), (5, 4064, 33)])
def test_qgemv_x_equals_two_launches(tq, qtype, act, M, K, N):
    """Quantize fused into the GEMV gives bit-identical y (same arithmetic),
    with and without the K split, and meets the oracle's tolerance."""
    inp = make(qtype, K, N, M, seed=M + K + N + len(act), act=act)
    tiles, tdev = _dev(inp, qtype, K, N)
    x = to_dev_act(inp.x, act)
    for split in (True, False):
        qd, dd = tq.quantize_act(x)
        y2 = tq.qgemv(qtype, tdev, K, N, qd, dd, lut=LUT, split=split)
        y1 = tq.qgemv_x(qtype, tdev, K, N, x, lut=LUT, split=split)
        assert torch.equal(y1.view(torch.int32), y2.view(torch.int32)), (split,)
    dt = {"f32": oracle.F32, "bf16": oracle.BF16, "f16": oracle.F16}[act]
    q, d = oracle.quantize_act(inp.x, dt)
    y_ref, acond = oracle.matmul(qtype, tiles, K, N, q, d, LUT)
    check_y(y1.cpu().numpy(), y_ref, acond, (qtype, act, M, K, N))


def test_qgemv_x_row_stride(tq):
    K, N, M = 512, 64, 2
    inp = make(Q8_0, K, N, M, seed=77)
    _, tdev = _dev(inp, Q8_0, K, N)
    wide = torch.from_numpy(np.concatenate([inp.x, np.full((M, 64), 9e5, np.float32)], 1)).cuda()
    y1 = tq.qgemv_x(Q8_0, tdev, K, N, wide[:, :K])
    qd, dd = tq.quantize_act(torch.from_numpy(inp.x).cuda())
    y2 = tq.qgemv(Q8_0, tdev, K, N, qd, dd)
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("offset", [4, 8, 12])
def test_mxfp4_repack_flat_offsets(tq, offset):
    """17-byte MXFP4 blocks start at every byte phase; moving the whole flat
    buffer by 4..12 bytes changes the phase of every dword the kernel reads,
    and the buffer ends exactly at its last block."""
    K, N = 96, 35
    inp = make(MXFP4, K, N, 1, seed=offset)
    ref = oracle.repack(MXFP4, inp.flat, K, N)
    big = torch.zeros(inp.flat.size + offset, dtype=torch.uint8, device="cuda")
    big[offset:] = torch.from_numpy(inp.flat).cuda()
    got = tq.repack_tiles(MXFP4, big[offset:], K, N).cpu().numpy()
    assert np.array_equal(got, ref)


def test_mxfp4_every_scale_byte(tq):
    """Every E8M0 byte 0..255 (the zero, normal and clamped ranges) and every
    code, through both kernels: block dots bit-exact, y within tolerance."""
    K, N, M = 64, 256, 3
    rng = np.random.default_rng(17)
    codes = synth.draw_codes(rng, MXFP4, N, K)
    e = np.stack([np.arange(256), np.arange(256)[::-1]], axis=1).astype(np.uint16)
    flat = synth.pack_flat(MXFP4, codes, e)
    x = synth.draw_activations(rng, M, K)
    tiles = oracle.repack(MXFP4, flat, K, N)
    q, d = oracle.quantize_act(x)
    tdev = tq.repack_tiles(MXFP4, torch.from_numpy(flat).cuda(), K, N)
    assert np.array_equal(tdev.cpu().numpy(), tiles)
    qd, dd = tq.quantize_act(torch.from_numpy(x).cuda())
    ref = oracle.block_dots(MXFP4, tiles, K, N, q)
    y_ref, acond = oracle.matmul(MXFP4, tiles, K, N, q, d)
    for path, fn in ((tq.PATH_GEMV, tq.qgemv), (tq.PATH_GEMM, tq.qgemm)):
        got = tq.block_dots(MXFP4, tdev, K, N, qd, path=path).cpu().numpy()
        assert np.array_equal(got, ref), path
        y = fn(MXFP4, tdev, K, N, qd, dd).cpu().numpy()
        check_y(y, y_ref, acond, ("mxfp4 scales", path))


@pytest.mark.parametrize("M", [1, 3, 8, 40, 130])
def test_q4_1_min_term(tq, M):
    """Q4_1 with all codes 0 is the min term alone (m * da * sum(q) per
    block); with large activations the block sums reach +-4064.  Both
    kernels, and the fused decode, against the oracle."""
    K, N = 320, 70
    rng = np.random.default_rng(M)
    codes = np.zeros((N, K), np.uint8)
    codes[:, ::7] = 15
    pairs = synth.draw_scales(rng, "minmax", N, K)
    flat = synth.pack_flat(Q4_1, codes, pairs)
    x = synth.draw_activations(rng, M, K)
    x[:, :64] = np.abs(x[:, :64]) + 3.0          # blocks 0, 1: all of one sign
    x[0, 64:96] = -1.0                            # block 2 of row 0: q = -127 throughout
    tiles = oracle.repack(Q4_1, flat, K, N)
    q, d = oracle.quantize_act(x)
    assert q[0, 64:96].sum() == -127 * 32
    y_ref, acond = oracle.matmul(Q4_1, tiles, K, N, q, d)
    tdev = tq.repack_tiles(Q4_1, torch.from_numpy(flat).cuda(), K, N)
    assert np.array_equal(tdev.cpu().numpy(), tiles)
    qd, dd = tq.quantize_act(torch.from_numpy(x).cuda())
    fns = [tq.qgemm] + ([tq.qgemv] if M <= 8 else [])
    for fn in fns:
        check_y(fn(Q4_1, tdev, K, N, qd, dd).cpu().numpy(), y_ref, acond, ("q4_1 min", fn.__name__, M))
    if M <= 8:
        yx = tq.qgemv_x(Q4_1, tdev, K, N, torch.from_numpy(x).cuda())
        check_y(yx.cpu().numpy(), y_ref, acond, ("q4_1 min fused", M))


Q4K_SHAPES = [(256, 1), (256, 33), (512, 65), (1024, 97), (4096, 100)]


@pytest.mark.parametrize("K,N", Q4K_SHAPES)
def test_q4_k_repack_bitexact(tq, K, N):
    """Q4_K super-blocks -> tiles: quant bytes and the fp16 pair products."""
    inp = make(Q4_K, K, N, 1, seed=K + N)
    ref = oracle.repack(Q4_K, inp.flat, K, N)
    out = torch.full((ref.size + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    tq.repack_tiles(Q4_K, torch.from_numpy(inp.flat).cuda(), K, N, out=out[:ref.size])
    got = out.cpu().numpy()
    bad = np.nonzero(got[:ref.size] != ref)[0]
    assert bad.size == 0, [(int(b) // 640, int(b) % 640, int(got[b]), int(ref[b])) for b in bad[:12]]
    assert (got[ref.size:] == 0xA5).all()


def test_q4_k_extreme_scales(tq):
    """All 6-bit scale / min values, d and dmin from subnormal to large and of
    either sign, zeros included (the fp16 products round, overflow to inf,
    or are zeros of either sign)."""
    K, N = 256, 64
    rng = np.random.default_rng(5)
    codes = synth.draw_codes(rng, Q4_K, N, K)
    p = synth.draw_scales(rng, "q4k", N, K)
    p.sc[:] = np.arange(N * 8).reshape(N, 8) % 64
    p.m[:] = (np.arange(N * 8).reshape(N, 8) * 5) % 64
    vals = np.array([2.0 ** -24, 6.1e-5, 0.0999, 1.0, 1000.0, 2000.0, 65504.0, 0.0,
                     -0.0, -1.0, -0.375, -2.0 ** -20], np.float16)
    p.d[:, 0] = vals[np.arange(N) % len(vals)].view(np.uint16)
    p.dmin[:, 0] = vals[(np.arange(N) * 5) % len(vals)].view(np.uint16)
    flat = synth.pack_flat(Q4_K, codes, p)
    ref = oracle.repack(Q4_K, flat, K, N)
    got = tq.repack_tiles(Q4_K, torch.from_numpy(flat).cuda(), K, N).cpu().numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("M", [1, 3, 8, 9, 130])
@pytest.mark.parametrize("K,N", [(256, 33), (1024, 97), (4096, 100)])
def test_q4_k_products(tq, M, K, N):
    """Block dots (both kernels) bit-exact, y within tolerance, fused decode."""
    inp = make(Q4_K, K, N, M, seed=M * 17 + K + N)
    tiles, tdev = _dev(inp, Q4_K, K, N)
    q, d = oracle.quantize_act(inp.x)
    qd, dd = tq.quantize_act(torch.from_numpy(inp.x).cuda())
    ref = oracle.block_dots(Q4_K, tiles, K, N, q)
    paths = [tq.PATH_GEMM] + ([tq.PATH_GEMV] if M <= 8 else [])
    for path in paths:
        got = tq.block_dots(Q4_K, tdev, K, N, qd, path=path).cpu().numpy()
        assert np.array_equal(got, ref), path
    y_ref, acond = oracle.matmul(Q4_K, tiles, K, N, q, d)
    check_y(tq.matmul(Q4_K, tdev, K, N, qd, dd).cpu().numpy(), y_ref, acond, ("q4_k", M, K, N))
    check_y(tq.qgemm(Q4_K, tdev, K, N, qd, dd).cpu().numpy(), y_ref, acond, ("q4_k gemm", M, K, N))
    if M <= 8:
        yx = tq.qgemv_x(Q4_K, tdev, K, N, torch.from_numpy(inp.x).cuda())
        check_y(yx.cpu().numpy(), y_ref, acond, ("q4_k fused", M, K, N))
