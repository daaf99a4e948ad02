"""The M dispatch through the C ABI: tq_matmul on every path it takes (one
decode launch, decode passes of 8 rows, the GEMM with K split over
workgroups, the plain GEMM) and tq_matmul_x (activations in: the fused
decode or quantize + tq_matmul), against the oracle.

The split GEMM adds its partial planes in a fixed order, so it is checked
for bitwise repeatability; its results differ from the unsplit GEMM's only
in the order of the fp32 sums (both within the tolerance of gpu_helpers).
The workspace's slot region (the decode split's zero-kept slots) must stay
zero after any sequence of calls that share it.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import check_y, make, to_dev_act

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TYPES = [synth.Q4_0, synth.Q8_0, synth.IQ4_NL, synth.MXFP4, synth.Q4_1]
LUT = synth.IQ4_NL_STANDIN_LUT


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_matmul_repack_amd as tq
    tq.lib()
    return tq


def _case(qtype, K, N, M, seed, act="f32"):
    inp = make(qtype, K, N, M, seed=seed, act=act)
    tiles_ref = oracle.repack(qtype, inp.flat, K, N)
    dt = {"f32": oracle.F32, "bf16": oracle.BF16, "f16": oracle.F16}[act]
    qr, dr = oracle.quantize_act(inp.x, dt)
    lut = LUT if qtype == synth.IQ4_NL else None
    y_ref, acond = oracle.matmul(qtype, tiles_ref, K, N, qr, dr, lut)
    return inp, tiles_ref, qr, dr, lut, y_ref, acond


def _dev(qr, dr):
    return (torch.from_numpy(qr).cuda(),
            torch.from_numpy(dr.view(np.int16)).cuda().view(torch.float16))


def slots_zero(tq):
    from block_quantized_matmul_repack_amd import ops
    torch.cuda.synchronize()
    return all(int(torch.count_nonzero(ws[: 1 << 20])) == 0 for ws in ops._workspaces.values())


# (K, N, M): shapes whose 128 x 64 output grid is small (split) or not;
# K = 4160 (130 k-tiles) with S = 8 ranges of 20 leaves the last range empty
# (it must write a zero plane)
SPLIT_SHAPES = [(4096, 4096, 16), (4096, 4096, 128), (1024, 300, 40), (2048, 97, 130),
                (512, 4096, 9), (4096, 1000, 64), (8192, 512, 200), (4160, 1000, 40)]


@pytest.mark.parametrize("qtype", TYPES)
@pytest.mark.parametrize("K,N,M", SPLIT_SHAPES)
def test_matmul_paths_match_oracle(tq, qtype, K, N, M):
    inp, tiles_ref, qr, dr, lut, y_ref, acond = _case(qtype, K, N, M, seed=K + N + M + qtype)
    tiles = torch.from_numpy(tiles_ref).cuda()
    q, d = _dev(qr, dr)
    path = tq.matmul_path(qtype, K, N, M)
    out = torch.full((M, N + 8), 5.0, dtype=torch.float32, device="cuda")
    y = tq.matmul(qtype, tiles, K, N, q, d, lut=lut, out=out[:, :N])
    got = out.cpu().numpy()
    assert (got[:, N:] == 5.0).all()                 # columns past N untouched
    check_y(got[:, :N], y_ref, acond, ("matmul", qtype, K, N, M, path))
    y2 = tq.matmul(qtype, tiles, K, N, q, d, lut=lut)
    assert torch.equal(y, y2), "not bitwise repeatable"
    yg = tq.qgemm(qtype, tiles, K, N, q, d, lut=lut).cpu().numpy()
    check_y(yg, y_ref, acond, ("qgemm", qtype, K, N, M))
    assert slots_zero(tq)


def test_split_paths_are_taken(tq):
    assert tq.matmul_path(synth.Q4_0, 4096, 4096, 128) == tq.PATH_GEMM_SPLIT
    assert tq.matmul_path(synth.Q4_0, 4096, 4096, 512) == tq.PATH_GEMM
    assert tq.matmul_path(synth.Q4_0, 4096, 4096, 8) == tq.PATH_GEMV


def test_shared_workspace_across_shapes(tq):
    """A split GEMM writes its planes into the workspace's scratch; a decode
    of another shape with many split slots then runs on the same workspace
    (the binding keeps one per stream) and must still be exact."""
    # the split GEMM first (largest planes), then a decode with S = 4 over
    # 127 stripes (slots for 8 rows: 780,288 bytes)
    a = _case(synth.Q8_0, 4096, 4096, 128, seed=3)
    b = _case(synth.Q8_0, 4096, 4064, 8, seed=4)
    for (inp, tiles_ref, qr, dr, lut, y_ref, acond), K, N in ((a, 4096, 4096), (b, 4096, 4064),
                                                             (a, 4096, 4096), (b, 4096, 4064)):
        q, d = _dev(qr, dr)
        y = tq.matmul(synth.Q8_0, torch.from_numpy(tiles_ref).cuda(), K, N, q, d)
        check_y(y.cpu().numpy(), y_ref, acond, ("shared ws", N))
    assert slots_zero(tq)


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("qtype", [synth.Q4_0, synth.Q8_0, synth.IQ4_NL])
@pytest.mark.parametrize("K,N,M", [(4096, 4096, 1), (4096, 4096, 8), (1024, 14336, 4),
                                   (1024, 14336, 1), (2048, 1000, 12), (1024, 4096, 130),
                                   (512, 300, 300)])
def test_matmul_x(tq, act, qtype, K, N, M):
    inp, tiles_ref, qr, dr, lut, y_ref, acond = _case(qtype, K, N, M, seed=7 * M + N, act=act)
    tiles = torch.from_numpy(tiles_ref).cuda()
    x = to_dev_act(inp.x, act)
    y = tq.matmul_x(qtype, tiles, K, N, x, lut=lut)
    check_y(y.cpu().numpy(), y_ref, acond, ("matmul_x", act, qtype, K, N, M))
    # the same as quantize_act + matmul, bit for bit
    q, d = tq.quantize_act(x)
    assert np.array_equal(q.cpu().numpy(), qr)
    y2 = tq.matmul(qtype, tiles, K, N, q, d, lut=lut) if M > 8 else None
    if y2 is not None:
        assert torch.equal(y, y2)
    assert slots_zero(tq)


def test_matmul_x_rejects_short_workspace(tq):
    from block_quantized_matmul_repack_amd import TiledqError
    from block_quantized_matmul_repack_amd._lib import lib
    import ctypes
    K, N, M = 1024, 4096, 40
    inp, tiles_ref, *_ = _case(synth.Q4_0, K, N, M, seed=1)
    tiles = torch.from_numpy(tiles_ref).cuda()
    x = torch.from_numpy(inp.x).cuda()
    y = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    need = lib().tq_matmul_x_workspace_bytes(synth.Q4_0, K, N, M)
    assert need > (1 << 20)
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    st = lib().tq_matmul_x(synth.Q4_0, ctypes.c_void_p(tiles.data_ptr()), K, N, 0,
                           ctypes.c_void_p(x.data_ptr()), K, M, None,
                           ctypes.c_void_p(y.data_ptr()), N, ctypes.c_void_p(ws.data_ptr()),
                           ws.numel(), None)
    assert st == 3                                     # TQ_E_SHAPE, nothing launched
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(y)) == 0
