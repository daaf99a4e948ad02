"""GPU parity of the flat (un-repacked) path against the CPU oracle.

Page: "supports_op Independence from Buffer and Repack State" -- a supported
type must work tiled and flat.  Bit-exact: device unpack (tiles -> flat
blocks: the input flat bytes again) and the integer block dots of the flat
GEMV and GEMM kernels against the oracle's flat block dots.  fp32 y: within
the tolerance of gpu_helpers against the oracle's flat matmul, which equals
its tiled matmul exactly.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import check_y, make

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LUT = synth.IQ4_NL_STANDIN_LUT
TYPES = [synth.Q4_0, synth.Q8_0, synth.IQ4_NL, synth.MXFP4, synth.Q4_1, synth.Q4_K]


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_matmul_repack_amd as tq
    tq.lib()
    return tq


def _k(qtype, K):
    return max(256, K - K % 256) if qtype == synth.Q4_K else K


@pytest.mark.parametrize("qtype", TYPES[:5])
@pytest.mark.parametrize("K,N", [(32, 1), (96, 33), (512, 65), (4096, 100)])
@pytest.mark.parametrize("shift", [False, True])
def test_unpack_roundtrip(tq, qtype, K, N, shift):
    """Every byte of the flat buffer comes back, and nothing around it is
    written.  shift: the output starts at the smallest offset the type's
    alignment allows (2 or 4 bytes), so that each row's run of blocks is
    written with narrower stores than from an aligned start."""
    inp = make(qtype, K, N, 1, seed=K + N)
    tiles = torch.from_numpy(oracle.repack(qtype, inp.flat, K, N)).cuda()
    off = (4 if qtype in (synth.MXFP4, synth.Q4_1) else 2) if shift else 0
    out = torch.full((inp.flat.size + 64 + off,), 0xA5, dtype=torch.uint8, device="cuda")
    tq.unpack_tiles(qtype, tiles, K, N, out=out[off:off + inp.flat.size])
    got = out.cpu().numpy()
    bad = np.nonzero(got[off:off + inp.flat.size] != inp.flat)[0]
    assert bad.size == 0, [(int(b), int(got[off + b]), int(inp.flat[b])) for b in bad[:8]]
    assert (got[:off] == 0xA5).all() and (got[off + inp.flat.size:] == 0xA5).all()


@pytest.mark.parametrize("qtype", TYPES)
@pytest.mark.parametrize("M", [1, 3, 8, 9, 130])
@pytest.mark.parametrize("K,N", [(256, 1), (512, 33), (1024, 97), (4096, 70)])
def test_flat_products(tq, qtype, M, K, N):
    K = _k(qtype, K)
    inp = make(qtype, K, N, M, seed=M * 31 + K + N)
    q, d = oracle.quantize_act(inp.x)
    flat = torch.from_numpy(inp.flat).cuda()
    qd, dd = tq.quantize_act(torch.from_numpy(inp.x).cuda())
    ref = oracle.block_dots_flat(qtype, inp.flat, K, N, q, LUT)
    paths = [tq.PATH_GEMM_FLAT] + ([tq.PATH_GEMV_FLAT] if M <= 8 else [])
    for path in paths:
        got = tq.block_dots(qtype, flat, K, N, qd, lut=LUT, path=path).cpu().numpy()
        assert np.array_equal(got, ref), (path, np.argwhere(got != ref)[:4])
    y_ref, acond = oracle.matmul_flat(qtype, inp.flat, K, N, q, d, LUT)
    check_y(tq.matmul_flat(qtype, flat, K, N, qd, dd, lut=LUT).cpu().numpy(), y_ref, acond,
            ("flat", qtype, M, K, N))
    check_y(tq.qgemm_flat(qtype, flat, K, N, qd, dd, lut=LUT).cpu().numpy(), y_ref, acond,
            ("flat gemm", qtype, M, K, N))


@pytest.mark.parametrize("offset", [4, 8, 12])
def test_mxfp4_flat_at_every_phase(tq, offset):
    """17-byte blocks at shifted buffer starts, the buffer ending exactly at
    its last block: both flat kernels read every byte phase."""
    K, N, M = 96, 35, 2
    inp = make(synth.MXFP4, K, N, M, seed=offset)
    q, d = oracle.quantize_act(inp.x)
    big = torch.zeros(inp.flat.size + offset, dtype=torch.uint8, device="cuda")
    big[offset:] = torch.from_numpy(inp.flat).cuda()
    flat = big[offset:]
    qd = torch.from_numpy(q).cuda()
    ref = oracle.block_dots_flat(synth.MXFP4, inp.flat, K, N, q)
    for path in (tq.PATH_GEMV_FLAT, tq.PATH_GEMM_FLAT):
        assert np.array_equal(tq.block_dots(synth.MXFP4, flat, K, N, qd, path=path).cpu().numpy(), ref)


def test_flat_and_tiled_agree(tq):
    """The same weights tiled and flat: identical block dots, y within
    tolerance of each other's oracle (the oracle's are equal)."""
    for qtype in TYPES:
        K, N, M = 512, 64, 4
        inp = make(qtype, K, N, M, seed=qtype)
        flat = torch.from_numpy(inp.flat).cuda()
        tiles = tq.repack_tiles(qtype, flat, K, N)
        qd, _ = tq.quantize_act(torch.from_numpy(inp.x).cuda())
        a = tq.block_dots(qtype, tiles, K, N, qd, lut=LUT, path=tq.PATH_GEMV)
        b = tq.block_dots(qtype, flat, K, N, qd, lut=LUT, path=tq.PATH_GEMV_FLAT)
        assert torch.equal(a, b), qtype
