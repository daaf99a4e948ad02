"""GPU parity at the edges of the documented domains, against the oracle.

- Activation quantization (tq_quantize_act and the quantization inside the
  fused decode, tq_qgemv_x) on blocks whose maximum sits at the domain's
  ends: amax = 2^-120 and just above, amax = 127 * 2^-126 (the smallest
  normal fp32 d) and just below (a subnormal fp32 d), maxima whose stored
  fp16 d is an fp16 subnormal or rounds to +0, subnormal fp32 / bf16 / fp16
  inputs, signed zeros, exact half-way products, and the upper end
  amax = 65504 * 127 -- q and d bit for bit.
- Q8_0 weights over the whole int8 range: code -128 against activation codes
  +-127, up to the extreme block dot 32 * 128 * 127, through every kernel
  that reads Q8_0 weights (decode on v_dot4 for M <= 4 and on the matrix
  cores from M = 5, the GEMM, the flat decode and flat GEMM) -- block dots
  bit for bit, y within the tolerance of gpu_helpers.
- One-block products (K = 32) with fp16 subnormal and zero weight scales and
  the edge activations: each output is then one rounding of an exact value,
  fp32(isum * fp32(dw * da)), so y must match bit for bit.  This also shows
  that fp16 subnormal scales keep their value inside every kernel.

All inputs come from the seeded generators in synth.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import check_y, to_dev_act

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

Q4_0, Q8_0, IQ4_NL, MXFP4 = synth.Q4_0, synth.Q8_0, synth.IQ4_NL, synth.MXFP4
LUT = synth.IQ4_NL_STANDIN_LUT
_DT = {"f32": oracle.F32, "bf16": oracle.BF16, "f16": oracle.F16}


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_matmul_repack_amd as tq
    tq.lib()
    return tq


def _bits(d):
    return d.cpu().view(torch.int16).numpy().view(np.uint16)


def edge_x(M, K, act, seed):
    return synth.draw_edge_activations(np.random.default_rng(seed), M, K, act)


@pytest.mark.parametrize("act", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("M,K", [(1, 512), (3, 512), (8, 1024), (13, 2048)])
def test_quantize_edges_bitexact(tq, act, M, K):
    x = edge_x(M, K, act, seed=M * 31 + K)
    qr, dr = oracle.quantize_act(x, _DT[act])
    d16 = oracle.f16_to_f32_array(dr)
    assert np.isfinite(d16).all()
    # the generator reaches the edges it is meant to: fp16-subnormal and
    # zero-rounded stored scales beside nonzero codes
    nz = np.abs(qr.reshape(M, -1, 32)).max(axis=2) > 0
    assert ((dr & 0x7C00) == 0)[nz].any()
    q, d = tq.quantize_act(to_dev_act(x, act))
    assert np.array_equal(q.cpu().numpy(), qr)
    assert np.array_equal(_bits(d), dr)


def _tiles(qtype, K, N, seed, dist=None, q8_full=False):
    rng = np.random.default_rng(seed)
    if q8_full:
        codes = synth.draw_codes_q8_full(rng, N, K)
    else:
        codes = synth.draw_codes(rng, qtype, N, K)
    dist = dist or {Q8_0: "absnormal", MXFP4: "e8m0"}.get(qtype, "uniform")
    sb = synth.draw_scales(rng, dist, N, K)
    flat = synth.pack_flat(qtype, codes, sb)
    return flat, oracle.repack(qtype, flat, K, N)


@pytest.mark.parametrize("act", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
@pytest.mark.parametrize("M", [1, 4, 5, 8])
def test_fused_decode_edges(tq, act, qtype, M):
    """tq_qgemv_x quantizes inside the decode kernel: bit-identical y to
    tq_quantize_act + tq_qgemv (both split modes), and y within tolerance
    of the oracle."""
    K, N = 1024, 96
    x = edge_x(M, K, act, seed=M * 17 + qtype)
    flat, tiles_ref = _tiles(qtype, K, N, seed=M + 100 * qtype, q8_full=qtype == Q8_0)
    tiles = torch.from_numpy(tiles_ref).cuda()
    xd = to_dev_act(x, act)
    qr, dr = oracle.quantize_act(x, _DT[act])
    y_ref, acond = oracle.matmul(qtype, tiles_ref, K, N, qr, dr)
    for split in (True, False):
        y1 = tq.qgemv_x(qtype, tiles, K, N, xd, split=split)
        q, d = tq.quantize_act(xd)
        y2 = tq.qgemv(qtype, tiles, K, N, q, d, split=split)
        assert torch.equal(y1, y2), (act, qtype, M, split)
        check_y(y1.cpu().numpy(), y_ref, acond, ("fused edges", act, qtype, M, split))


@pytest.fixture(scope="module")
def q8_full():
    """Q8_0 weights holding -128 (every third row all -128) and edge
    activations (constant blocks give all-+-127 codes)."""
    K, N = 512, 70
    flat, tiles_ref = _tiles(Q8_0, K, N, seed=7, q8_full=True)
    return K, N, flat, tiles_ref


def _act(M, K, seed):
    x = edge_x(M, K, "f32", seed)
    return x, oracle.quantize_act(x, oracle.F32)


@pytest.mark.parametrize("path,M", [("gemv", 1), ("gemv", 4), ("gemv", 5), ("gemv", 8),
                                    ("gemm", 9), ("gemm", 40), ("gemv_flat", 1),
                                    ("gemv_flat", 8), ("gemm_flat", 40)])
def test_q8_minus128_block_dots(tq, q8_full, path, M):
    K, N, flat, tiles_ref = q8_full
    _, (qr, _) = _act(M, K, seed=M)
    flat_path = path.endswith("flat")
    w = torch.from_numpy(flat if flat_path else tiles_ref).cuda()
    p = {"gemv": tq.PATH_GEMV, "gemm": tq.PATH_GEMM, "gemv_flat": tq.PATH_GEMV_FLAT,
         "gemm_flat": tq.PATH_GEMM_FLAT}[path]
    got = tq.block_dots(Q8_0, w, K, N, torch.from_numpy(qr).cuda(), path=p).cpu().numpy()
    ref = (oracle.block_dots_flat(Q8_0, flat, K, N, qr) if flat_path
           else oracle.block_dots(Q8_0, tiles_ref, K, N, qr))
    assert np.array_equal(got, ref), (path, M)
    # the extreme dot -128 * 127 * 32 is reached (all -128 row, all +127 block)
    assert np.abs(ref).max() == 32 * 128 * 127


@pytest.mark.parametrize("fn,M", [("qgemv", 1), ("qgemv", 4), ("qgemv", 5), ("qgemv", 8),
                                  ("qgemm", 40), ("qgemv_flat", 1), ("qgemv_flat", 8),
                                  ("qgemm_flat", 40), ("matmul", 24)])
def test_q8_minus128_y(tq, q8_full, fn, M):
    K, N, flat, tiles_ref = q8_full
    _, (qr, dr) = _act(M, K, seed=M + 50)
    flat_path = fn.endswith("flat")
    w = torch.from_numpy(flat if flat_path else tiles_ref).cuda()
    q = torch.from_numpy(qr).cuda()
    d = torch.from_numpy(dr.view(np.int16)).cuda().view(torch.float16)
    y = getattr(tq, fn)(Q8_0, w, K, N, q, d).cpu().numpy()
    y_ref, acond = oracle.matmul(Q8_0, tiles_ref, K, N, qr, dr)
    check_y(y, y_ref, acond, ("q8 -128", fn, M))


def _one_block_expect(isum, wsc, asc):
    """+0 + fp32(isum * fp32(dw * da)): dw * da is exact in fp32 (two 11-bit
    significands; the smallest product 2^-48 is a normal fp32) and so is
    isum * (dw * da) in fp64 (at most 20 + 22 significant bits); the only
    rounding is the final one to fp32.  The sum over blocks starts at +0, so
    a zero term (a zero scale against a negative dot) gives +0, not -0."""
    sc = (wsc[None, :].astype(np.float64) * asc[:, None].astype(np.float64))
    assert np.array_equal(sc, sc.astype(np.float32).astype(np.float64))
    return (isum[:, :, 0].astype(np.float64) * sc).astype(np.float32) + np.float32(0.0)


@pytest.mark.parametrize("qtype", [Q4_0, Q8_0, IQ4_NL, MXFP4])
@pytest.mark.parametrize("fn,M", [("qgemv", 1), ("qgemv", 3), ("qgemv", 5), ("qgemv", 8),
                                  ("qgemm", 40), ("qgemv_flat", 1), ("qgemv_flat", 8),
                                  ("qgemm_flat", 40)])
def test_one_block_bitexact(tq, qtype, fn, M):
    K, N = 32, 70
    dist = "e8m0" if qtype == MXFP4 else "edge"
    flat, tiles_ref = _tiles(qtype, K, N, seed=3 + qtype, dist=dist, q8_full=qtype == Q8_0)
    _, (qr, dr) = _act(M, K, seed=M * 5 + qtype)
    lut = LUT if qtype == IQ4_NL else None
    isum = oracle.block_dots(qtype, tiles_ref, K, N, qr, lut)
    # the weight's scale as the kernels apply it: the fp16 row scale, or for
    # MXFP4 half the E8M0 power of two (the block dot uses 2 * E2M1)
    ts = oracle.tile_bytes(qtype)
    if qtype == MXFP4:
        e = tiles_ref.reshape(-1, ts)[:, 512:544].reshape(-1)[:N].astype(np.int64)
        wsc = np.where(e <= 112, 0.0, np.ldexp(1.0, np.clip(e, 113, 142) - 127)) / 2
    else:
        off = 1024 if qtype == Q8_0 else 512
        sb = tiles_ref.reshape(-1, ts)[:, off:off + 64].copy().view(np.uint16).reshape(-1)[:N]
        wsc = oracle.f16_to_f32_array(sb).astype(np.float64)
    asc = oracle.f16_to_f32_array(dr[:, 0]).astype(np.float64)
    expect = _one_block_expect(isum, wsc, asc)
    w = torch.from_numpy(flat if fn.endswith("flat") else tiles_ref).cuda()
    q = torch.from_numpy(qr).cuda()
    d = torch.from_numpy(dr.view(np.int16)).cuda().view(torch.float16)
    y = getattr(tq, fn)(qtype, w, K, N, q, d, lut=lut).cpu().numpy()
    bad = np.nonzero(y.view(np.uint32) != expect.view(np.uint32))
    assert bad[0].size == 0, (fn, M, [(int(i), int(j), float(y[i, j]), float(expect[i, j]))
                                      for i, j in zip(*bad)][:5])
