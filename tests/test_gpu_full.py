"""GPU parity at the workloads' full sizes, through the same binding calls
(and so the same launch geometry, K split included) that bench.py times.

Repack and quantization are compared in full, bit for bit.  y is compared in
full where the oracle finishes in seconds to tens of seconds with its output
rows split over the host threads (the M = 512 GEMM workloads, the lm-head
at M = 128 and M = 1), else on 40 sampled 32-row stripes (the ragged last
one included).  Integer block dots are
compared on first, middle and last stripe, running the GEMV / GEMM kernel on
that stripe's slice of the tile buffer.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import check_mx, check_y, oracle_matmul_rows, to_dev_act

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LUT = synth.IQ4_NL_STANDIN_LUT
_DT = {"f32": oracle.F32, "bf16": oracle.BF16, "f16": oracle.F16}


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_matmul_repack_amd as tq
    tq.lib()
    return tq


class Case:
    """One workload: inputs, oracle repack and quantization, device copies."""

    def __init__(self, tq, name, M=None):
        w = synth.WORKLOADS[name]
        self.w = w
        self.M = w.M if M is None else M
        print(f"[full] {name} M={self.M}: generating", flush=True)
        self.inp = synth.make_inputs(w, M=self.M)
        self.tiles_ref = oracle.repack(w.qtype, self.inp.flat, w.K, w.N)
        self.q_ref, self.d_ref = oracle.quantize_act(self.inp.x, _DT[w.act_dtype])
        print(f"[full] {name}: device repack + quantize", flush=True)
        flat = torch.from_numpy(self.inp.flat).cuda()
        self.tiles = tq.repack_tiles(w.qtype, flat, w.K, w.N)
        del flat
        self.q, self.d = tq.quantize_act(to_dev_act(self.inp.x, w.act_dtype))
        torch.cuda.synchronize()


def _stripes(w, many=False):
    """First, middle and the ragged last stripe; many=True: 40 stripes spread
    over the matrix (the last one included)."""
    nct = w.n_col_tiles
    if many:
        return sorted({nct * i // 39 for i in range(39)} | {nct - 1})
    return sorted({0, nct // 2, nct - 1})


def _check_case(tq, c, fn, full_y):
    w = c.w
    assert np.array_equal(c.tiles.cpu().numpy(), c.tiles_ref), "repack differs"
    assert np.array_equal(c.q.cpu().numpy(), c.q_ref), "quantized activations differ"
    assert np.array_equal(c.d.cpu().view(torch.int16).numpy().view(np.uint16), c.d_ref)
    print(f"[full] {w.name}: {fn.__name__}", flush=True)
    y = fn(w.qtype, c.tiles, w.K, w.N, c.q, c.d, lut=c.inp.lut).cpu().numpy()
    if full_y:
        # every output, the oracle's rows split over the host threads
        y_ref, acond = oracle_matmul_rows(w.qtype, c.tiles_ref, w.K, w.N, c.q_ref, c.d_ref,
                                          c.inp.lut)
        check_y(y, y_ref, acond, w.name)
    else:
        for s in _stripes(w, many=True):
            n0, n1 = 32 * s, min(32 * s + 32, w.N)
            y_ref, acond = oracle.matmul(w.qtype, c.tiles_ref, w.K, w.N, c.q_ref, c.d_ref,
                                         c.inp.lut, n0=n0, n1=n1)
            check_y(y[:, n0:n1], y_ref[:, n0:n1], acond[:, n0:n1], (w.name, s))


def _check_dots(tq, c, path):
    """Block dots of sampled stripes, from the kernel run on the stripe's slice."""
    w = c.w
    ts = oracle.tile_bytes(w.qtype)
    nkt = w.K // 32
    for s in _stripes(w):
        n = min(32, w.N - 32 * s)
        sl = c.tiles[s * nkt * ts:(s + 1) * nkt * ts]
        sl_ref = c.tiles_ref[s * nkt * ts:(s + 1) * nkt * ts]
        got = tq.block_dots(w.qtype, sl, w.K, n, c.q, lut=c.inp.lut, path=path).cpu().numpy()
        ref = oracle.block_dots(w.qtype, sl_ref, w.K, n, c.q_ref, c.inp.lut)
        assert np.array_equal(got, ref), (w.name, s)


def test_q4_0_k256_n64_m1(tq):
    c = Case(tq, "q4_0_gemv_k256_n64_m1")
    _check_case(tq, c, tq.qgemv, full_y=True)
    _check_dots(tq, c, tq.PATH_GEMV)


def test_q8_0_k4096_n4096_m1(tq):
    c = Case(tq, "q8_0_gemv_k4096_n4096_m1")
    _check_case(tq, c, tq.qgemv, full_y=True)
    _check_dots(tq, c, tq.PATH_GEMV)
    got = tq.block_dots(c.w.qtype, c.tiles, c.w.K, c.w.N, c.q, path=tq.PATH_GEMV).cpu().numpy()
    ref = oracle.block_dots(c.w.qtype, c.tiles_ref, c.w.K, c.w.N, c.q_ref)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("M", [1, 4, 8])
def test_q4_0_k4096_n14336(tq, M):
    c = Case(tq, "q4_0_gemv_k4096_n14336_m1", M=M)
    _check_case(tq, c, tq.qgemv, full_y=True)
    _check_dots(tq, c, tq.PATH_GEMV)


def test_iq4_nl_m512_k4096_n4096(tq):
    c = Case(tq, "iq4_nl_gemm_m512_k4096_n4096")
    _check_case(tq, c, tq.qgemm, full_y=True)
    _check_dots(tq, c, tq.PATH_GEMM)


@pytest.mark.parametrize("M", [1, 4])
def test_mxfp4_k4096_n14336(tq, M):
    c = Case(tq, "mxfp4_gemv_k4096_n14336_m1", M=M)
    _check_case(tq, c, tq.qgemv, full_y=True)
    _check_dots(tq, c, tq.PATH_GEMV)


def test_mxfp4_m512_k4096_n4096(tq):
    c = Case(tq, "mxfp4_gemm_m512_k4096_n4096")
    _check_case(tq, c, tq.qgemm, full_y=True)
    _check_dots(tq, c, tq.PATH_GEMM)


def test_mxfp4_mx_m512_k4096_n4096(tq):
    """The same workload on the block-scaled matrix cores: MXFP8 activations
    bit for bit in full, y on the sampled stripes."""
    c = Case(tq, "mxfp4_gemm_m512_k4096_n4096")
    w = c.w
    assert np.array_equal(c.tiles.cpu().numpy(), c.tiles_ref), "repack differs"
    qr, er = oracle.quantize_act_mx(c.inp.x, _DT[w.act_dtype])
    print(f"[full] {w.name}: quantize_act_mx + qgemm_mx", flush=True)
    q, e = tq.quantize_act_mx(to_dev_act(c.inp.x, w.act_dtype))
    assert np.array_equal(q.cpu().numpy(), qr) and np.array_equal(e.cpu().numpy(), er)
    y = tq.qgemm_mx(c.tiles, w.K, w.N, q, e).cpu().numpy()
    for s in _stripes(w, many=True):
        n0, n1 = 32 * s, min(32 * s + 32, w.N)
        y_ref, acond = oracle.matmul_mx(c.tiles_ref, w.K, w.N, qr, er, n0=n0, n1=n1)
        # the block-scaled matrix core's bound (derived in test_gpu_mx)
        check_mx(y[:, n0:n1], y_ref[:, n0:n1], acond[:, n0:n1], (w.name, "mx", s), w.K)


@pytest.mark.parametrize("M", [1, 8])
def test_q4_1_k4096_n14336(tq, M):
    c = Case(tq, "q4_1_gemv_k4096_n14336_m1", M=M)
    _check_case(tq, c, tq.qgemv, full_y=True)
    _check_dots(tq, c, tq.PATH_GEMV)


def test_q4_1_m512_k4096_n4096(tq):
    c = Case(tq, "q4_1_gemm_m512_k4096_n4096")
    _check_case(tq, c, tq.qgemm, full_y=True)
    _check_dots(tq, c, tq.PATH_GEMM)


def test_q4_k_k4096_n14336_m1(tq):
    c = Case(tq, "q4_k_gemv_k4096_n14336_m1")
    _check_case(tq, c, tq.qgemv, full_y=True)
    _check_dots(tq, c, tq.PATH_GEMV)


@pytest.mark.parametrize("name", ["q4_0_gemv_k4096_n14336_m1", "q8_0_gemv_k4096_n4096_m1"])
def test_flat_full_size(tq, name):
    """The flat path at full size: device unpack of the repacked tiles gives
    the flat bytes back; the flat GEMV's y against the oracle (in full) and
    its block dots on sampled stripes."""
    c = Case(tq, name)
    w = c.w
    flat = torch.from_numpy(c.inp.flat).cuda()
    assert np.array_equal(tq.unpack_tiles(w.qtype, c.tiles, w.K, w.N).cpu().numpy(), c.inp.flat)
    y = tq.qgemv_flat(w.qtype, flat, w.K, w.N, c.q, c.d, lut=c.inp.lut).cpu().numpy()
    y_ref, acond = oracle.matmul_flat(w.qtype, c.inp.flat, w.K, w.N, c.q_ref, c.d_ref, c.inp.lut)
    check_y(y, y_ref, acond, ("flat", w.name))
    nb = w.K // 32
    bb = oracle.block_bytes(w.qtype)
    for s in _stripes(w):
        n0, n1 = 32 * s, min(32 * s + 32, w.N)
        sl = c.inp.flat[n0 * nb * bb:n1 * nb * bb]
        got = tq.block_dots(w.qtype, flat[n0 * nb * bb:n1 * nb * bb], w.K, n1 - n0, c.q,
                            lut=c.inp.lut, path=tq.PATH_GEMV_FLAT).cpu().numpy()
        assert np.array_equal(got, oracle.block_dots_flat(w.qtype, sl, w.K, n1 - n0, c.q_ref,
                                                          c.inp.lut)), (w.name, s)


@pytest.fixture(scope="module")
def lmhead(tq):
    return Case(tq, "q8_0_lmhead_k4096_n128001_m128")


def test_q8_0_lmhead_n128001_m1(tq, lmhead):
    """Decode over the 128001-row lm-head (ragged last tile, 1 valid row)."""
    w = lmhead.w
    assert w.n_col_tiles == 4001 and w.N - 32 * (w.n_col_tiles - 1) == 1
    assert np.array_equal(lmhead.tiles.cpu().numpy(), lmhead.tiles_ref), "repack differs"
    q1, d1 = lmhead.q[:1].contiguous(), lmhead.d[:1].contiguous()
    y = tq.qgemv(w.qtype, lmhead.tiles, w.K, w.N, q1, d1).cpu().numpy()
    y_ref, acond = oracle.matmul(w.qtype, lmhead.tiles_ref, w.K, w.N, lmhead.q_ref[:1],
                                 lmhead.d_ref[:1])
    check_y(y, y_ref, acond, "lmhead m1")


def test_q8_0_lmhead_n128001_m128(tq, lmhead):
    """Prefill over the lm-head: every output (128 x 128001, the ragged last
    stripe included), the oracle's rows split over the host threads."""
    _check_case(tq, lmhead, tq.qgemm, full_y=True)
    _check_dots(tq, lmhead, tq.PATH_GEMM)
