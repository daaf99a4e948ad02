"""tq_qgemv_noalloc (the decode product for callers that cannot allocate:
its K-split scratch is a device array inside the library) against tq_qgemv
with a caller-owned workspace, through the C ABI.

Both run the same kernels with the same split, so y must be bit-identical;
it is also checked against the oracle within the stated tolerance.  The
calls come in a row on one stream, each next one with a smaller input, so
that a later call runs on the scratch an earlier, larger one left behind.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import check_y, make

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LUT = synth.IQ4_NL_STANDIN_LUT


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_matmul_repack_amd as tq
    tq.lib()
    return tq


# (type, K, N, M), largest first; workspace bytes (K split S) in the comments
CASES = [
    (synth.Q8_0, 4096, 4064, 8),     # 127 stripes, S = 4: 780,288 B
    (synth.Q4_0, 4096, 4096, 4),     # 128 stripes, S = 2: 131,072 B
    (synth.IQ4_NL, 1024, 300, 3),    # 10 stripes, S = 8: 53,760 B
    (synth.Q4_1, 512, 70, 1),        # 3 stripes, S = 8: 5,376 B
    (synth.Q8_0, 64, 33, 1),         # 2 k-tiles: no split
]


def _inputs(tq, qtype, K, N, M, seed):
    inp = make(qtype, K, N, M, seed=seed)
    tiles_ref = oracle.repack(qtype, inp.flat, K, N)
    qr, dr = oracle.quantize_act(inp.x)
    tiles = torch.from_numpy(tiles_ref).cuda()
    q = torch.from_numpy(qr).cuda()
    d = torch.from_numpy(dr.view(np.int16)).cuda().view(torch.float16)
    lut = LUT if qtype == synth.IQ4_NL else None
    return tiles_ref, qr, dr, tiles, q, d, lut


def test_noalloc_calls_in_a_row_match_qgemv(tq):
    for rep in range(2):
        for i, (qtype, K, N, M) in enumerate(CASES):
            print(f"[noalloc] rep {rep} case {i}: type {qtype} K={K} N={N} M={M}", flush=True)
            tiles_ref, qr, dr, tiles, q, d, lut = _inputs(tq, qtype, K, N, M, seed=11 * i + rep)
            assert tq.lib().tq_qgemv_workspace_bytes(qtype, K, N, M) <= (1 << 20)
            out = torch.full((M, N), 3.0, dtype=torch.float32, device="cuda")
            y0 = tq.qgemv_noalloc(qtype, tiles, K, N, q, d, lut=lut, out=out)
            y1 = tq.qgemv(qtype, tiles, K, N, q, d, lut=lut)
            assert torch.equal(y0, y1), (rep, i)
            y_ref, acond = oracle.matmul(qtype, tiles_ref, K, N, qr, dr, lut)
            check_y(y0.cpu().numpy(), y_ref, acond, ("noalloc", rep, i))


def test_noalloc_repeats_bitwise(tq):
    qtype, K, N, M = CASES[2]
    _, _, _, tiles, q, d, lut = _inputs(tq, qtype, K, N, M, seed=5)
    a = tq.qgemv_noalloc(qtype, tiles, K, N, q, d, lut=lut)
    b = tq.qgemv_noalloc(qtype, tiles, K, N, q, d, lut=lut)
    assert torch.equal(a, b)


def test_noalloc_rejects_before_launch(tq):
    from block_quantized_matmul_repack_amd import TiledqError
    qtype, K, N = synth.Q4_0, 256, 64
    _, _, _, tiles, q, d, _ = _inputs(tq, qtype, K, N, 9, seed=1)
    with pytest.raises(TiledqError):
        tq.qgemv_noalloc(qtype, tiles, K, N, q, d)            # M = 9 > 8
    empty_q = torch.zeros((0, K), dtype=torch.int8, device="cuda")
    empty_d = torch.zeros((0, K // 32), dtype=torch.float16, device="cuda")
    assert tq.qgemv_noalloc(qtype, tiles, K, N, empty_q, empty_d).shape == (0, N)
