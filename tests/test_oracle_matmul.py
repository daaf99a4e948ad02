"""Pins of the oracle's integer block dots and matmul.

Definition: y[m][n] = sum_k (dw[n][k/32] * w[n][k]) * (da[m][k/32] * q[m][k])
(GGML dst = src0^T * src1, ne0 = K, ne1 = N, each block scaled by its row scale
d as the page "Hexagon backend developer details", "Block-32 Quantized
Formats", states for the tiles).  Pins: numpy int64 products on the
generator's own codes, exact special cases (unit scales, zero-point codes,
constant inputs), a naive brute force that decodes flat GGML blocks itself and
never touches tiles, and IQ4_NL with the table i-8 reducing to Q4_0.
"""
import numpy as np
import pytest

import synth

Q4_0, Q8_0, IQ4_NL = synth.Q4_0, synth.Q8_0, synth.IQ4_NL
LUT = synth.IQ4_NL_STANDIN_LUT


def _ints(qtype, codes, lut=LUT):
    if qtype == Q4_0:
        return codes.astype(np.int64) - 8
    if qtype == IQ4_NL:
        return lut.astype(np.int64)[codes]
    return codes.astype(np.int8).astype(np.int64)


def _setup(qtype, K, N, M, seed, dist="uniform"):
    rng = np.random.default_rng(seed)
    codes = synth.draw_codes(rng, qtype, N, K)
    sb = synth.draw_scales(rng, dist, N, K)
    flat = synth.pack_flat(qtype, codes, sb)
    x = synth.draw_activations(rng, M, K)
    return codes, sb, flat, x


@pytest.mark.parametrize("qtype", [Q4_0, Q8_0, IQ4_NL])
@pytest.mark.parametrize("K,N,M", [(32, 1, 1), (64, 33, 3), (256, 64, 2), (128, 70, 5)])
def test_block_dots_vs_numpy(orc, qtype, K, N, M):
    codes, sb, flat, x = _setup(qtype, K, N, M, K + N + M)
    tiles = orc.repack(qtype, flat, K, N)
    q, _ = orc.quantize_act(x)
    isum = orc.block_dots(qtype, tiles, K, N, q, LUT)
    w = _ints(qtype, codes).reshape(N, K // 32, 32)
    qq = q.astype(np.int64).reshape(M, K // 32, 32)
    ref = np.einsum("nbj,mbj->mnb", w, qq)
    assert np.array_equal(isum.astype(np.int64), ref)


def test_block_dots_extremes(orc):
    """|isum| reaches 32*128*127 with Q8_0 code -128 against q = -127."""
    K, N = 32, 32
    codes = np.full((N, K), -128, np.int8)
    tiles = orc.repack(Q8_0, synth.pack_flat(Q8_0, codes, np.zeros((N, 1), np.uint16)), K, N)
    q = np.full((2, K), -127, np.int8)
    q[1] = 127
    isum = orc.block_dots(Q8_0, tiles, K, N, q)
    assert (isum[0] == 32 * 128 * 127).all() and (isum[1] == -32 * 128 * 127).all()


@pytest.mark.parametrize("qtype", [Q4_0, Q8_0, IQ4_NL])
def test_unit_scales_equal_integer_matmul(orc, qtype):
    K, N, M = 128, 40, 3
    codes, _, _, _ = _setup(qtype, K, N, M, 11)
    rng = np.random.default_rng(12)
    ones = np.full((N, K // 32), 0x3C00, np.uint16)
    flat = synth.pack_flat(qtype, codes, ones)
    tiles = orc.repack(qtype, flat, K, N)
    q = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    d = np.full((M, K // 32), 0x3C00, np.uint16)
    y, _ = orc.matmul(qtype, tiles, K, N, q, d, LUT)
    ref = q.astype(np.int64) @ _ints(qtype, codes).T
    assert np.array_equal(y, ref.astype(np.float64))


def test_zero_point_codes_give_exact_zero(orc):
    K, N, M = 96, 33, 2
    codes = np.full((N, K), 8, np.uint8)
    rng = np.random.default_rng(3)
    sb = synth.draw_scales(rng, "uniform", N, K)
    tiles = orc.repack(Q4_0, synth.pack_flat(Q4_0, codes, sb), K, N)
    q, d = orc.quantize_act(synth.draw_activations(rng, M, K))
    y, _ = orc.matmul(Q4_0, tiles, K, N, q, d)
    assert (y == 0.0).all()


def test_constant_closed_form(orc):
    """Constant code c, scale dw, activation x0 > 0:
    y = K * (c - 8) * dw * fp16(x0/127) * 127."""
    K, N, M, c, x0 = 256, 5, 1, 13, 0.75
    dw_bits = np.float16(0.0042).view(np.uint16)
    codes = np.full((N, K), c, np.uint8)
    sb = np.full((N, K // 32), dw_bits, np.uint16)
    tiles = orc.repack(Q4_0, synth.pack_flat(Q4_0, codes, sb), K, N)
    q, d = orc.quantize_act(np.full((M, K), x0, np.float32))
    y, _ = orc.matmul(Q4_0, tiles, K, N, q, d)
    da = float(np.float16(np.float32(x0) / np.float32(127)))
    expect = K * (c - 8) * float(np.float16(0.0042)) * da * 127
    assert np.allclose(y, expect, rtol=1e-15, atol=0)


def _brute_force_from_flat(qtype, flat, K, N, q, d, lut):
    """Naive loops over the flat GGML blocks; never touches the tile layout."""
    bb = {Q4_0: 18, Q8_0: 34, IQ4_NL: 18}[qtype]
    nb = K // 32
    M = q.shape[0]
    y = np.zeros((M, N))
    for n in range(N):
        for b in range(nb):
            blk = flat[(n * nb + b) * bb:(n * nb + b + 1) * bb]
            dw = float(np.array([int(blk[0]) | (int(blk[1]) << 8)], np.uint16).view(np.float16)[0])
            for j in range(32):
                if qtype == Q8_0:
                    w = int(blk[2 + j]) - 256 * (int(blk[2 + j]) >= 128)
                else:
                    code = int(blk[2 + j] & 15) if j < 16 else int(blk[2 + j - 16] >> 4)
                    w = code - 8 if qtype == Q4_0 else int(lut[code])
                for m in range(M):
                    da = float(np.array([d[m, b]], np.uint16).view(np.float16)[0])
                    y[m, n] += (dw * w) * (da * int(q[m, b * 32 + j]))
    return y


@pytest.mark.parametrize("qtype", [Q4_0, Q8_0, IQ4_NL])
@pytest.mark.parametrize("K,N,M", [(32, 1, 1), (32, 33, 2), (64, 7, 3), (64, 32, 1)])
def test_matmul_brute_force(orc, qtype, K, N, M):
    codes, sb, flat, x = _setup(qtype, K, N, M, 100 + K + N + M,
                                "absnormal" if qtype == Q8_0 else "uniform")
    tiles = orc.repack(qtype, flat, K, N)
    q, d = orc.quantize_act(x)
    y, acond = orc.matmul(qtype, tiles, K, N, q, d, LUT)
    yb = _brute_force_from_flat(qtype, flat, K, N, q, d, LUT)
    assert np.all(np.abs(y - yb) <= 1e-12 * acond)


def test_matmul_is_scaled_block_dots(orc):
    """y equals sum_kt dw*da*isum (exact products in fp64)."""
    K, N, M = 256, 64, 2
    codes, sb, flat, x = _setup(Q8_0, K, N, M, 77, "absnormal")
    tiles = orc.repack(Q8_0, flat, K, N)
    q, d = orc.quantize_act(x)
    y, acond = orc.matmul(Q8_0, tiles, K, N, q, d)
    isum = orc.block_dots(Q8_0, tiles, K, N, q)
    dw = sb.view(np.float16).astype(np.float64)
    da = d.view(np.float16).astype(np.float64)
    ref = np.einsum("nb,mb,mnb->mn", dw, da, isum.astype(np.float64))
    assert np.all(np.abs(y - ref) <= 1e-12 * acond)


def test_iq4_identity_table_equals_q4_0(orc):
    K, N, M = 128, 45, 3
    codes, sb, flat, x = _setup(Q4_0, K, N, M, 5)
    ident = (np.arange(16) - 8).astype(np.int8)
    t4 = orc.repack(Q4_0, flat, K, N)
    ti = orc.repack(IQ4_NL, flat, K, N)
    assert np.array_equal(t4, ti)
    q, d = orc.quantize_act(x)
    assert np.array_equal(orc.block_dots(Q4_0, t4, K, N, q), orc.block_dots(IQ4_NL, ti, K, N, q, ident))
    y4, _ = orc.matmul(Q4_0, t4, K, N, q, d)
    yi, _ = orc.matmul(IQ4_NL, ti, K, N, q, d, ident)
    assert np.array_equal(y4, yi)


def test_ragged_rows_equal_padded(orc):
    """A row's result does not depend on how many rows follow it: N = 33 vs
    the same first 33 rows inside N = 64."""
    K, M = 96, 2
    codes, sb, flat, x = _setup(Q8_0, K, 64, M, 21, "absnormal")
    q, d = orc.quantize_act(x)
    t64 = orc.repack(Q8_0, flat, K, 64)
    nb = K // 32
    t33 = orc.repack(Q8_0, flat[:33 * nb * 34], K, 33)
    y64, _ = orc.matmul(Q8_0, t64, K, 64, q, d)
    y33, _ = orc.matmul(Q8_0, t33, K, 33, q, d)
    assert np.array_equal(y64[:, :33], y33)


def test_row_range(orc):
    K, N, M = 64, 70, 2
    _, _, flat, x = _setup(Q4_0, K, N, M, 8)
    tiles = orc.repack(Q4_0, flat, K, N)
    q, d = orc.quantize_act(x)
    yf, _ = orc.matmul(Q4_0, tiles, K, N, q, d)
    yp, _ = orc.matmul(Q4_0, tiles, K, N, q, d, n0=31, n1=66)
    assert np.array_equal(yp[:, 31:66], yf[:, 31:66]) and (yp[:, :31] == 0).all()
