"""Pins of the oracle's MXFP4 support against what the pages and the OCP
Microscaling spec fix.

Page: "Hexagon backend developer details", section "Tiled Weight Formats",
subsection "Block-32 Quantized Formats" (MXFP4): 544-byte tiles, quants in
the Q4_0 nibble layout, 32 E8M0 row bytes at 512 + row, the scale the FP16
power of two with exponent bits clamp(e - 112, 0, 30), codes OCP FP4 (E2M1).
Pins: hand-worked fixtures (tests/golden/mxfp4_*.txt), the E2M1 value table
as printed in the OCP MX v1.0 specification, the scale's closed form at every
byte value, exhaustive one-hot repack, an independent brute force from flat
blocks, and the reduction to IQ4_NL with a fixed table and scale 1/2.
"""
import numpy as np
import pytest

import synth
from conftest import read_golden

MXFP4, Q4_0, IQ4_NL = synth.MXFP4, synth.Q4_0, synth.IQ4_NL

# E2M1 values of codes 0..15 as the OCP MX v1.0 specification tabulates them.
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                 -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def _scale(e):
    """Power-of-two FP16 scale of E8M0 byte e: 2^(clamp(e-112, 0, 30) - 15),
    and 0 where the clamped exponent field is 0."""
    x = min(max(int(e) - 112, 0), 30)
    return 0.0 if x == 0 else 2.0 ** (x - 15)


def _tiles(orc, codes, e):
    N, K = codes.shape
    return orc.repack(MXFP4, synth.pack_flat(MXFP4, codes, e), K, N)


def test_sizes(orc):
    assert orc.tile_bytes(MXFP4) == 544 and orc.block_bytes(MXFP4) == 17
    assert orc.tiled_bytes(MXFP4, 4096, 14336) == 128 * 448 * 544
    assert orc.tiled_bytes(MXFP4, 64, 33) == 2 * 2 * 544
    assert orc.flat_bytes(MXFP4, 64, 33) == 33 * 2 * 17


def test_worked_tile(orc):
    r = np.arange(32)[:, None]
    c = np.arange(32)[None, :]
    codes = ((3 * r + c) % 16).astype(np.uint8)
    e = (100 + 3 * np.arange(32)).astype(np.uint16).reshape(32, 1)
    tile = _tiles(orc, codes, e)
    assert tile.size == 544
    for off, byte, *_ in read_golden("mxfp4_tile_example.txt"):
        assert tile[int(off)] == int(byte, 16), (off, hex(tile[int(off)]), byte)


def test_one_hot_exhaustive(orc):
    """Every (row, col, code != 0): one quant byte changes, at column pair
    col//2's run, byte `row`, in the even column's low nibble or the odd
    column's high nibble; every E8M0 byte lands alone at 512 + row."""
    zero_e = np.zeros((32, 1), np.uint16)
    for row in range(32):
        for col in range(32):
            for code in range(1, 16):
                codes = np.zeros((32, 32), np.uint8)
                codes[row, col] = code
                tile = _tiles(orc, codes, zero_e)
                nz = np.nonzero(tile)[0]
                assert nz.size == 1
                b = int(nz[0])
                assert b == (col // 2) * 32 + row
                assert tile[b] == (code if col % 2 == 0 else code << 4)
        for ev in (1, 127, 255):
            e = zero_e.copy()
            e[row, 0] = ev
            tile = _tiles(orc, np.zeros((32, 32), np.uint8), e)
            assert list(np.nonzero(tile)[0]) == [512 + row] and tile[512 + row] == ev


def test_e2m1_table(orc):
    """Integer weights are twice the OCP E2M1 values: block dots of one-hot
    activations read each code's weight back."""
    K, N = 32, 32
    codes = np.tile(np.arange(32) % 16, (N, 1)).astype(np.uint8)
    tiles = _tiles(orc, codes, np.full((N, 1), 127, np.uint16))
    q = np.eye(32, dtype=np.int8)
    isum = orc.block_dots(MXFP4, tiles, K, N, q)
    for m in range(32):
        assert (isum[m, :, 0] == 2 * E2M1[m % 16]).all()


def test_scale_closed_form_every_byte(orc):
    for e in range(256):
        assert orc.row_scale(MXFP4, e) == 0.5 * _scale(e), e
    assert _scale(127) == 1.0 and _scale(113) == 2.0 ** -14 and _scale(142) == 2.0 ** 15
    assert _scale(112) == 0.0 and _scale(255) == 2.0 ** 15


def test_worked_dequant(orc):
    """y of a one-element product equals the hand-worked weight value."""
    rows = read_golden("mxfp4_dequant_example.txt")
    N, K = len(rows), 32
    codes = np.zeros((N, K), np.uint8)
    e = np.zeros((N, 1), np.uint16)
    want = np.zeros(N)
    for n, (code, ev, value, *_) in enumerate(rows):
        codes[n, 5] = int(code, 16)
        e[n, 0] = int(ev)
        want[n] = float(value)
    tiles = _tiles(orc, codes, e)
    q = np.zeros((1, K), np.int8)
    q[0, 5] = 1
    d = np.array([[0x3C00]], np.uint16)          # fp16 1.0
    y, _ = orc.matmul(MXFP4, tiles, K, N, q, d)
    assert np.array_equal(y[0], want), (y[0], want)


def _brute_force_from_flat(flat, K, N, q, d):
    """y from flat MXFP4 blocks, decoded here: byte 0 the E8M0 scale, bytes
    1..16 the nibbles (low: element j, high: element j + 16)."""
    M = q.shape[0]
    nb = K // 32
    blocks = flat.reshape(N, nb, 17)
    da = d.view(np.float16).astype(np.float64)
    y = np.zeros((M, N))
    for n in range(N):
        for b in range(nb):
            blk = blocks[n, b]
            s = _scale(blk[0])
            for j in range(32):
                code = blk[1 + j] & 0xF if j < 16 else blk[1 + j - 16] >> 4
                w = s * E2M1[code]
                for m in range(M):
                    y[m, n] += w * (da[m, b] * int(q[m, b * 32 + j]))
    return y


@pytest.mark.parametrize("K,N,M", [(32, 1, 1), (32, 33, 2), (64, 7, 3), (96, 32, 1)])
def test_matmul_brute_force(orc, K, N, M):
    rng = np.random.default_rng(300 + K + N + M)
    codes = synth.draw_codes(rng, MXFP4, N, K)
    e = synth.draw_scales(rng, "e8m0", N, K)
    flat = synth.pack_flat(MXFP4, codes, e)
    x = synth.draw_activations(rng, M, K)
    tiles = orc.repack(MXFP4, flat, K, N)
    q, d = orc.quantize_act(x)
    y, acond = orc.matmul(MXFP4, tiles, K, N, q, d)
    yb = _brute_force_from_flat(flat, K, N, q, d)
    assert np.all(np.abs(y - yb) <= 1e-12 * acond)


def test_reduces_to_iq4_nl(orc):
    """With every E8M0 byte 127 (scale 1), MXFP4 equals IQ4_NL whose table is
    2 * E2M1 and whose fp16 row scales are all 1/2: same quant bytes, same
    block dots, same y."""
    K, N, M = 128, 45, 3
    rng = np.random.default_rng(9)
    codes = synth.draw_codes(rng, MXFP4, N, K)
    x = synth.draw_activations(rng, M, K)
    tm = _tiles(orc, codes, np.full((N, K // 32), 127, np.uint16))
    half = np.full((N, K // 32), 0x3800, np.uint16)   # fp16 0.5
    ti = orc.repack(IQ4_NL, synth.pack_flat(IQ4_NL, codes, half), K, N)
    lut = (2 * E2M1).astype(np.int8)
    tm4 = tm.reshape(-1, 544)
    ti4 = ti.reshape(-1, 576)
    assert np.array_equal(tm4[:, :512], ti4[:, :512])
    q, d = orc.quantize_act(x)
    assert np.array_equal(orc.block_dots(MXFP4, tm, K, N, q), orc.block_dots(IQ4_NL, ti, K, N, q, lut))
    ym, _ = orc.matmul(MXFP4, tm, K, N, q, d)
    yi, _ = orc.matmul(IQ4_NL, ti, K, N, q, d, lut)
    assert np.array_equal(ym, yi)


@pytest.mark.parametrize("K,N", [(32, 1), (64, 31), (96, 33), (128, 65)])
def test_roundtrip_and_padding(orc, K, N):
    rng = np.random.default_rng(K + 7 * N)
    codes = synth.draw_codes(rng, MXFP4, N, K)
    e = synth.draw_scales(rng, "e8m0", N, K)
    flat = synth.pack_flat(MXFP4, codes, e)
    tiles = orc.repack(MXFP4, flat, K, N)
    c2, s2 = orc.unpack(MXFP4, tiles, K, N)
    assert np.array_equal(c2, codes) and np.array_equal(s2, e)
    c3, s3 = orc.flat_decode(MXFP4, flat, K, N)
    assert np.array_equal(c3, codes) and np.array_equal(s3, e)
    t = tiles.reshape(-1, K // 32, 544)[-1]
    nvalid = N - 32 * ((N + 31) // 32 - 1)
    for row in range(nvalid, 32):
        assert not t[:, [cp * 32 + row for cp in range(16)]].any()
        assert not t[:, 512 + row].any()
