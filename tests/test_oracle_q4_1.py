"""Pins of the oracle's Q4_1 support against what the page fixes.

Page: "Hexagon backend developer details", section "Tiled Weight Formats",
subsection "Block-32 Quantized Formats" (Q4_1): 640-byte tiles, quants in the
Q4_0 nibble layout, then 32 fp16 pairs per tile, scale[2*row] = d (the scale)
and scale[2*row + 1] = m (the min).  The value of a code is read as GGML's
Q4_1, d * code + m.  Pins: a hand-worked tile (tests/golden/
q4_1_tile_example.txt), exhaustive one-hot repack, hand-computed values of d *
code + m, an independent brute force from flat blocks, the reduction to Q4_0
when m = -8 d, and the min-only closed form.
"""
import numpy as np
import pytest

import synth
from conftest import read_golden

Q4_1, Q4_0 = synth.Q4_1, synth.Q4_0


def _tiles(orc, codes, pairs):
    N, K = codes.shape
    return orc.repack(Q4_1, synth.pack_flat(Q4_1, codes, pairs), K, N)


def _pairs(N, nb, d, m):
    p = np.zeros((N, nb, 2), np.uint16)
    p[..., 0] = d
    p[..., 1] = m
    return p


def test_sizes(orc):
    assert orc.tile_bytes(Q4_1) == 640 and orc.block_bytes(Q4_1) == 20
    assert orc.scale_count(Q4_1) == 2 and orc.scale_count(Q4_0) == 1
    assert orc.tiled_bytes(Q4_1, 4096, 14336) == 128 * 448 * 640
    assert orc.flat_bytes(Q4_1, 64, 33) == 33 * 2 * 20


def test_worked_tile(orc):
    r = np.arange(32)[:, None]
    c = np.arange(32)[None, :]
    codes = ((3 * r + c) % 16).astype(np.uint8)
    pairs = _pairs(32, 1, (0x3C00 + np.arange(32))[:, None], (0xBC00 + np.arange(32))[:, None])
    tile = _tiles(orc, codes, pairs)
    assert tile.size == 640
    for off, byte, *_ in read_golden("q4_1_tile_example.txt"):
        assert tile[int(off)] == int(byte, 16), (off, hex(tile[int(off)]), byte)


def test_one_hot_exhaustive(orc):
    zero = _pairs(32, 1, 0, 0)
    for row in range(32):
        for col in range(32):
            for code in range(1, 16):
                codes = np.zeros((32, 32), np.uint8)
                codes[row, col] = code
                tile = _tiles(orc, codes, zero)
                nz = np.nonzero(tile)[0]
                assert list(nz) == [(col // 2) * 32 + row]
                assert tile[nz[0]] == (code if col % 2 == 0 else code << 4)
        for i, base in ((0, 512), (1, 514)):
            p = zero.copy()
            p[row, 0, i] = 0xABCD
            tile = _tiles(orc, np.zeros((32, 32), np.uint8), p)
            o = base + 4 * row
            assert list(np.nonzero(tile)[0]) == [o, o + 1]
            assert tile[o] == 0xCD and tile[o + 1] == 0xAB


def test_block_dots_are_code_dots(orc):
    """The integer weight is the code, 0..15: one-hot activations read it back."""
    K, N = 32, 32
    codes = np.tile(np.arange(32) % 16, (N, 1)).astype(np.uint8)
    tiles = _tiles(orc, codes, _pairs(N, 1, 0x3C00, 0xC000))
    isum = orc.block_dots(Q4_1, tiles, K, N, np.eye(32, dtype=np.int8))
    for m in range(32):
        assert (isum[m, :, 0] == m % 16).all()


# (code, d bits, m bits, value): value = d * code + m, worked by hand
WORKED = [
    (0, 0x3800, 0xC000, -2.0),        # d = 0.5, m = -2
    (15, 0x3800, 0xC000, 5.5),        # 7.5 - 2
    (4, 0x3800, 0xC000, 0.0),         # 2 - 2
    (9, 0x2E66, 0xB266, 0.6998291),   # d = 0.0999756, m = -0.1999512: 0.8997803 - 0.1999512
    (1, 0x0001, 0x0000, 2.0 ** -24),  # smallest subnormal d, m = +0
    (7, 0x7BFF, 0xFBFF, 6 * 65504.0), # d = max, m = -max
]


def test_worked_values(orc):
    N, K = len(WORKED), 32
    codes = np.zeros((N, K), np.uint8)
    pairs = np.zeros((N, 1, 2), np.uint16)
    for n, (code, db, mb, _) in enumerate(WORKED):
        codes[n, 3] = code
        pairs[n, 0] = (db, mb)
    tiles = _tiles(orc, codes, pairs)
    q = np.zeros((1, K), np.int8)
    q[0, 3] = 1
    y, _ = orc.matmul(Q4_1, tiles, K, N, q, np.array([[0x3C00]], np.uint16))
    for n, (code, db, mb, want) in enumerate(WORKED):
        d = float(np.array(db, np.uint16).view(np.float16))
        m = float(np.array(mb, np.uint16).view(np.float16))
        assert y[0, n] == d * code + m
        assert abs(y[0, n] - want) <= 1e-6 * max(1.0, abs(want)), (n, y[0, n], want)


def _brute_force_from_flat(flat, K, N, q, d):
    """y from flat Q4_1 blocks decoded here: bytes 0..1 d, 2..3 m, 4..19 the
    nibbles (low: element j, high: element j + 16)."""
    M = q.shape[0]
    nb = K // 32
    blocks = flat.reshape(N, nb, 20)
    da = d.view(np.float16).astype(np.float64)
    y = np.zeros((M, N))
    for n in range(N):
        for b in range(nb):
            blk = blocks[n, b]
            dw = float(blk[0:2].view(np.float16)[0])
            mw = float(blk[2:4].view(np.float16)[0])
            for j in range(32):
                code = blk[4 + j] & 0xF if j < 16 else blk[4 + j - 16] >> 4
                w = dw * int(code) + mw
                for m in range(M):
                    y[m, n] += w * (da[m, b] * int(q[m, b * 32 + j]))
    return y


@pytest.mark.parametrize("K,N,M", [(32, 1, 1), (32, 33, 2), (64, 7, 3), (96, 32, 1)])
def test_matmul_brute_force(orc, K, N, M):
    rng = np.random.default_rng(500 + K + N + M)
    codes = synth.draw_codes(rng, Q4_1, N, K)
    pairs = synth.draw_scales(rng, "minmax", N, K)
    flat = synth.pack_flat(Q4_1, codes, pairs)
    x = synth.draw_activations(rng, M, K)
    tiles = orc.repack(Q4_1, flat, K, N)
    q, d = orc.quantize_act(x)
    y, acond = orc.matmul(Q4_1, tiles, K, N, q, d)
    yb = _brute_force_from_flat(flat, K, N, q, d)
    assert np.all(np.abs(y - yb) <= 1e-12 * acond)


def test_reduces_to_q4_0(orc):
    """m = -8 d (exact in fp16) is Q4_0 with the same d: same y; the block
    dots differ by 8 * sum(q) per block."""
    K, N, M = 128, 45, 3
    rng = np.random.default_rng(41)
    codes = synth.draw_codes(rng, Q4_1, N, K)
    d = synth.draw_scales(rng, "uniform", N, K)
    dv = d.view(np.float16)
    m = (-8 * dv.astype(np.float32)).astype(np.float16)
    assert np.array_equal(m.astype(np.float64), -8 * dv.astype(np.float64))
    pairs = np.stack([d, m.view(np.uint16)], axis=-1)
    x = synth.draw_activations(rng, M, K)
    t1 = _tiles(orc, codes, pairs)
    t0 = orc.repack(Q4_0, synth.pack_flat(Q4_0, codes, d), K, N)
    q, da = orc.quantize_act(x)
    y1, _ = orc.matmul(Q4_1, t1, K, N, q, da)
    y0, _ = orc.matmul(Q4_0, t0, K, N, q, da)
    assert np.array_equal(y1, y0)
    b1 = orc.block_dots(Q4_1, t1, K, N, q).astype(np.int64)
    b0 = orc.block_dots(Q4_0, t0, K, N, q).astype(np.int64)
    qs = q.astype(np.int64).reshape(M, 1, K // 32, 32).sum(axis=-1)
    assert np.array_equal(b1, b0 + 8 * qs)


def test_min_only_closed_form(orc):
    """Codes all 0: y[m][n] = m_n * sum_k da * q, whatever d."""
    K, N, M = 96, 40, 2
    rng = np.random.default_rng(3)
    codes = np.zeros((N, K), np.uint8)
    pairs = synth.draw_scales(rng, "minmax", N, K)
    pairs[..., 1] = np.float16(-0.25).view(np.uint16)
    x = synth.draw_activations(rng, M, K)
    tiles = _tiles(orc, codes, pairs)
    q, da = orc.quantize_act(x)
    y, acond = orc.matmul(Q4_1, tiles, K, N, q, da)
    a = (da.view(np.float16).astype(np.float64).repeat(32, axis=1) * q).sum(axis=1)
    assert np.all(np.abs(y - (-0.25) * a[:, None]) <= 1e-12 * acond)


@pytest.mark.parametrize("K,N", [(32, 1), (64, 31), (96, 33), (128, 65)])
def test_roundtrip_and_padding(orc, K, N):
    rng = np.random.default_rng(K + 11 * N)
    codes = synth.draw_codes(rng, Q4_1, N, K)
    pairs = synth.draw_scales(rng, "minmax", N, K)
    flat = synth.pack_flat(Q4_1, codes, pairs)
    tiles = orc.repack(Q4_1, flat, K, N)
    c2, s2 = orc.unpack(Q4_1, tiles, K, N)
    assert np.array_equal(c2, codes) and np.array_equal(s2, pairs)
    c3, s3 = orc.flat_decode(Q4_1, flat, K, N)
    assert np.array_equal(c3, codes) and np.array_equal(s3, pairs)
    t = tiles.reshape(-1, K // 32, 640)[-1]
    nvalid = N - 32 * ((N + 31) // 32 - 1)
    for row in range(nvalid, 32):
        assert not t[:, [cp * 32 + row for cp in range(16)]].any()
        assert not t[:, 512 + 4 * row: 516 + 4 * row].any()
