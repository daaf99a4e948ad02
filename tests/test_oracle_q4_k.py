"""Pins of the oracle's Q4_K support.

Page: "Hexagon backend developer details", section "Tiled Weight Formats",
subsection "K-Quants": GGML packs 256 elements per super-block; each splits
along K into 8 tiles of 32 k; the Q4_K tile has the Q4_1 tile's layout, 4-bit
quants at 32*cp + r, then per row the FP16 pair (d * sc, -dmin * m).
Pins: the tile's pair values against numpy's own fp16 rounding of the
products; the pair position and quant layout by one-hot inputs; an
independent brute force from flat super-blocks; Q4_K tiles behaving exactly
as Q4_1 tiles with the same bytes.  The flat super-block itself (GGML's
layout and 6-bit packing of scales and mins) is not printed on the pages:
parity unpinned there (checked only for consistency with the generator).
"""
import numpy as np
import pytest

import synth

Q4_K, Q4_1 = synth.Q4_K, synth.Q4_1
F16_ONE = np.float16(1.0).view(np.uint16)


def _params(N, K, d=F16_ONE, dmin=F16_ONE, sc=0, m=0):
    nsb = K // 256
    return synth.Q4KScales(np.full((N, nsb), d, np.uint16), np.full((N, nsb), dmin, np.uint16),
                           np.full((N, K // 32), sc, np.uint8), np.full((N, K // 32), m, np.uint8))


def _tiles(orc, codes, p):
    N, K = codes.shape
    return orc.repack(Q4_K, synth.pack_flat(Q4_K, codes, p), K, N)


def test_sizes(orc):
    assert orc.tile_bytes(Q4_K) == 640 and orc.block_bytes(Q4_K) == 144
    assert orc.block_elems(Q4_K) == 256 and orc.block_elems(Q4_1) == 32
    assert orc.flat_bytes(Q4_K, 4096, 14336) == 14336 * 16 * 144
    assert orc.tiled_bytes(Q4_K, 512, 33) == 16 * 2 * 640


def test_pairs_are_fp16_products(orc):
    """Tile row r of sub-block j holds fp16(d * sc_j) at 512 + 4r and
    fp16(-(dmin * m_j)) at 514 + 4r, rounded to nearest even (numpy's
    conversion here, the oracle's own in C)."""
    K, N = 256, 32
    rng = np.random.default_rng(1)
    p = synth.draw_scales(rng, "q4k", N, K)
    p.sc[0, :] = [63, 1, 32, 17, 48, 5, 60, 33]      # all 6 bits in play
    p.m[0, :] = [0, 63, 16, 47, 2, 59, 31, 40]
    tiles = _tiles(orc, np.zeros((N, K), np.uint8), p).reshape(8, 640)
    d = p.d.view(np.float16).astype(np.float32)
    dmin = p.dmin.view(np.float16).astype(np.float32)
    for j in range(8):
        pair = tiles[j, 512:640].view(np.uint16).reshape(32, 2)
        want_a = (d[:, 0] * p.sc[:, j].astype(np.float32)).astype(np.float16).view(np.uint16)
        want_b = (-(dmin[:, 0] * p.m[:, j].astype(np.float32))).astype(np.float16).view(np.uint16)
        assert np.array_equal(pair[:, 0], want_a), j
        assert np.array_equal(pair[:, 1], want_b), j
    assert tiles[0, 512 + 2] == 0x00 and tiles[0, 512 + 3] == 0x80      # -(1.0 * 0) = -0.0


def test_unit_scales_give_exact_pairs(orc):
    """d = dmin = 1: the pair is (sc, -m) exactly, for every 6-bit value."""
    K, N = 256, 64
    p = _params(N, K)
    p.sc[:] = np.arange(N)[:, None] % 64
    p.m[:] = (np.arange(N)[:, None] * 7 + np.arange(8)[None, :]) % 64
    tiles = _tiles(orc, np.zeros((N, K), np.uint8), p).reshape(2, 8, 640)
    for ct in range(2):
        for j in range(8):
            pair = tiles[ct, j, 512:640].view(np.float16).reshape(32, 2).astype(np.float64)
            rows = np.arange(32 * ct, 32 * ct + 32)
            assert np.array_equal(pair[:, 0], p.sc[rows, j])
            assert np.array_equal(pair[:, 1], -p.m[rows, j].astype(np.float64))


def test_quant_layout_one_hot(orc):
    """Every element of a super-block lands as one nibble of its 32-k tile at
    the Q4_0 position (column pair col // 2, byte `row`, even column low)."""
    K, N = 256, 3
    for e in range(256):
        codes = np.zeros((N, K), np.uint8)
        codes[1, e] = 9
        tiles = _tiles(orc, codes, _params(N, K)).reshape(8, 640)
        kt, col = divmod(e, 32)
        nz = [(t, b) for t in range(8) for b in np.nonzero(tiles[t, :512])[0]]
        assert nz == [(kt, (col // 2) * 32 + 1)], (e, nz)
        assert tiles[kt, (col // 2) * 32 + 1] == (9 if col % 2 == 0 else 9 << 4)


def _decode_flat(flat, K, N):
    """Codes and the six-bit scales and mins, decoded here from GGML Q4_K."""
    nsb = K // 256
    b = flat.reshape(N, nsb, 144)
    d = b[:, :, 0:2].copy().view(np.float16)[..., 0].astype(np.float32)
    dmin = b[:, :, 2:4].copy().view(np.float16)[..., 0].astype(np.float32)
    s = b[:, :, 4:16].astype(np.int64)
    sc = np.zeros((N, nsb, 8), np.int64)
    mn = np.zeros((N, nsb, 8), np.int64)
    for j in range(8):
        if j < 4:
            sc[..., j] = s[..., j] & 63
            mn[..., j] = s[..., j + 4] & 63
        else:
            sc[..., j] = (s[..., j + 4] & 15) + 16 * (s[..., j - 4] >> 6)
            mn[..., j] = (s[..., j + 4] >> 4) + 16 * (s[..., j] >> 6)
    q = b[:, :, 16:].reshape(N, nsb, 4, 32)
    codes = np.concatenate([q & 15, q >> 4], axis=-1).reshape(N, K)
    return codes, d, dmin, sc, mn


@pytest.mark.parametrize("K,N,M", [(256, 1, 1), (256, 33, 2), (512, 7, 3)])
def test_matmul_brute_force(orc, K, N, M):
    rng = np.random.default_rng(700 + K + N + M)
    codes = synth.draw_codes(rng, Q4_K, N, K)
    p = synth.draw_scales(rng, "q4k", N, K)
    flat = synth.pack_flat(Q4_K, codes, p)
    x = synth.draw_activations(rng, M, K)
    tiles = orc.repack(Q4_K, flat, K, N)
    q, da = orc.quantize_act(x)
    y, acond = orc.matmul(Q4_K, tiles, K, N, q, da)
    c, d, dmin, sc, mn = _decode_flat(flat, K, N)
    a16 = (d[:, :, None] * sc.astype(np.float32)).astype(np.float16).astype(np.float64)
    b16 = (-(dmin[:, :, None] * mn.astype(np.float32))).astype(np.float16).astype(np.float64)
    w = a16.reshape(N, K // 32).repeat(32, axis=1) * c + b16.reshape(N, K // 32).repeat(32, axis=1)
    act = da.view(np.float16).astype(np.float64).repeat(32, axis=1) * q
    yb = act @ w.T
    assert np.all(np.abs(y - yb) <= 1e-12 * acond)


def test_tiles_compute_as_q4_1(orc):
    """Q4_K and Q4_1 tiles with the same bytes give the same block dots and y."""
    K, N, M = 512, 40, 3
    rng = np.random.default_rng(8)
    p = synth.draw_scales(rng, "q4k", N, K)
    tiles = _tiles(orc, synth.draw_codes(rng, Q4_K, N, K), p)
    q, da = orc.quantize_act(synth.draw_activations(rng, M, K))
    assert np.array_equal(orc.block_dots(Q4_K, tiles, K, N, q), orc.block_dots(Q4_1, tiles, K, N, q))
    assert np.array_equal(orc.matmul(Q4_K, tiles, K, N, q, da)[0], orc.matmul(Q4_1, tiles, K, N, q, da)[0])


@pytest.mark.parametrize("K,N", [(256, 1), (256, 31), (512, 33), (768, 65)])
def test_roundtrip_and_padding(orc, K, N):
    rng = np.random.default_rng(K + 13 * N)
    codes = synth.draw_codes(rng, Q4_K, N, K)
    p = synth.draw_scales(rng, "q4k", N, K)
    flat = synth.pack_flat(Q4_K, codes, p)
    tiles = orc.repack(Q4_K, flat, K, N)
    c2, s2 = orc.unpack(Q4_K, tiles, K, N)
    c3, s3 = orc.flat_decode(Q4_K, flat, K, N)
    assert np.array_equal(c2, codes) and np.array_equal(c3, codes)
    assert np.array_equal(s2, s3)
    t = tiles.reshape(-1, K // 32, 640)[-1]
    nvalid = N - 32 * ((N + 31) // 32 - 1)
    for row in range(nvalid, 32):
        assert not t[:, [cp * 32 + row for cp in range(16)]].any()
        assert not t[:, 512 + 4 * row: 516 + 4 * row].any()
