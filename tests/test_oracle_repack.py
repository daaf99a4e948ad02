"""Pins of the oracle's tile repack against what the page fixes.

Page: "Hexagon backend developer details", section "Tiled Weight Formats",
subsections "Tile Dimensions and Grid Layout" and "Block-32 Quantized Formats".
Pins: hand-worked fixtures (tests/golden/*.txt, derived by hand from the
page's formulas); the page's prose as properties (each column pair owns one
contiguous run of bytes, rows are consecutive inside it, even column in the
low nibble); sizes; padding; lossless round trip against the generator's own
codes (not the oracle's decode).
"""
import numpy as np
import pytest

import synth
from conftest import read_golden

Q4_0, Q8_0, IQ4_NL = synth.Q4_0, synth.Q8_0, synth.IQ4_NL
TILE = {Q4_0: 576, Q8_0: 1088, IQ4_NL: 576}


def _tile_from_codes(orc, qtype, codes, scale_bits):
    N, K = codes.shape
    flat = synth.pack_flat(qtype, codes, scale_bits)
    return orc.repack(qtype, flat, K, N)


@pytest.mark.parametrize("qtype", [Q4_0, IQ4_NL])
def test_q4_worked_example(orc, qtype):
    r = np.arange(32)[:, None]
    c = np.arange(32)[None, :]
    codes = ((3 * r + c) % 16).astype(np.uint8)
    sb = (0x3C00 + np.arange(32)).astype(np.uint16).reshape(32, 1)
    tile = _tile_from_codes(orc, qtype, codes, sb)
    assert tile.size == 576
    for off, byte, *_ in read_golden("q4_0_tile_example.txt"):
        assert tile[int(off)] == int(byte, 16), (off, hex(tile[int(off)]), byte)


def test_q8_worked_example(orc):
    r = np.arange(32)[:, None]
    c = np.arange(32)[None, :]
    codes = (r - c).astype(np.int8)
    sb = (0x2000 + 3 * np.arange(32)).astype(np.uint16).reshape(32, 1)
    tile = _tile_from_codes(orc, Q8_0, codes, sb)
    assert tile.size == 1088
    for off, byte, *_ in read_golden("q8_0_tile_example.txt"):
        assert tile[int(off)] == int(byte, 16), (off, hex(tile[int(off)]), byte)


def test_grid_worked_example(orc):
    for tname, n, k, code, tb, off, byte, *_ in read_golden("grid_example.txt"):
        qtype = {"q4_0": Q4_0, "q8_0": Q8_0}[tname]
        K, N = 96, 70
        codes = np.zeros((N, K), np.int8 if qtype == Q8_0 else np.uint8)
        codes[int(n), int(k)] = int(code)
        sb = np.zeros((N, K // 32), np.uint16)
        tiles = _tile_from_codes(orc, qtype, codes, sb)
        assert tiles.size == int(tb) == orc.tiled_bytes(qtype, K, N)
        nz = np.nonzero(tiles)[0]
        assert list(nz) == [int(off)], (tname, n, k, nz)
        assert tiles[int(off)] == int(byte, 16)


def test_q4_one_hot_exhaustive(orc):
    """Every (row, col, code != 0) on one tile: exactly one byte changes; it is
    byte `row` of column pair col//2's 32-byte run, and the code sits in the low
    nibble for an even column, the high nibble for an odd one."""
    for row in range(32):
        for col in range(32):
            for code in range(1, 16):
                codes = np.zeros((32, 32), np.uint8)
                codes[row, col] = code
                tile = _tile_from_codes(orc, Q4_0, codes, np.zeros((32, 1), np.uint16))
                nz = np.nonzero(tile)[0]
                assert nz.size == 1
                b = int(nz[0])
                cp, r = divmod(b, 32)
                assert b < 512 and cp == col // 2 and r == row
                nib = (tile[b] & 0xF) if col % 2 == 0 else (tile[b] >> 4)
                other = (tile[b] >> 4) if col % 2 == 0 else (tile[b] & 0xF)
                assert nib == code and other == 0


def test_q8_one_hot(orc):
    """Every (row, col) with several codes: the only changed byte lies in
    column pair col//2's 64-byte run, at the row's pair of bytes, the even
    column first."""
    for row in range(32):
        for col in range(32):
            for code in (1, -1, 127, -128, 37):
                codes = np.zeros((32, 32), np.int8)
                codes[row, col] = code
                tile = _tile_from_codes(orc, Q8_0, codes, np.zeros((32, 1), np.uint16))
                nz = np.nonzero(tile)[0]
                assert nz.size == 1
                b = int(nz[0])
                cp, rem = divmod(b, 64)
                assert b < 1024 and cp == col // 2 and rem // 2 == row and rem % 2 == col % 2
                assert np.int8(tile[b].view(np.int8)) == code


@pytest.mark.parametrize("qtype", [Q4_0, Q8_0, IQ4_NL])
def test_scales_at_row_offsets(orc, qtype):
    """32 fp16 row scales follow the quants: row r's scale at base + 2r."""
    base = 1024 if qtype == Q8_0 else 512
    for row in range(32):
        codes = np.zeros((32, 32), np.int8 if qtype == Q8_0 else np.uint8)
        sb = np.zeros((32, 1), np.uint16)
        sb[row, 0] = 0xABCD
        tile = _tile_from_codes(orc, qtype, codes, sb)
        assert list(np.nonzero(tile)[0]) == [base + 2 * row, base + 2 * row + 1]
        assert tile[base + 2 * row] == 0xCD and tile[base + 2 * row + 1] == 0xAB


@pytest.mark.parametrize("qtype", [Q4_0, Q8_0, IQ4_NL])
@pytest.mark.parametrize("K,N", [(32, 1), (64, 31), (96, 33), (32, 64), (128, 65), (256, 64)])
def test_roundtrip_and_sizes(orc, qtype, K, N):
    rng = np.random.default_rng(K * 1000 + N)
    codes = synth.draw_codes(rng, qtype, N, K)
    sb = synth.draw_scales(rng, "uniform", N, K)
    flat = synth.pack_flat(qtype, codes, sb)
    assert flat.size == orc.flat_bytes(qtype, K, N) == N * (K // 32) * {0: 18, 1: 34, 2: 18}[qtype]
    tiles = orc.repack(qtype, flat, K, N)
    assert tiles.size == (K // 32) * ((N + 31) // 32) * TILE[qtype]
    if N % 32 == 0:
        assert tiles.size == flat.size          # repack is a byte permutation
        assert np.array_equal(np.sort(np.unpackbits(tiles)), np.sort(np.unpackbits(flat)))
    c2, s2 = orc.unpack(qtype, tiles, K, N)
    assert np.array_equal(c2, codes.view(np.uint8))
    assert np.array_equal(s2, sb)
    c3, s3 = orc.flat_decode(qtype, flat, K, N)
    assert np.array_equal(c3, codes.view(np.uint8)) and np.array_equal(s3, sb)


@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
@pytest.mark.parametrize("N", [1, 31, 33, 65])
def test_padding_rows_zero(orc, qtype, N):
    K = 64
    rng = np.random.default_rng(N)
    codes = synth.draw_codes(rng, qtype, N, K)
    codes[codes == 0] = 1      # make every valid code non-zero
    sb = synth.draw_scales(rng, "uniform", N, K)
    tiles = orc.repack(qtype, synth.pack_flat(qtype, codes, sb), K, N).reshape(-1, K // 32, TILE[qtype])
    last = tiles[-1]
    nvalid = N - 32 * (tiles.shape[0] - 1)
    for kt in range(K // 32):
        t = last[kt]
        base = 1024 if qtype == Q8_0 else 512
        for row in range(32):
            if qtype == Q8_0:
                qb = np.concatenate([t[cp * 64 + 2 * row: cp * 64 + 2 * row + 2] for cp in range(16)])
            else:
                qb = t[[cp * 32 + row for cp in range(16)]]
            sc = t[base + 2 * row: base + 2 * row + 2]
            if row >= nvalid:
                assert not qb.any() and not sc.any()
            else:
                assert sc.any()
