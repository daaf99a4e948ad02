"""Pins of the oracle's products over flat GGML blocks.

Page: "Hexagon backend developer details", "supports_op Independence from
Buffer and Repack State": a supported type must work both repacked into
tiles and stored flat.  The flat products are pinned to the tiled ones
(themselves pinned in test_oracle_matmul / _mxfp4 / _q4_1 / _q4_k): for
every type, block dots and y over the flat blocks equal those over the
repacked tiles exactly, at ragged N.
"""
import numpy as np
import pytest

import synth

LUT = synth.IQ4_NL_STANDIN_LUT
DIST = {synth.Q8_0: "absnormal", synth.MXFP4: "e8m0", synth.Q4_1: "minmax", synth.Q4_K: "q4k"}


@pytest.mark.parametrize("qtype", [synth.Q4_0, synth.Q8_0, synth.IQ4_NL, synth.MXFP4,
                                   synth.Q4_1, synth.Q4_K])
@pytest.mark.parametrize("N,M", [(1, 1), (33, 3), (70, 2)])
def test_flat_equals_tiled(orc, qtype, N, M):
    K = 512
    w = synth.Workload("t", qtype, K, N, M, DIST.get(qtype, "uniform"), seed=N * 10 + M)
    inp = synth.make_inputs(w)
    tiles = orc.repack(qtype, inp.flat, K, N)
    q, d = orc.quantize_act(inp.x)
    assert np.array_equal(orc.block_dots_flat(qtype, inp.flat, K, N, q, LUT),
                          orc.block_dots(qtype, tiles, K, N, q, LUT))
    yf, af = orc.matmul_flat(qtype, inp.flat, K, N, q, d, LUT)
    yt, at = orc.matmul(qtype, tiles, K, N, q, d, LUT)
    assert np.array_equal(yf, yt) and np.array_equal(af, at)


def test_flat_row_range(orc):
    K, N, M = 256, 70, 2
    inp = synth.make_inputs(synth.Workload("t", synth.Q4_0, K, N, M, "uniform", seed=4))
    q, d = orc.quantize_act(inp.x)
    yf, _ = orc.matmul_flat(synth.Q4_0, inp.flat, K, N, q, d)
    yp, _ = orc.matmul_flat(synth.Q4_0, inp.flat, K, N, q, d, n0=31, n1=66)
    assert np.array_equal(yp[:, 31:66], yf[:, 31:66]) and (yp[:, :31] == 0).all()
