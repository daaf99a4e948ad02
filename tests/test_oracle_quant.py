"""Pins of the oracle's dynamic activation quantization.

Reading (the page "Hexagon backend developer details" says only that
activations are dynamically quantized and that the vector dot runs against
Q8_0 activation tiles): per 32-element block, d = amax/127 in fp32,
id = 1/d (0 if d = 0), q = round-half-away(x*id), stored scale = fp16(d).
Pins: closed forms, constructed ties, an independent numpy re-derivation, and
properties that hold for any input.
"""
import numpy as np
import pytest

import synth


def test_constant_block(orc):
    for c in (1.0, 0.37, 5e-3, 123.0, 7e-6):
        x = np.full((1, 32), c, np.float32)
        q, d = orc.quantize_act(x)
        assert (q == 127).all()
        assert d[0, 0] == np.float16(np.float32(c) / np.float32(127)).view(np.uint16)
        q, d = orc.quantize_act(-x)
        assert (q == -127).all()


def test_tiny_block_outside_domain_is_reported(orc):
    # amax so small that 1/d overflows: the oracle reports it, never wraps
    x = np.full((1, 32), 2.0 ** -130, np.float32)
    with pytest.raises(ValueError):
        orc.quantize_act(x)


def test_zero_block(orc):
    x = np.zeros((2, 64), np.float32)
    x[1, 32:] = 2.0
    q, d = orc.quantize_act(x)
    assert (q[0] == 0).all() and (d[0] == 0).all()
    assert (q[1, :32] == 0).all() and d[1, 0] == 0 and (q[1, 32:] == 127).all()


def test_ties_round_away_from_zero(orc):
    """amax = 127 makes d = 1 and id = 1 exactly, so x*id = x: the halves
    must round away from zero (2.5 -> 3, -2.5 -> -3, 0.5 -> 1), unlike
    round-half-to-even."""
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 127.0
    x[0, 1:9] = [2.5, -2.5, 0.5, -0.5, 1.5, 126.5, -126.5, 3.49]
    q, d = orc.quantize_act(x)
    assert d[0, 0] == 0x3C00
    assert list(q[0, :9]) == [127, 3, -3, 1, -1, 2, 127, -127, 3]


def test_amax_maps_to_127(orc):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 32 * 16)).astype(np.float32)
    q, _ = orc.quantize_act(x)
    xb = x.reshape(64, 16, 32)
    qb = q.reshape(64, 16, 32)
    i = np.abs(xb).argmax(-1)
    top = np.take_along_axis(qb, i[..., None], -1)[..., 0]
    sgn = np.sign(np.take_along_axis(xb, i[..., None], -1)[..., 0])
    assert (top == 127 * sgn).all()


def _numpy_reference(x):
    """Independent re-derivation in numpy: fp32 arithmetic where the format
    fixes it, rounding half away from zero done in float64 (numpy's own
    round() is half-to-even and would be wrong here)."""
    M, K = x.shape
    xb = x.reshape(M, K // 32, 32).astype(np.float32)
    amax = np.abs(xb).max(-1)
    d = (amax / np.float32(127)).astype(np.float32)
    with np.errstate(divide="ignore"):
        idv = np.where(d != 0, np.float32(1) / d, np.float32(0)).astype(np.float32)
    v = (xb * idv[..., None]).astype(np.float32).astype(np.float64)
    q = (np.sign(v) * np.floor(np.abs(v) + 0.5)).astype(np.int8)
    return q.reshape(M, K), d.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("seed", range(4))
def test_matches_numpy_rederivation(orc, seed):
    rng = np.random.default_rng(seed)
    scale = [1.0, 1e-3, 30.0, 1e-6][seed]
    x = (rng.standard_normal((7, 32 * 40)) * scale).astype(np.float32)
    x[0, :32] = 0.0
    q, d = orc.quantize_act(x)
    qr, dr = _numpy_reference(x)
    assert np.array_equal(q, qr)
    assert np.array_equal(d, dr)


def test_bf16_f16_inputs_and_stride(orc):
    rng = np.random.default_rng(9)
    xb = synth.draw_activations(rng, 3, 96, "bf16")
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(orc.quantize_act(xb, orc.BF16)[0], orc.quantize_act(xf)[0])
    assert np.array_equal(orc.quantize_act(xb, orc.BF16)[1], orc.quantize_act(xf)[1])
    xh = synth.draw_activations(rng, 3, 96, "f16")
    xhf = xh.view(np.float16).astype(np.float32)
    assert np.array_equal(orc.quantize_act(xh, orc.F16)[0], orc.quantize_act(xhf)[0])
    # row stride larger than K: only the first K columns are read
    wide = np.concatenate([xf, np.full((3, 32), 1e6, np.float32)], axis=1)
    q1, d1 = orc.quantize_act(wide, K=96)
    q0, d0 = orc.quantize_act(xf)
    assert np.array_equal(q1, q0) and np.array_equal(d1, d0)


hyp = pytest.importorskip("hypothesis")
from hypothesis import assume, given, settings, strategies as st  # noqa: E402
from hypothesis.extra import numpy as hnp  # noqa: E402


@settings(max_examples=200, deadline=None)
@given(hnp.arrays(np.float32, (2, 64),
                  elements=st.floats(-1e4, 1e4, allow_nan=False, width=32)))
def test_properties(orc, x):
    # domain of the reading: each block is all zero or has amax >= 2^-120, so
    # that 1/d is finite
    xb = x.reshape(2, 2, 32)
    am = np.abs(xb).max(-1)
    assume(np.all((am == 0) | (am >= 2.0 ** -120)))
    q, d = orc.quantize_act(x)
    qb = q.reshape(2, 2, 32).astype(np.float64)
    amax = np.abs(xb).max(-1)
    dd = (amax / np.float32(127)).astype(np.float32)
    for i in range(2):
        for b in range(2):
            if dd[i, b] == 0:
                assert (qb[i, b] == 0).all()
                continue
            idv = np.float32(1) / dd[i, b]
            v = (xb[i, b] * idv).astype(np.float32).astype(np.float64)
            assert np.all(np.abs(v - qb[i, b]) <= 0.5)
            assert np.all(np.abs(qb[i, b]) <= 127)
            assert np.all((qb[i, b] == 0) | (np.sign(qb[i, b]) == np.sign(xb[i, b])))
