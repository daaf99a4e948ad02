"""Pins of the oracle's MXFP8 activation quantizer and MXFP4 x MXFP8 product
against things other than itself: torch's FP8 E4M3 type (decode table and
its round-to-nearest-even cast), closed forms of the OCP Microscaling scale
rule, bounds that hold for every element, and a dequantize-then-matmul in
numpy built from the already-pinned tile unpack and the OCP E2M1 values."""
import numpy as np
import pytest
import torch

import oracle
import synth

E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


def torch_e4m3(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def test_e4m3_decode_matches_torch():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    want = torch_e4m3(codes)
    got = np.array([oracle.e4m3_value(c) for c in codes])
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def block_with_unit_scale(vals):
    """Blocks whose first element 511 fixes X = 1 (amax in [256, 512))."""
    vals = np.asarray(vals, np.float32)
    n = (len(vals) + 30) // 31
    x = np.zeros((n, 32), np.float32)
    x[:, 0] = 511.0
    flat = x[:, 1:].reshape(-1)
    flat[:len(vals)] = vals
    x[:, 1:] = flat.reshape(n, 31)
    return x, len(vals)


def test_rounding_matches_torch_cast():
    rng = np.random.default_rng(3)
    exact = torch_e4m3(np.arange(0x7F, dtype=np.uint8))
    mids = (exact[1:] + exact[:-1]) / 2                      # every tie
    vals = np.concatenate([exact, mids, rng.uniform(0, 448, 3000),
                           rng.uniform(0, 2.0 ** -5, 1000),
                           np.nextafter(mids.astype(np.float32), 0),
                           np.nextafter(mids.astype(np.float32), 1000)]).astype(np.float32)
    vals = vals[vals < 448]
    vals = np.concatenate([vals, -vals])
    x, n = block_with_unit_scale(vals)
    q, e = oracle.quantize_act_mx(x.reshape(1, -1))
    assert (e == 127).all()
    got = q.reshape(-1, 32)[:, 1:].reshape(-1)[:n]
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_saturation_and_sign():
    x, n = block_with_unit_scale([448.0, 460.0, 464.0, 479.0, 500.0, -490.0, -0.0, 0.0])
    q, e = oracle.quantize_act_mx(x.reshape(1, -1))
    got = q.reshape(-1, 32)[0, :n + 1]
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00]


@pytest.mark.parametrize("c", [1.0, 1.5, 0.75, 3.0, 1e-3, 65504.0, 2.0 ** -100])
def test_constant_block_closed_form(c):
    """A constant block c: X = 2^(floor(log2 c) - 8), every element E4M3 of
    c / X = 256 * (c / 2^floor(log2 c)) in [256, 512)."""
    x = np.full((1, 64), c, np.float32)
    q, e = oracle.quantize_act_mx(x)
    c32 = float(np.float32(c))
    fl = int(np.floor(np.log2(c32)))
    assert (e == fl - 8 + 127).all()
    v = c32 / 2.0 ** (fl - 8)
    want = 0x7E if v >= 448 else int(torch.tensor([v], dtype=torch.float32).to(
        torch.float8_e4m3fn).view(torch.uint8)[0])
    assert (q == want).all()


def test_scale_clamps_and_zero_block():
    x = np.zeros((3, 32), np.float32)
    x[1, :] = 2.0 ** -120            # floor(log2) - 8 = -128 -> clamped to e = 0 (X = 2^-127)
    x[2, 0] = np.float32(2.0 ** -140)   # fp32 subnormal amax
    q, e = oracle.quantize_act_mx(x)
    assert list(e[:, 0]) == [0, 0, 0]
    assert (q[0] == 0).all()
    assert (q[1] == 0x70).all()      # 2^-120 / 2^-127 = 128 = E4M3 0x70
    assert q[2, 0] == 0              # 2^-13 rounds to 0 (smallest E4M3 is 2^-9)


def test_error_bound_and_amax_code():
    """Every element within half an E4M3 step of x / X (or saturated), the
    amax element coded in [256, 448]."""
    x = synth.draw_activations(np.random.default_rng(7), 5, 256) * np.float32(3.0)
    q, e = oracle.quantize_act_mx(x)
    X = 2.0 ** (e.astype(np.float64) - 127)
    v = x.astype(np.float64).reshape(5, 8, 32) / X[:, :, None]
    P = torch_e4m3(q.reshape(-1)).reshape(5, 8, 32)
    a = np.abs(v)
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    sat = a >= 448
    assert (np.abs(P - v)[~sat] <= step[~sat] / 2).all()
    assert (np.abs(P[sat]) == 448).all()
    amax_code = np.abs(P).max(axis=2)
    assert ((amax_code >= 256) & (amax_code <= 448)).all()


def test_bf16_f16_inputs_are_converted_exactly():
    rng = np.random.default_rng(11)
    x = synth.draw_activations(rng, 3, 128)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    xh = torch.from_numpy(x).to(torch.float16)
    for t, dt in ((xb, oracle.BF16), (xh, oracle.F16)):
        bits = t.view(torch.int16).numpy().view(np.uint16)
        got = oracle.quantize_act_mx(bits, dtype=dt)
        want = oracle.quantize_act_mx(t.to(torch.float32).numpy())
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def mxfp4_tiles(rng, K, N, ebytes=None):
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    e = rng.integers(115, 130, (N, K // 32)).astype(np.uint8) if ebytes is None else ebytes
    flat = synth.pack_flat(synth.MXFP4, codes, e.astype(np.uint16))
    return oracle.repack(oracle.MXFP4, flat, K, N), codes, e


def page_scale(e):
    """The page's MXFP4 scale: FP16 with exponent bits clamp(e - 112, 0, 30)."""
    ex = np.clip(e.astype(np.int64) - 112, 0, 30)
    return np.where(ex == 0, 0.0, 2.0 ** (ex - 15.0))


@pytest.mark.parametrize("M,K,N", [(1, 32, 1), (3, 64, 33), (5, 256, 64)])
def test_matmul_mx_dequantize_then_dot(M, K, N):
    rng = np.random.default_rng(M * 1000 + N)
    tiles, codes, e = mxfp4_tiles(rng, K, N)
    x = synth.draw_activations(rng, M, K)
    q, ea = oracle.quantize_act_mx(x)
    ucodes, uscales = oracle.unpack(oracle.MXFP4, tiles, K, N)
    assert np.array_equal(ucodes, codes)
    W = E2M1[ucodes] * np.repeat(page_scale(uscales.reshape(N, -1)), 32, axis=1)
    A = torch_e4m3(q.reshape(-1)).reshape(M, K) * np.repeat(2.0 ** (ea - 127.0), 32, axis=1)
    want = A @ W.T
    y, acond = oracle.matmul_mx(tiles, K, N, q, ea)
    assert np.all(np.abs(y - want) <= 1e-12 * acond + 1e-300)
    assert np.allclose(acond, np.abs(A) @ np.abs(W).T, rtol=1e-12, atol=0)


def test_matmul_mx_scale_edges():
    """Row scales e <= 112 give exactly zero weights; e >= 142 all act as 2^15."""
    rng = np.random.default_rng(2)
    K, N, M = 64, 4, 2
    e = np.array([[0, 112], [113, 142], [143, 254], [200, 142]], np.uint8)
    tiles, codes, _ = mxfp4_tiles(rng, K, N, ebytes=e)
    x = synth.draw_activations(rng, M, K)
    q, ea = oracle.quantize_act_mx(x)
    y, _ = oracle.matmul_mx(tiles, K, N, q, ea)
    A = torch_e4m3(q.reshape(-1)).reshape(M, K) * np.repeat(2.0 ** (ea - 127.0), 32, axis=1)
    assert (y[:, 0] == 0).all()
    w1 = np.concatenate([E2M1[codes[1, :32]] * 2.0 ** -14, E2M1[codes[1, 32:]] * 2.0 ** 15])
    assert np.allclose(y[:, 1], A @ w1, rtol=1e-12, atol=0)
    w2 = E2M1[codes[2]] * 2.0 ** 15
    assert np.allclose(y[:, 2], A @ w2, rtol=1e-12, atol=0)
