"""Pins of the oracle's binary16 / bfloat16 conversions against library
routines (numpy float16, torch bfloat16) -- exhaustive where the domain is."""
import numpy as np
import pytest


def test_f16_to_f32_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = orc.f16_to_f32_array(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_roundtrip_identity(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float32)
    keep = ~np.isnan(vals)
    back = orc.f32_to_f16_array(vals[keep])
    assert np.array_equal(back, bits[keep])


def _f32_cases():
    rng = np.random.default_rng(123)
    parts = [
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(20000) * 0.01).astype(np.float32),
        (rng.standard_normal(20000) * 1e-5).astype(np.float32),   # fp16 subnormal range
        (rng.standard_normal(5000) * 1e-8).astype(np.float32),    # underflow to zero
        (rng.standard_normal(5000) * 3e4).astype(np.float32),     # near overflow
        np.array([65504, 65519.996, 65520, 65536, 1e30, -65520, 2.0**-24, 2.0**-25,
                  2.0**-25 * 1.0000001, 3 * 2.0**-26, 0.0, -0.0, np.inf, -np.inf],
                 dtype=np.float32),
    ]
    # exact midpoints between adjacent fp16 values (ties -> even)
    b = np.arange(0, 0x7BFF, 7, dtype=np.uint32).astype(np.uint16)
    lo = b.view(np.float16).astype(np.float64)
    hi = (b + 1).view(np.float16).astype(np.float64)
    parts.append(((lo + hi) / 2).astype(np.float32))
    parts.append(-((lo + hi) / 2).astype(np.float32))
    return np.concatenate(parts)


def test_f32_to_f16_matches_numpy(orc):
    x = _f32_cases()
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = orc.f32_to_f16_array(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_bf16_to_f32_matches_torch(orc):
    torch = pytest.importorskip("torch")
    bits = np.arange(0, 65536, 3, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    got = np.array([orc.bf16_to_f32(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(t)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), t[~nan].view(np.uint32))


def test_synth_bf16_rounding_matches_torch():
    """The input generator's fp32 -> bf16 rounding equals torch's (RNE)."""
    torch = pytest.importorskip("torch")
    import synth
    rng = np.random.default_rng(5)
    x = synth.draw_activations(rng, 8, 1024, "f32")
    rng = np.random.default_rng(5)
    b = synth.draw_activations(rng, 8, 1024, "bf16")
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, t)
