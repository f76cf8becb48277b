"""Seeded input generation: rounding to 16-bit storage and the workload recipes."""
import numpy as np
import pytest
import torch

import workloads as W


def _edge_f32():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(20000).astype(np.float32) * 10
    # exact ties and values straddling the rounding boundary of bf16/fp16
    base = np.array([1.0, 1.5, -2.25, 3.0e-3, 65504.0, 1e-8, -1e-30, 0.0, -0.0],
                    dtype=np.float32).view(np.uint32)
    extra = np.concatenate([base, base + 0x7FFF, base + 0x8000, base + 0x8001,
                            base + 0x18000, base + 0x1000, base + 0x1001]).view(np.float32)
    return np.concatenate([x, extra[np.isfinite(extra)]])


def test_bf16_rne_matches_torch():
    x = _edge_f32()
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_f16_rne_matches_torch():
    x = _edge_f32()
    x = x[np.abs(x) < 60000]
    ours = W.f32_to_f16_bits(x)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


@pytest.mark.parametrize("dt", [W.F16, W.BF16])
def test_decode_is_exact(dt):
    x = _edge_f32()
    x = x[np.abs(x) < 60000]
    bits = W.round_bits(x, dt)
    tdt = torch.float16 if dt == W.F16 else torch.bfloat16
    ref = torch.from_numpy(x).to(tdt).to(torch.float64).numpy()
    np.testing.assert_array_equal(W.decode(bits, dt), ref)
    # decoding then re-rounding is the identity on 16-bit values
    np.testing.assert_array_equal(W.round_bits(W.decode(bits, dt).astype(np.float32), dt), bits)


def test_make_inputs_deterministic_and_shaped():
    w = W.WORKLOADS["tiny"]
    a = W.make_inputs(w)
    b = W.make_inputs(w)
    for x, y in zip(a, b):
        assert x.shape == (1, 1, 128, 64) and x.dtype == np.uint16
        np.testing.assert_array_equal(x, y)
    # causal and non-causal variants share tensors (same seed)
    c = W.make_inputs(W.WORKLOADS["tiny_causal"])
    for x, y in zip(a, c):
        np.testing.assert_array_equal(x, y)
    # Q, K, V differ
    assert not np.array_equal(a[0], a[1])


def test_ramp_recipe():
    w = W.Workload("r", 1, 2, 256, 32, W.BF16, True, 7, ramp=0.05)
    q, k, v = W.make_inputs(w)
    q0, k0, v0 = W.make_inputs(w, ramp_override=0.0)
    np.testing.assert_array_equal(v, v0)
    dk = W.decode(k, W.BF16) - W.decode(k0, W.BF16)
    dq = W.decode(q, W.BF16) - W.decode(q0, W.BF16)
    # the key offset grows linearly along the key axis in one fixed direction
    u = dq[0, 0].mean(axis=0)
    u /= np.linalg.norm(u)
    proj = dk[0, 0] @ u
    j = np.arange(256)
    slope = np.polyfit(j, proj, 1)[0]
    assert abs(slope - 0.05) < 0.005
    # the same offsets in every head
    np.testing.assert_allclose(dk[0, 0], dk[0, 1], atol=0.1)


def test_workload_table():
    w = W.WORKLOADS["long"]
    assert (w.B, w.H, w.S, w.D, w.dtype, w.causal) == (2, 16, 8192, 128, W.BF16, True)
    assert w.flops == 4 * 2 * 16 * 8192 ** 2 * 128 / 2
    assert w.algorithmic_bytes == 269_484_032
    assert W.WORKLOADS["bat"].flops == 171_798_691_840
    assert W.WORKLOADS["dec"].algorithmic_bytes == 8_454_144
    assert W.WORKLOADS["tiny"].scale == np.float32(0.125)
