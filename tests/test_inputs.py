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


# ---- 8-bit float E4M3FN (OCP 8-bit floating point specification) ----------

def test_e4m3_decode_known_codes():
    # exponent bias 7, three mantissa bits, no infinities, S.1111.111 is NaN
    codes = np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0x39, 0x3F, 0x40, 0x7E, 0xB8, 0xFE])
    want = [0.0, -0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.125, 1.875, 2.0, 448.0,
            -1.0, -448.0]
    got = W.decode(codes, W.E4M3)
    np.testing.assert_array_equal(got, want)
    assert np.signbit(got[1]) and not np.signbit(got[0])
    assert np.isnan(W.decode(np.array([0x7F, 0xFF]), W.E4M3)).all()


def test_e4m3_codes_are_monotone_and_spaced():
    v = W.decode(np.arange(0x7F), W.E4M3)
    d = np.diff(v)
    assert (d > 0).all()
    # spacing 2^-9 through the subnormals and the first binade, then doubles per binade
    assert (d[:15] == 2.0 ** -9).all()
    for e in range(1, 16):
        assert (d[8 * e: 8 * e + 7] == 2.0 ** (e - 10)).all()


def test_e4m3_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = W.decode(codes, W.E4M3)
    np.testing.assert_array_equal(W.f32_to_e4m3_bits(vals.astype(np.float32)), codes)


def test_e4m3_ties_to_even_and_saturation():
    x = np.array([1.0625, 1.1875, 3 * 2.0 ** -10, 2.0 ** -10, 464.0, 500.0, 1e30, -1e30, np.nan])
    np.testing.assert_array_equal(W.f32_to_e4m3_bits(x),
                                  [0x38, 0x3A, 0x02, 0x00, 0x7E, 0x7E, 0x7E, 0xFE, 0x7F])


def test_e4m3_rounding_matches_torch_in_range():
    x = _edge_f32()
    x = np.concatenate([x / 64, x * 16, x / 4096])
    x = x[np.abs(x) <= 448]
    ours = W.f32_to_e4m3_bits(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_fp8_inputs_span_the_range_and_round_to_nearest():
    w = W.Workload("t8", 1, 2, 256, 128, W.E4M3, True, 9)
    (qc, kc, vc), ds = W.make_fp8_inputs(w)
    rng = np.random.default_rng(9)
    xs = [rng.standard_normal((1, 2, 256, 128), dtype=np.float32) for _ in range(3)]
    for c, d, x in zip((qc, kc, vc), ds, xs):
        assert c.dtype == np.uint8 and c.shape == x.shape
        assert d == float(np.float32(np.abs(x).max() / 448))
        val = W.decode(c, W.E4M3)
        assert np.abs(val).max() == 448.0  # the largest magnitude maps to 448
        # each code is a nearest E4M3 value of x / d: within half a spacing
        y = x.astype(np.float64) / d
        err = np.abs(val - y)
        _, e = np.frexp(np.abs(y))
        half = np.where(e - 1 >= -6, np.ldexp(1.0, e - 5), 2.0 ** -10)
        assert (err <= half * (1 + 1e-12)).all()
    assert W.WORKLOADS["long8"].algorithmic_bytes == 5 * 2 * 16 * 8192 * 128 + 4 * 2 * 16 * 8192
