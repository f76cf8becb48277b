"""Pins for the 8-bit-input oracle and for its P-rounding error bound (CPU only).

The bound is checked against a second, independent rounding to E4M3 written
from frexp (not from the code table the input generator uses): rounding the
scaled probabilities that way must never move O by more than the bound, the
worst rounding the grid allows must stay within it, and the bound must be
within a factor of two of that worst case.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as F
import workloads as W


def rne_e4m3(x: np.ndarray) -> np.ndarray:
    """Round non-negative x (<= 448) to E4M3, nearest with ties to even, via frexp."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)  # x = f * 2^e with f in [0.5, 1)
    quantum = np.where(e - 1 >= -6, np.ldexp(1.0, e - 4), 2.0 ** -9)
    return np.round(x / quantum) * quantum  # numpy rounds halves to even


def half_ulp_e4m3(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    h = np.where(e - 1 >= -6, np.ldexp(1.0, e - 5), 2.0 ** -10)
    return np.where(x == 0, 0.0, h)  # zero (a hidden key) is exact


def _codes(shape, seed, std=1.0):
    rng = np.random.default_rng(seed)
    return W.f32_to_e4m3_bits((std * rng.standard_normal(shape)).astype(np.float32))


def _probs(q, k, causal, scale):
    """Unnormalised P = exp(X - m) and L per row, the plain definition."""
    x = scale * (q @ k.T)
    if causal:
        i, j = np.indices(x.shape)
        x = np.where(j > i + (k.shape[0] - q.shape[0]), -np.inf, x)
    m = x.max(axis=1, keepdims=True)
    p = np.exp(x - m)
    return p, p.sum(axis=1)


def test_frexp_rounding_agrees_with_the_code_table():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(0, 448, 20000), np.exp(rng.uniform(-25, 6, 20000)),
                        W.decode(np.arange(0x7F), W.E4M3),
                        # midpoints between neighbouring codes (ties)
                        0.5 * (W.decode(np.arange(0x7E), W.E4M3)
                               + W.decode(np.arange(1, 0x7F), W.E4M3))])
    x = x[x <= 448].astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(rne_e4m3(x), W.decode(W.f32_to_e4m3_bits(x), W.E4M3))


def test_descales_multiply_the_values():
    S, D = 96, 64
    q, k, v = (W.decode(_codes((S, D), s), W.E4M3) for s in (1, 2, 3))
    o1, l1 = F.attention_fp8(q, k, v, (2.0, 0.25, 3.0), True, 0.125)
    o2, l2 = oracle.attention_fwd(2 * q, 0.25 * k, 3 * v, True, 0.125)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    # only the product dq*dk enters the logits
    o3, l3 = F.attention_fp8(q, k, v, (0.5, 1.0, 3.0), True, 0.125)
    np.testing.assert_allclose(o3, o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l3, l1, rtol=1e-12, atol=1e-12)


def test_constant_v_code_gives_its_descaled_value():
    S, D = 64, 32
    q, k = (W.decode(_codes((S, D), s), W.E4M3) for s in (4, 5))
    v = W.decode(np.full((S, D), 0x3A, dtype=np.uint8), W.E4M3)  # 1.25
    o, _ = F.attention_fp8(q, k, v, (1.0, 1.0, 0.75), False, 0.2)
    np.testing.assert_allclose(o, np.full((S, D), 0.9375), rtol=1e-14)


def test_fp8_oracle_matches_torch_sdpa_on_decoded_values():
    S, D = 80, 64
    q, k, v = (W.decode(_codes((2, S, D), s), W.E4M3) for s in (6, 7, 8))
    ds = (0.03125, 0.5, 1.5)
    o, lse = F.attention_fp8(q, k, v, ds, True, 1 / math.sqrt(D))
    tq, tk, tv = (torch.from_numpy(x * d) for x, d in zip((q, k, v), ds))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                           scale=1 / math.sqrt(D))
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-10, atol=1e-12)
    x = (tq @ tk.transpose(-1, -2)) / math.sqrt(D)
    x = x.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(x, -1).numpy(), rtol=1e-12, atol=1e-12)


def _case(seed, Sq, Sk, D, causal, std_q=1.0, dominant=False):
    q = W.decode(_codes((Sq, D), seed, std_q), W.E4M3)
    k = W.decode(_codes((Sk, D), seed + 1), W.E4M3)
    v = W.decode(_codes((Sk, D), seed + 2), W.E4M3) * 0.5
    if dominant:  # one key far ahead of the rest: most P are tiny (subnormal after scaling)
        k[0] = 8 * np.sign(q.sum(axis=0) + 1e-9)
    return q, k, v, float(np.float32(1 / math.sqrt(D)))


CASES = [(11, 64, 64, 64, False, 1.0, False), (12, 96, 160, 64, True, 1.0, False),
         (13, 128, 128, 128, True, 3.0, False), (14, 64, 200, 32, False, 0.3, False),
         (15, 64, 256, 64, False, 1.0, True), (16, 48, 48, 128, True, 1.0, True)]


@pytest.mark.parametrize("case", CASES)
def test_rounding_p_stays_within_the_bound(case):
    q, k, v, scale = _case(*case[:5], std_q=case[5], dominant=case[6])
    causal = case[4]
    rows = np.arange(q.shape[0])
    o, _ = oracle.attention_rows(q, k, v, rows, causal, scale)
    bound = F.pv_rounding_bound(q, k, v, rows, causal, scale)
    p, l = _probs(q, k, causal, scale)
    s = F.P_SCALE
    # nearest rounding of the scaled probabilities
    o_near = (rne_e4m3(s * p) / s) @ v / l[:, None]
    assert (np.abs(o_near - o) <= bound * (1 + 1e-9) + 1e-15).all()
    # a factor that differs per key (the running base moves between key
    # tiles): any power of two from p_scale up to the one that puts the
    # row maximum (p = 1) at the top of the lagging base's range, 2^8
    top = int(round(math.log2(F.P_MAX / s)))
    f = s * 2.0 ** np.random.default_rng(case[0]).integers(0, top + 1, size=p.shape[1])
    o_var = (rne_e4m3(f * p) / f) @ v / l[:, None]
    assert (np.abs(o_var - o) <= bound * (1 + 1e-9) + 1e-15).all()
    # the worst any rounding to a neighbouring grid point within half a spacing
    # can do, column by column: each error pushed in the sign of V
    worst = (half_ulp_e4m3(s * p) / s) @ np.abs(v) / l[:, None]
    assert (worst <= bound * (1 + 1e-9) + 1e-15).all()
    # and the bound is no more than twice that worst case
    assert (bound <= 2 * worst + 1e-15).all()


@pytest.mark.parametrize("case", CASES[:4])
def test_bound_covers_every_scale_in_the_lagging_range(case):
    """The bound is taken at the least favourable factor the reading allows
    (the row maximum at 1). Rounding after any larger power-of-two factor
    that keeps the row maximum within 2^8 stays inside the same bound, so it
    does not depend on which factor an implementation picks."""
    q, k, v, scale = _case(*case[:5], std_q=case[5], dominant=case[6])
    causal = case[4]
    rows = np.arange(q.shape[0])
    o, _ = oracle.attention_rows(q, k, v, rows, causal, scale)
    bound = F.pv_rounding_bound(q, k, v, rows, causal, scale)
    p, l = _probs(q, k, causal, scale)
    for e in range(0, 9):
        f = 2.0 ** e
        assert (f * p).max() <= F.P_MAX
        o_f = (rne_e4m3(f * p) / f) @ v / l[:, None]
        assert (np.abs(o_f - o) <= bound * (1 + 1e-9) + 1e-15).all(), e
    # and a bound taken at a larger factor is tighter: the factor matters to
    # the bound only through the absolute term
    tighter = F.pv_rounding_bound(q, k, v, rows, causal, scale, p_scale=64.0)
    assert (tighter <= bound).all()


def test_reading_constants():
    """The reading's constants: E4M3 (3 mantissa bits, smallest normal 2^-6,
    subnormal spacing 2^-9, largest 448) and V41's range (0, 2^8]."""
    assert F.REL_HALF_ULP == 2.0 ** -4 and F.ABS_HALF_ULP == 2.0 ** -10
    assert F.P_MAX == 2.0 ** 8 and F.P_MAX < 448 and F.P_SCALE == 1.0
    # the largest finite E4M3 code decodes to 448
    assert W.decode(np.array([0x7E], np.uint8), W.E4M3)[0] == 448.0


def test_bound_needs_its_absolute_term(monkeypatch):
    """With most probabilities below the normal range the relative term alone fails."""
    q, k, v, scale = _case(15, 64, 256, 64, False, dominant=True)
    rows = np.arange(q.shape[0])
    p, l = _probs(q, k, False, scale)
    worst = (half_ulp_e4m3(F.P_SCALE * p) / F.P_SCALE) @ np.abs(v) / l[:, None]
    monkeypatch.setattr(F, "ABS_HALF_ULP", 0.0)
    bound = F.pv_rounding_bound(q, k, v, rows, False, scale)
    assert (worst > bound * (1 + 1e-9)).any()


def test_bound_needs_its_full_relative_term(monkeypatch):
    q, k, v, scale = _case(11, 64, 64, 64, False)
    rows = np.arange(q.shape[0])
    p, l = _probs(q, k, False, scale)
    worst = (half_ulp_e4m3(F.P_SCALE * p) / F.P_SCALE) @ np.abs(v) / l[:, None]
    monkeypatch.setattr(F, "REL_HALF_ULP", F.REL_HALF_ULP / 2)
    bound = F.pv_rounding_bound(q, k, v, rows, False, scale)
    assert (worst > bound * (1 + 1e-9)).any()


def test_bound_follows_the_causal_mask():
    """Keys a row cannot see add nothing to its bound."""
    q, k, v, scale = _case(12, 96, 160, 64, True)
    rows = np.arange(96)
    b = F.pv_rounding_bound(q, k, v, rows, True, scale)
    v2 = v.copy()
    v2[100:] *= 1000  # keys 100.. are visible only from row 36 on (offset 64)
    b2 = F.pv_rounding_bound(q, k, v2, rows, True, scale)
    np.testing.assert_array_equal(b2[:36], b[:36])
    assert (b2[36:] > b[36:]).all()


def test_bound_is_zero_for_rows_that_see_no_key():
    q, k, v, scale = _case(16, 48, 20, 32, True)
    b = F.pv_rounding_bound(q, k, v, np.arange(48), True, scale)
    assert (b[:28] == 0).all() and (b[28:] > 0).all()
