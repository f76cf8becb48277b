"""Pins for the CPU oracle: brute force, closed forms, invariants, a library
routine, and planted mistakes that the pins must catch.

Nothing here touches a GPU or the HIP library.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as OA
import oracle.online as OO
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("S", [1, 2, 3, 8, 17, 32])
@pytest.mark.parametrize("D", [1, 4, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_oracle_matches_bruteforce(S, D, causal):
    q, k, v = (_rand((S, D), s) for s in (11 * S + D, 12 * S + D, 13 * S + D))
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attention_fwd(q, k, v, causal, scale)
    ob, lb = oracle.attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), causal, scale)
    np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lb), rtol=0, atol=1e-12)


# ------------------------------------------------------------- closed forms

def _eval(expr):
    return float(eval(expr, {"__builtins__": {}}, {"e": math.e, "ln": math.log}))


def _golden_cases():
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
@pytest.mark.parametrize("causal", [False, True])
def test_oracle_closed_forms(case, causal):
    q, k, v = (np.array(case[n], dtype=np.float64) for n in ("q", "k", "v"))
    exp = case["causal" if causal else "noncausal"]
    o, lse = oracle.attention_fwd(q, k, v, causal, case["scale"])
    np.testing.assert_allclose(o, [[_eval(x) for x in r] for r in exp["o"]], atol=1e-14)
    np.testing.assert_allclose(lse, [_eval(x) for x in exp["lse"]], atol=1e-14)


# --------------------------------------------------------------- invariants

@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(causal):
    q, k = _rand((40, 16), 1), _rand((40, 16), 2)
    p = oracle.attention_probs(q, k, causal, 0.25)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
    if causal:
        assert np.all(np.triu(p, 1) == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_returns_constant(causal):
    q, k = _rand((33, 8), 3, std=3.0), _rand((33, 8), 4, std=3.0)
    v = np.full((33, 8), 0.7311)
    o, _ = oracle.attention_fwd(q, k, v, causal, 0.5)
    np.testing.assert_allclose(o, 0.7311, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("mag", [1.0, 400.0])
def test_identical_keys_mean_and_lse(causal, mag):
    """All keys equal: every visible key has the same weight.

    O_i is the mean of the visible V rows and lse_i = scale*q_i.k + ln(n_i).
    mag=400 makes the logits ~1e3 so that a missing max-subtraction overflows.
    """
    S, D = 24, 6
    q = _rand((S, D), 5) * mag
    kk = _rand((1, D), 6)
    k = np.repeat(kk, S, axis=0)
    v = _rand((S, D), 7)
    scale = 0.75
    o, lse = oracle.attention_fwd(q, k, v, causal, scale)
    n = np.arange(1, S + 1) if causal else np.full(S, S)
    mean = np.cumsum(v, axis=0) / n[:, None] if causal else np.repeat(v.mean(0, keepdims=True), S, 0)
    np.testing.assert_allclose(o, mean, atol=1e-11)
    np.testing.assert_allclose(lse, scale * (q @ kk[0]) + np.log(n), rtol=1e-13, atol=1e-9)


def test_causal_row0_is_v0():
    q, k, v = _rand((16, 8), 8), _rand((16, 8), 9), _rand((16, 8), 10)
    o, lse = oracle.attention_fwd(q, k, v, True, 0.3)
    np.testing.assert_array_equal(o[0], v[0])
    assert abs(lse[0] - 0.3 * float(q[0] @ k[0])) < 1e-14


def test_causal_rows_ignore_future_keys():
    S, D = 20, 8
    q, k, v = _rand((S, D), 11), _rand((S, D), 12), _rand((S, D), 13)
    o, lse = oracle.attention_fwd(q, k, v, True, 0.4)
    for i in (0, 5, 13):
        k2, v2 = k.copy(), v.copy()
        k2[i + 1:] = _rand((S - i - 1, D), 100 + i) * 50
        v2[i + 1:] = _rand((S - i - 1, D), 200 + i) * 50
        o2, lse2 = oracle.attention_fwd(q, k2, v2, True, 0.4)
        np.testing.assert_array_equal(o2[: i + 1], o[: i + 1])
        np.testing.assert_array_equal(lse2[: i + 1], lse[: i + 1])


@pytest.mark.parametrize("causal", [False, True])
def test_logit_shift(causal):
    """K += w shifts row i's logits by scale*q_i.w: O unchanged, lse moves by it."""
    S, D = 30, 8
    q, k, v = _rand((S, D), 14), _rand((S, D), 15), _rand((S, D), 16)
    w = _rand((D,), 17)
    scale = 0.35
    o, lse = oracle.attention_fwd(q, k, v, causal, scale)
    o2, lse2 = oracle.attention_fwd(q, k + w, v, causal, scale)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2 - lse, scale * (q @ w), atol=1e-12)


def test_attention_rows_equals_full():
    S, D = 50, 16
    q, k, v = _rand((S, D), 18), _rand((S, D), 19), _rand((S, D), 20)
    o, lse = oracle.attention_fwd(q, k, v, True, 0.25)
    rows = np.array([0, 7, 31, 49])
    orr, lr = oracle.attention_rows(q, k, v, rows, True, 0.25)
    np.testing.assert_allclose(orr, o[rows], atol=1e-14)
    np.testing.assert_allclose(lr, lse[rows], atol=1e-14)


def test_batched_shapes():
    q = _rand((2, 3, 10, 4), 21)
    k = _rand((2, 3, 10, 4), 22)
    v = _rand((2, 3, 10, 4), 23)
    o, lse = oracle.attention_fwd(q, k, v, True, 0.5)
    assert o.shape == (2, 3, 10, 4) and lse.shape == (2, 3, 10)
    o11, l11 = oracle.attention_fwd(q[1, 1], k[1, 1], v[1, 1], True, 0.5)
    np.testing.assert_array_equal(o[1, 1], o11)
    np.testing.assert_array_equal(lse[1, 1], l11)


# --------------------------------------------------- independent library routine

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S,D", [(64, 64), (200, 128), (129, 64)])
def test_oracle_matches_torch_cpu_float64(causal, S, D):
    """torch's CPU attention kernel (float64) returns O and the natural-log LSE."""
    shape = (2, 3, S, D)
    q, k, v = _rand(shape, 24), _rand(shape, 25), _rand(shape, 26)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attention_fwd(q, k, v, causal, scale)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    to, tl = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        tq, tk, tv, 0.0, causal, scale=scale)[:2]
    np.testing.assert_allclose(o, to.numpy(), atol=1e-10)
    np.testing.assert_allclose(lse, tl.numpy(), atol=1e-10)
    to2 = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    np.testing.assert_allclose(o, to2.numpy(), atol=1e-10)


def test_oracle_on_tiny_workload_16bit_inputs():
    """The tiny workload's 16-bit inputs, decoded exactly, against torch float64."""
    w = W.WORKLOADS["tiny"]
    q, k, v = (W.decode(x, w.dtype) for x in W.make_inputs(w))
    for causal in (False, True):
        o, lse = oracle.attention_fwd(q, k, v, causal, w.scale)
        to, tl = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
            *(torch.from_numpy(x) for x in (q, k, v)), 0.0, causal, scale=w.scale)[:2]
        np.testing.assert_allclose(o, to.numpy(), atol=1e-11)
        np.testing.assert_allclose(lse, tl.numpy(), atol=1e-11)


# ------------------------------------------------ streaming algorithm (lagging max)

def _lazy_golden():
    with open(os.path.join(GOLDEN, "lazy_rescale.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("threshold", [0.0, 8.0])
def test_online_lagging_max_reaches_definition(causal, threshold):
    S, D = 300, 32
    q, k, v = _rand((S, D), 27), _rand((S, D), 28), _rand((S, D), 29)
    # a key ramp makes row maxima rise along the key axis
    u = _rand((D,), 30)
    u /= np.linalg.norm(u)
    k = k + 0.05 * np.arange(S)[:, None] * u
    q = q + u
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attention_fwd(q, k, v, causal, scale)
    r = oracle.online_softmax_attention(q, k, v, causal, scale, block_n=64,
                                        threshold_log2=threshold)
    np.testing.assert_allclose(r["o"], o, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse, atol=1e-12)
    g = _lazy_golden()
    if threshold == g["threshold_log2"]:
        assert 1.0 < r["max_p"] <= g["p_upper_bound"]
        assert r["min_history"] < g["history_when_rebased_at_most"]
        assert r["rescales"].sum() > 0
    else:
        assert r["max_p"] <= 1.0 + 1e-15


def test_online_threshold_reduces_rescales():
    S, D = 512, 32
    q, k, v = _rand((S, D), 31), _rand((S, D), 32), _rand((S, D), 33)
    eager = oracle.online_softmax_attention(q, k, v, True, 0.2, 64, 0.0)["rescales"].sum()
    lazy = oracle.online_softmax_attention(q, k, v, True, 0.2, 64, 8.0)["rescales"].sum()
    assert eager > 0 and lazy < eager / 10


def _rescale_golden():
    with open(os.path.join(GOLDEN, "rescale_counts.json")) as f:
        return json.load(f)


def _run_rescale_case(case, block_n):
    keys = np.array([x for t in case["tiles"] for x in t], dtype=np.float64)
    S = len(keys)
    q = np.ones((S, 1))
    k = keys[:, None]
    v = np.arange(S, dtype=np.float64)[:, None]
    return oracle.online_softmax_attention(q, k, v, False, math.log(2.0), block_n=block_n,
                                           threshold_log2=case["threshold_log2"])


def _rescale_golden_passes():
    g = _rescale_golden()
    assert math.log(2.0) * OO.LOG2E == 1.0  # the fixture's premise: ScaleLog2 is exactly 1
    for case in g["cases"]:
        r = _run_rescale_case(case, g["block_n"])
        if not (np.all(r["rescales"] == case["rescales_per_row"])
                and r["max_p"] == case["max_p"] and r["min_history"] == case["min_history"]):
            return False
    return True


def test_rescale_counts_match_the_hand_counted_cases():
    """The float64 model's rebase count is what the GPU's event counter is
    compared with; here it is pinned to cases counted by hand from the rule."""
    g = _rescale_golden()
    assert math.log(2.0) * OO.LOG2E == 1.0
    for case in g["cases"]:
        r = _run_rescale_case(case, g["block_n"])
        assert np.all(r["rescales"] == case["rescales_per_row"]), case["name"]
        assert r["max_p"] == case["max_p"], case["name"]
        assert r["min_history"] == case["min_history"], case["name"]
        # the result is still exact attention (the base cancels)
        keys = np.array([x for t in case["tiles"] for x in t])
        w = np.exp2(keys - keys.max())
        np.testing.assert_allclose(r["o"][:, 0], (w @ np.arange(len(keys))) / w.sum(),
                                   rtol=1e-12)


def _rebase_ge(b, m, thr):  # rebases at exactly b + threshold
    cand = np.maximum(b, m)
    rebase = cand >= b + thr
    with np.errstate(invalid="ignore"):
        hist = np.where(rebase, np.exp2(b - cand), 1.0)
    return np.where(rebase, cand, b), hist, rebase & np.isfinite(b)


def _rebase_first_counted(b, m, thr):  # the first tile counted as a rescale
    nb, hist, counted = _REBASE(b, m, thr)
    return nb, hist, counted | ~np.isfinite(b)


def _rebase_to_tile_max(b, m, thr):  # the base follows every tile's max, down as well
    nb = np.where(np.isfinite(m), m, b)
    with np.errstate(invalid="ignore"):
        hist = np.where(nb != b, np.exp2(b - nb), 1.0)
    return nb, hist, (nb != b) & np.isfinite(b)


def _rebase_history_inverted(b, m, thr):
    nb, hist, counted = _REBASE(b, m, thr)
    with np.errstate(divide="ignore"):
        return nb, np.where(counted, 1.0 / hist, hist), counted


_REBASE = OO._rebase
_REBASE_MUTANTS = {"rebase at exactly b + 8": _rebase_ge,
                   "first tile counted": _rebase_first_counted,
                   "base follows the tile max down": _rebase_to_tile_max,
                   "history inverted": _rebase_history_inverted}


@pytest.mark.parametrize("name", sorted(_REBASE_MUTANTS))
def test_planted_rebase_mistake_is_caught(name, monkeypatch):
    assert _rescale_golden_passes()
    monkeypatch.setattr(OO, "_rebase", _REBASE_MUTANTS[name])
    with np.errstate(all="ignore"):
        caught = not _rescale_golden_passes()
    assert caught, f"planted mistake not caught: {name}"


# ------------------------------------------- planted mistakes must fail a pin

def _pin_battery():
    """Brute force, closed forms and the overflow case; True if all pass."""
    try:
        for Sq, Sk, D, causal in ((8, 8, 4, False), (8, 8, 4, True), (5, 5, 3, True),
                                  (5, 8, 3, True), (8, 5, 3, True), (3, 7, 2, False)):
            q, k, v = _rand((Sq, D), 40 + Sq), _rand((Sk, D), 50 + Sk), _rand((Sk, D), 60 + Sk)
            o, lse = oracle.attention_fwd(q, k, v, causal, 0.6)
            ob, lb = oracle.attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), causal, 0.6)
            if not (np.allclose(o, ob, atol=1e-12, rtol=0)
                    and np.array_equal(np.isinf(lse), np.isinf(lb))
                    and np.allclose(np.nan_to_num(lse, neginf=0), np.nan_to_num(np.array(lb), neginf=0),
                                    atol=1e-12, rtol=0)):
                return False
        for case in _golden_cases():
            for causal in (False, True):
                q, k, v = (np.array(case[n]) for n in ("q", "k", "v"))
                exp = case["causal" if causal else "noncausal"]
                o, lse = oracle.attention_fwd(q, k, v, causal, case["scale"])
                if not np.allclose(o, [[_eval(x) for x in r] for r in exp["o"]], atol=1e-14, rtol=0):
                    return False
                if not np.allclose(lse, [_eval(x) for x in exp["lse"]], atol=1e-14, rtol=0):
                    return False
        # logits spread over thousands: any shift other than the row max
        # overflows or underflows exp (the max only guards the numeric range)
        q = _rand((6, 3), 70) * 2000
        k = np.repeat(_rand((1, 3), 71), 6, axis=0)
        v = _rand((6, 3), 72)
        with np.errstate(all="ignore"):
            o, lse = oracle.attention_fwd(q, k, v, True, 1.0)
        mean = np.cumsum(v, axis=0) / np.arange(1, 7)[:, None]
        return bool(np.allclose(o, mean, atol=1e-11) and np.all(np.isfinite(lse)))
    except Exception:
        return False


_MUTANTS = {
    "K and Q swapped in the logits": ("_logits", lambda q, k, scale: scale * (k @ q.T)),
    "scale dropped": ("_logits", lambda q, k, scale: q @ k.T),
    "mask hides the diagonal": ("_causal_mask", lambda x, rows, offset=0: np.where(
        np.arange(x.shape[1])[None, :] >= rows[:, None] + offset, -np.inf, x)),
    "mask keeps the upper triangle": ("_causal_mask", lambda x, rows, offset=0: np.where(
        np.arange(x.shape[1])[None, :] < rows[:, None] + offset, -np.inf, x)),
    "mask alignment offset ignored": ("_causal_mask", lambda x, rows, offset=0: np.where(
        np.arange(x.shape[1])[None, :] > rows[:, None], -np.inf, x)),
    "mask alignment offset negated": ("_causal_mask", lambda x, rows, offset=0: np.where(
        np.arange(x.shape[1])[None, :] > rows[:, None] - offset, -np.inf, x)),
    "max over the wrong axis": ("_row_max", lambda x: x.max(axis=0)),
    "max subtraction dropped": ("_row_max", lambda x: np.zeros(x.shape[0])),
    "exponent sign flipped": ("_exp_shifted", lambda x, m: np.exp(-(x - m[:, None]))),
    "base-2 exponential": ("_exp_shifted", lambda x, m: np.exp2(x - m[:, None])),
    "sum over the wrong axis": ("_row_sum", lambda p: p.sum(axis=0)),
    "normalisation dropped": ("_normalise", lambda acc, l: acc),
    "lse log term dropped": ("_lse", lambda m, l: m),
    "lse in log2": ("_lse", lambda m, l: m + np.log2(l)),
    "lse sign flipped": ("_lse", lambda m, l: m - np.log(l)),
}


def test_pin_battery_passes_on_the_oracle():
    assert _pin_battery()


@pytest.mark.parametrize("name", sorted(_MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = _MUTANTS[name]
    monkeypatch.setattr(OA, attr, fn)
    assert not _pin_battery(), f"planted mistake not caught: {name}"


# ------------------------------------- query and key lengths that differ; varlen

@pytest.mark.parametrize("Sq,Sk", [(1, 5), (3, 8), (8, 3), (5, 1), (7, 7), (4, 9)])
@pytest.mark.parametrize("causal", [False, True])
def test_two_lengths_match_bruteforce(Sq, Sk, causal):
    """Scalar loops (key j visible iff j - i <= Sk - Sq) against the vectorised oracle."""
    D = 4
    q, k, v = _rand((Sq, D), 300 + Sq), _rand((Sk, D), 310 + Sk), _rand((Sk, D), 320 + Sk)
    o, lse = oracle.attention_fwd(q, k, v, causal, 0.7)
    ob, lb = oracle.attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), causal, 0.7)
    np.testing.assert_allclose(o, ob, atol=1e-12, rtol=0)
    assert np.array_equal(np.isneginf(lse), np.isneginf(np.array(lb)))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse[fin], np.array(lb)[fin], atol=1e-12, rtol=0)


@pytest.mark.parametrize("S,Sq", [(40, 1), (40, 13), (129, 64)])
def test_bottom_right_is_the_end_of_a_square_causal_problem(S, Sq):
    """Invariant: the last Sq queries of a square causal problem over S keys give the
    same rows as those Sq queries alone against all S keys (bottom-right mask)."""
    D = 16
    q, k, v = _rand((S, D), 330), _rand((S, D), 331), _rand((S, D), 332)
    o_full, l_full = oracle.attention_fwd(q, k, v, True, D ** -0.5)
    o, l = oracle.attention_fwd(q[S - Sq:], k, v, True, D ** -0.5)
    np.testing.assert_allclose(o, o_full[S - Sq:], atol=1e-13, rtol=0)
    np.testing.assert_allclose(l, l_full[S - Sq:], atol=1e-13, rtol=0)


@pytest.mark.parametrize("Sq,Sk", [(64, 96), (96, 64), (33, 200)])
@pytest.mark.parametrize("causal", [False, True])
def test_two_lengths_match_torch_sdpa_with_explicit_mask(Sq, Sk, causal):
    """Library pin: torch's scaled_dot_product_attention (CPU, float64) with the
    bottom-right mask given explicitly, on the rows that see at least one key."""
    D = 32
    q, k, v = _rand((Sq, D), 340), _rand((Sk, D), 341), _rand((Sk, D), 342)
    o, lse = oracle.attention_fwd(q, k, v, causal, D ** -0.5)
    mask = torch.ones(Sq, Sk, dtype=torch.bool)
    if causal:
        mask = mask.tril(diagonal=Sk - Sq)
    seen = mask.any(dim=1).numpy()
    t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=mask[None], scale=D ** -0.5)[0].numpy()
    np.testing.assert_allclose(o[seen], t[seen], atol=1e-12, rtol=0)
    ref_lse = np.logaddexp.reduce(np.where(mask.numpy(), (q @ k.T) * D ** -0.5, -np.inf), axis=1)
    np.testing.assert_allclose(lse[seen], ref_lse[seen], atol=1e-12, rtol=0)


def test_rows_that_see_no_key():
    """Reading: a causal query with no visible key (Sk < Sq, its first Sq - Sk
    rows) returns a zero row and lse = -inf; with Sk = 0 every row does."""
    q, k, v = _rand((6, 3), 350), _rand((2, 3), 351), _rand((2, 3), 352)
    o, lse = oracle.attention_fwd(q, k, v, True, 1.0)
    assert np.all(o[:4] == 0) and np.all(np.isneginf(lse[:4]))
    assert np.all(np.isfinite(lse[4:]))
    o0, l0 = oracle.attention_fwd(q, np.zeros((0, 3)), np.zeros((0, 3)), False, 1.0)
    assert np.all(o0 == 0) and np.all(np.isneginf(l0))


def test_varlen_of_equal_lengths_is_the_batch():
    """Packing a [B, H, S, D] batch along the token axis with offsets 0, S, 2S, ...
    gives attention_fwd's result, rearranged."""
    B, H, S, D = 3, 2, 20, 8
    q, k, v = _rand((B, H, S, D), 360), _rand((B, H, S, D), 361), _rand((B, H, S, D), 362)
    cu = np.arange(B + 1) * S
    pack = lambda t: t.transpose(0, 2, 1, 3).reshape(B * S, H, D)
    for causal in (False, True):
        o, lse = oracle.attention_fwd(q, k, v, causal, 0.3)
        ov, lv = oracle.attention_varlen(pack(q), pack(k), pack(v), cu, cu, causal, 0.3)
        np.testing.assert_allclose(ov, pack(o), atol=1e-14, rtol=0)
        np.testing.assert_allclose(lv, lse.transpose(1, 0, 2).reshape(H, B * S), atol=1e-14, rtol=0)


def test_varlen_sequences_do_not_see_each_other():
    """Each sequence equals a separate call on its own rows; empty sequences and
    Sq != Sk per sequence included."""
    H, D = 2, 8
    lq, lk = [5, 0, 17, 3, 9], [5, 4, 17, 8, 2]
    cq, ck = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q, k, v = _rand((cq[-1], H, D), 370), _rand((ck[-1], H, D), 371), _rand((ck[-1], H, D), 372)
    for causal in (False, True):
        o, lse = oracle.attention_varlen(q, k, v, cq, ck, causal, 0.4)
        for b in range(len(lq)):
            qs, ks = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
            for h in range(H):
                ob, lb = oracle.attention_fwd(q[qs, h], k[ks, h], v[ks, h], causal, 0.4)
                np.testing.assert_array_equal(o[qs, h], ob)
                np.testing.assert_array_equal(lse[h, qs], lb)
