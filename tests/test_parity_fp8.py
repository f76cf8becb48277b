"""GPU parity of the 8-bit (E4M3) forward against the float64 oracle.

The oracle is exact attention of the decoded codes times their descales.
The kernel rounds the probabilities to E4M3 before the P V product, so O is
compared per element against the rounding bound the oracle derives
(:func:`oracle.pv_rounding_bound`) plus the fp32 and bf16 terms:

    |O_gpu - O| <= bound + 2^-10 * sum_j Pn_ij |V_jd| + 2^-8 |O| + 1e-6

(2^-10 covers fp32 accumulation over up to 2^14 keys and the fp32 logits'
effect on P; 2^-8 is half an ulp of the bf16 output). lse is not affected
by the P rounding and keeps the 16-bit path's tolerance.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_16_amd as fa
import oracle
import oracle.fp8 as F
import workloads as W
from gpu_util import LSE_TOL, device, max_abs_err, sample_rows

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(msg, flush=True)


def _dev(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes)).to(device())


def _inputs(shape, seed, stds=(1.0, 1.0, 1.0)):
    """Per-tensor scaled E4M3 codes and descales of N(0, std^2) draws."""
    rng = np.random.default_rng(seed)
    out = [W.quantize_e4m3(std * rng.standard_normal(shape).astype(np.float32)) for std in stds]
    return tuple(c for c, _ in out), tuple(d for _, d in out)


def _tolerance(q, k, v, rows, causal, scale, o_ref):
    bound = oracle.pv_rounding_bound(q, k, v, rows, causal, scale)
    weighted = oracle.pv_rounding_bound(q, k, v, rows, causal, scale,
                                        p_scale=math.inf) / F.REL_HALF_ULP
    return bound + 2.0 ** -10 * weighted + 2.0 ** -8 * np.abs(o_ref) + 1e-6


def _check_head(codes, ds, o_gpu, lse_gpu, b, h, rows, causal, scale, tag):
    qc, kc, vc = codes
    q = W.decode(qc[b, h], W.E4M3) * ds[0]
    k = W.decode(kc[b, h], W.E4M3) * ds[1]
    v = W.decode(vc[b, h], W.E4M3) * ds[2]
    o_ref, l_ref = oracle.attention_rows(q, k, v, rows, causal, scale)
    tol = _tolerance(q, k, v, rows, causal, scale, o_ref)
    og = o_gpu[b, h, rows]
    assert np.isfinite(og).all(), tag
    err = np.abs(og - o_ref)
    ratio = float((err / tol).max())
    el = max_abs_err(lse_gpu[b, h, rows], l_ref)
    return ratio, float(err.max()), el


def _run(codes, ds, causal, scale=None):
    q, k, v = (_dev(c) for c in codes)
    o, lse = fa.attention_fp8(q, k, v, ds[0], ds[1], ds[2], causal, scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,S", [(1, 2, 128), (1, 2, 200), (2, 3, 300), (1, 1, 1),
                                   (1, 2, 513), (1, 1, 1024), (1, 1, 257)])
def test_fp8_all_rows(B, H, S, causal, D):
    tag = f"fp8 B={B} H={H} S={S} D={D} causal={causal}"
    _banner(tag)
    codes, ds = _inputs((B, H, S, D), 7000 + S + causal + D)
    scale = float(np.float32(1 / math.sqrt(D)))
    og, lg = _run(codes, ds, causal)
    worst = (0.0, 0.0, 0.0)
    for b in range(B):
        for h in range(H):
            r = _check_head(codes, ds, og, lg, b, h, np.arange(S), causal, scale, tag)
            worst = tuple(max(x, y) for x, y in zip(worst, r))
    _banner(f"{tag}: max |dO|/tol={worst[0]:.3f} max|dO|={worst[1]:.3e} max|dlse|={worst[2]:.3e}")
    assert worst[0] <= 1.0, (tag, worst)
    assert worst[2] <= LSE_TOL, (tag, worst)


@pytest.mark.parametrize("stds,scale", [((1.0, 1.0, 1.0), 0.5), ((0.01, 30.0, 1e-3), None),
                                        ((4.0, 4.0, 100.0), 0.02)])
def test_fp8_descales_and_scales(stds, scale):
    """Descales far from 1 and sharp or flat softmax: the descales fold into the
    logit multiplier and the output, not into the codes."""
    tag = f"fp8 stds={stds} scale={scale}"
    _banner(tag)
    codes, ds = _inputs((1, 2, 384, 128), 7100 + int(stds[2] * 10), stds)
    og, lg = _run(codes, ds, True, scale)
    s = float(np.float32(scale if scale is not None else 1 / math.sqrt(128)))
    worst = (0.0, 0.0, 0.0)
    for h in range(2):
        r = _check_head(codes, ds, og, lg, 0, h, np.arange(384), True, s, tag)
        worst = tuple(max(x, y) for x, y in zip(worst, r))
    _banner(f"{tag}: max |dO|/tol={worst[0]:.3f} max|dlse|={worst[2]:.3e}")
    assert worst[0] <= 1.0 and worst[2] <= LSE_TOL, (tag, worst)


def test_fp8_float8_tensors_equal_uint8_codes():
    codes, ds = _inputs((1, 2, 256, 128), 7200)
    q, k, v = (_dev(c) for c in codes)
    o1, l1 = fa.attention_fp8(q, k, v, *ds, True)
    o2, l2 = fa.attention_fp8(*(t.view(torch.float8_e4m3fn) for t in (q, k, v)), *ds, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fp8_full_size_sampled_rows():
    """The 8-bit long-context workload (2 x 16 heads x 8192 x 128, causal) in
    the launch the benchmark times, checked on sampled rows of several heads."""
    w = W.WORKLOADS["long8"]
    _banner(f"fp8 full size {w.B}x{w.H}x{w.S}x{w.D}")
    codes, ds = W.make_fp8_inputs(w)
    og, lg = _run(codes, ds, w.causal)
    worst = (0.0, 0.0, 0.0)
    for b, h in [(0, 0), (0, 7), (1, 8), (1, 15)]:
        rows = sample_rows(w.S, 24, seed=b * 16 + h, block_m=256)
        r = _check_head(codes, ds, og, lg, b, h, rows, w.causal, w.scale, "full")
        worst = tuple(max(x, y) for x, y in zip(worst, r))
    _banner(f"fp8 full size: max |dO|/tol={worst[0]:.3f} max|dO|={worst[1]:.3e} "
            f"max|dlse|={worst[2]:.3e}")
    assert worst[0] <= 1.0 and worst[2] <= LSE_TOL, worst
    assert np.isfinite(og).all() and np.isfinite(lg).all()


def test_fp8_head_dim_64_full_size_sampled_rows():
    """The batched non-causal shape (10 x 64 heads x 1024 x 64) in 8-bit."""
    w = W.WORKLOADS["bat8"]
    _banner(f"fp8 full size {w.B}x{w.H}x{w.S}x{w.D}")
    codes, ds = W.make_fp8_inputs(w)
    og, lg = _run(codes, ds, w.causal)
    worst = (0.0, 0.0, 0.0)
    for b, h in [(0, 0), (3, 17), (9, 63)]:
        rows = sample_rows(w.S, 24, seed=100 + b * 64 + h, block_m=256)
        r = _check_head(codes, ds, og, lg, b, h, rows, w.causal, w.scale, "bat8")
        worst = tuple(max(x, y) for x, y in zip(worst, r))
    _banner(f"fp8 D=64 full size: max |dO|/tol={worst[0]:.3f} max|dlse|={worst[2]:.3e}")
    assert worst[0] <= 1.0 and worst[2] <= LSE_TOL, worst


def test_fp8_stream_and_repeat_are_deterministic():
    codes, ds = _inputs((2, 4, 640, 128), 7300)
    q, k, v = (_dev(c) for c in codes)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o1, l1 = fa.attention_fp8(q, k, v, *ds, True, stream=s)
    s.synchronize()
    o2, l2 = fa.attention_fp8(q, k, v, *ds, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
