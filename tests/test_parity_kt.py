"""GPU parity of fa_fwd_kt (K given transposed, [B, H, D, S]) against the
float64 oracle on the same 16-bit values, with the dense path's tolerances.
The oracle takes K as [S, D]; the test transposes it for the kernel."""
import math

import numpy as np
import pytest
import torch

import exact_attention_16_amd as fa
import oracle
import workloads as W
from gpu_util import LSE_TOL, O_TOL, compare_rows, device, o_to_f64, sample_rows, to_dev

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(msg, flush=True)


def _run_kt(qb, kb, vb, dtype, causal, scale):
    q, k, v = (to_dev(x, dtype) for x in (qb, kb, vb))
    kt = k.transpose(-1, -2).contiguous()
    o, lse = fa.attention_kt(q, kt, v, causal, scale)
    torch.cuda.synchronize()
    return o_to_f64(o), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [8, 64, 200, 264, 520])
def test_kt_all_rows(S, causal, D, dtype):
    tag = f"kt S={S} D={D} {dtype} causal={causal}"
    _banner(tag)
    shape = (1, 2, S, D)
    seed = 8000 + S + D + causal + (dtype == W.BF16)
    qb, kb, vb = (W.random_bits(shape, dtype, seed + i) for i in range(3))
    scale = float(np.float32(1 / math.sqrt(D)))
    og, lg = _run_kt(qb, kb, vb, dtype, causal, scale)
    o_ref, l_ref = oracle.attention_fwd(W.decode(qb, dtype), W.decode(kb, dtype),
                                        W.decode(vb, dtype), causal, scale)
    assert np.isfinite(og).all() and np.isfinite(lg).all(), tag
    eo, el = float(np.abs(og - o_ref).max()), float(np.abs(lg - l_ref).max())
    _banner(f"{tag}: max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= O_TOL[dtype] and el <= LSE_TOL, (tag, eo, el)


def test_kt_agrees_with_row_major_k():
    dt, shape = W.BF16, (2, 4, 1000, 128)
    qb, kb, vb = (W.random_bits(shape, dt, 8100 + i) for i in range(3))
    og, lg = _run_kt(qb, kb, vb, dt, True, 128 ** -0.5)
    q, k, v = (to_dev(x, dt) for x in (qb, kb, vb))
    o, lse = fa.attention(q, k, v, True, 128 ** -0.5)
    torch.cuda.synchronize()
    assert np.abs(og - o_to_f64(o)).max() <= O_TOL[dt]
    assert np.abs(lg - lse.cpu().numpy()).max() <= LSE_TOL


def test_kt_full_size_sampled_rows():
    """The long-context workload (2 x 16 heads x 8192 x 128, bf16, causal) with K
    given transposed, sampled rows against the oracle."""
    w = W.WORKLOADS["long"]
    _banner("kt full size long")
    qb, kb, vb = W.make_inputs(w)
    og, lg = _run_kt(qb, kb, vb, w.dtype, w.causal, w.scale)
    plan = [((b, h), sample_rows(w.S, 24, seed=40 + h, block_m=256))
            for b, h in [(0, 0), (1, 9), (1, 15)]]
    eo, el = compare_rows(qb, kb, vb, w.dtype, w.causal, w.scale, og, lg, plan)
    _banner(f"kt full size: max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= O_TOL[w.dtype] and el <= LSE_TOL


def test_kt_writes_only_its_outputs():
    B, H, S, D, dt = 1, 3, 136, 128, W.F16
    qb, kb, vb = (W.random_bits((B, H, S, D), dt, 8200 + i) for i in range(3))
    q, k, v = (to_dev(x, dt) for x in (qb, kb, vb))
    kt = k.transpose(-1, -2).contiguous()
    n, nl, g = B * H * S * D, B * H * S, 4096
    obuf = torch.full((n + 2 * g,), 7.0, dtype=torch.float16, device=device())
    lbuf = torch.full((nl + 2 * g,), -3.0, dtype=torch.float32, device=device())
    o, lse = obuf[g:g + n].view(B, H, S, D), lbuf[g:g + nl].view(B, H, S)
    fa.attention_kt(q, kt, v, True, D ** -0.5, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(obuf[:g] == 7.0) and torch.all(obuf[g + n:] == 7.0)
    assert torch.all(lbuf[:g] == -3.0) and torch.all(lbuf[g + nl:] == -3.0)
    assert torch.all(torch.isfinite(o)) and torch.all(torch.isfinite(lse))
