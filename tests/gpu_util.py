"""Helpers shared by the GPU tests: move seeded 16-bit inputs to the device,
run the HIP path through the C ABI, and compare with the CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

import exact_attention_16_amd as fa
import oracle
import workloads as W
from diag import fa_fwd_diag

# Tolerances stated for this path: max |O_gpu - O| over all elements, and
# max |lse_gpu - lse|, against the float64 oracle on the same 16-bit inputs.
O_TOL = {W.F16: 5e-3, W.BF16: 2e-2}
LSE_TOL = 1e-3

TORCH_DT = {W.F16: torch.float16, W.BF16: torch.bfloat16}


def device():
    return torch.device("cuda:0")


def to_dev(bits: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(TORCH_DT[dtype]).to(device())


def run(qb, kb, vb, dtype, causal, scale, stream=None, variant=None):
    """fa_fwd on the seeded bits; returns device tensors (o, lse).

    variant None: fa_fwd (the kernel it picks for the shape). Otherwise
    fa_fwd_diag with that kernel choice (diag.VARIANT_*), production threshold.
    """
    q, k, v = (to_dev(x, dtype) for x in (qb, kb, vb))
    if variant is None:
        o, lse = fa.attention(q, k, v, causal, scale, stream=stream)
    else:
        assert stream is None
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=device())
        ev = torch.zeros(1, dtype=torch.int64, device=device())
        B, H, S, D = q.shape
        fa_fwd_diag(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       B, H, S, D, int(causal), scale, torch.cuda.current_stream().cuda_stream,
                       W.DTYPE_CODE[dtype], 8, variant, ev.data_ptr())
    torch.cuda.synchronize()
    return o, lse


def o_to_f64(o: torch.Tensor) -> np.ndarray:
    return o.float().cpu().numpy().astype(np.float64)


def max_abs_err(got, ref) -> float:
    """max |got - ref| where a NaN anywhere counts as an infinite error (so it
    can never pass a tolerance) and equal infinities (lse = -inf for a row that
    sees no key, on both sides) count as no error."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    same_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    with np.errstate(invalid="ignore"):
        d = np.where(same_inf, 0.0, np.abs(got - ref))
    d = np.where(np.isnan(d), np.inf, d)
    return float(d.max()) if d.size else 0.0


def compare_rows(qb, kb, vb, dtype, causal, scale, o_gpu, lse_gpu, heads_rows):
    """Max errors of the GPU result against the oracle on selected rows.

    heads_rows: iterable of ((b, h), rows). Returns (max_abs_O, max_abs_lse);
    a NaN on either side makes the error infinite.
    """
    eo = el = 0.0
    scale = float(np.float32(scale))  # the value the kernel receives
    for (b, h), rows in heads_rows:
        rows = np.asarray(rows)
        q = W.decode(qb[b, h], dtype)
        k = W.decode(kb[b, h], dtype)
        v = W.decode(vb[b, h], dtype)
        o_ref, l_ref = oracle.attention_rows(q, k, v, rows, causal, scale)
        eo = max(eo, max_abs_err(o_gpu[b, h, rows], o_ref))
        el = max(el, max_abs_err(lse_gpu[b, h, rows], l_ref))
    return eo, el


def sample_rows(S: int, n: int, seed: int, block_m: int = 128) -> np.ndarray:
    """Rows 0, 1, the ends of query tiles, S-1, plus n random rows."""
    rng = np.random.default_rng(seed)
    fixed = {0, 1, 2, 31, 32, 63, 64, S - 1, S - 2}
    for t in range(0, S, block_m * max(1, S // (block_m * 8))):
        fixed.update({t, t + block_m - 1})
    rows = np.array(sorted(r for r in fixed if 0 <= r < S))
    extra = rng.choice(S, size=min(n, S), replace=False)
    return np.unique(np.concatenate([rows, extra]))
