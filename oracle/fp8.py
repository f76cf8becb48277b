"""Attention on 8-bit float inputs, and the error bound of an 8-bit P -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module; the product path never imports it.

The 8-bit forward is the support for FP8 that the hotdry.top page,
"FlashAttention的Triton性能考古学", lists among the strategies for Ampere and
later GPUs (section "架构感知优化策略"). The page gives no details, so what
follows is a reading:

* Q, K and V arrive as E4M3FN codes with one float descale per tensor: the
  value of element x is decode(x) * descale. What the method should return is
  then exact attention (:mod:`oracle.attention`) of those values, and
  :func:`attention_fp8` is exactly that.
* A fast kernel also rounds the probabilities P to E4M3 before the P V
  product (it runs on the 8-bit matrix units). That rounding is an
  approximation, so the comparison needs a bound: :func:`pv_rounding_bound`.
  Reading (the pages fix no 8-bit P): the probabilities live in the range the
  lagging base gives them, p = 2^(s*c - b) in (0, 2^8] with b allowed to
  trail the running max by up to 8 binades (hjcheng0602.cn, "Flash Attention
  CUDA Kernel 优化 ... G6", section "V41: Conditional Scale"); 2^8 is below
  E4M3's largest value 448, so that range needs no clamping. Within it, a
  row's largest probability may sit anywhere in [1, 2^8]: at 1 right after a
  rebase, higher while b lags. The least favourable case for rounding is the
  smallest, 1 (more of the row's small probabilities then fall below E4M3's
  normal range), so the bound takes that: ``p_scale`` = 1 by default. An
  implementation that multiplies the probabilities by a larger power of two
  before rounding (while keeping them at or below 2^8) only tightens its own
  error; the bound does not depend on that choice. The row sum and the
  log-sum-exp use the unrounded probabilities.

Bound for one row i and one column d, in the units of the (descaled) V:
the rounding error of a normal E4M3 value is at most half its unit in the
last place, 2^-4 of its size (three mantissa bits); below 2^-6 the spacing
is 2^-9, so the error is at most 2^-10 in the scaled units, at most
2^-10 / p_scale in the units of P. Dividing by the row sum
L_i = sum_j exp(X_ij - m_i):

    |dO_id| <= sum_j |P^_ij - P_ij| |V_jd| / L_i
            <= 2^-4 sum_j Pn_ij |V_jd|  +  2^-10 / p_scale * sum_j |V_jd| / L_i

with Pn = P / L the normalised weights. (The factor a probability is
multiplied by may differ between key tiles as the running base moves; the
relative part does not depend on it and the absolute part only shrinks when
it is larger than p_scale.)
"""
from __future__ import annotations

import numpy as np

from .attention import (_causal_mask, _exp_shifted, _logits, _row_max, _row_sum,
                        attention_fwd)

# E4M3: three mantissa bits (relative half-ulp 2^-4), smallest normal 2^-6,
# subnormal spacing 2^-9 (absolute half-ulp 2^-10).
REL_HALF_ULP = 2.0 ** -4
ABS_HALF_ULP = 2.0 ** -10
# The smallest factor the reading allows on a row's probabilities before they
# are rounded: the largest probability at 1, right after a rebase.
P_SCALE = 1.0
# The largest value a scaled probability may take: 2^8, the top of the
# lagging base's range (V41), below E4M3's largest value 448.
P_MAX = 256.0


def attention_fp8(q: np.ndarray, k: np.ndarray, v: np.ndarray, descale, causal: bool,
                  scale: float):
    """Exact attention of decoded 8-bit inputs times their per-tensor descales.

    q, k, v: float64 arrays of decoded E4M3 values, shape (..., S, D);
    descale: (dq, dk, dv). Returns (O, lse) as :func:`oracle.attention_fwd`.
    """
    dq, dk, dv = (float(x) for x in descale)
    return attention_fwd(np.asarray(q) * dq, np.asarray(k) * dk, np.asarray(v) * dv,
                         causal, scale)


def pv_rounding_bound(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows, causal: bool,
                      scale: float, p_scale: float = P_SCALE, offset: int | None = None):
    """Largest change of O that rounding p_scale * P to E4M3 can cause (rows x D).

    q, k, v are the descaled float64 values of one head (Sq x D, Sk x D);
    ``offset`` is the causal alignment as in :func:`oracle.attention_rows`.
    Rows that see no key get 0.
    """
    rows = np.asarray(rows, dtype=np.int64)
    if offset is None:
        offset = k.shape[0] - q.shape[0]
    out = np.zeros((len(rows), q.shape[1]))
    if k.shape[0] == 0:
        return out
    x = _logits(np.asarray(q)[rows], k, scale)
    if causal:
        x = _causal_mask(x, rows, offset)
    seen = np.isfinite(x).any(axis=1)
    if not seen.any():
        return out
    xs = x[seen]
    p = _exp_shifted(xs, _row_max(xs))
    l = _row_sum(p)
    av = np.abs(v)
    visible = np.isfinite(xs).astype(np.float64)
    rel = REL_HALF_ULP * (p @ av) / l[:, None]
    absolute = (ABS_HALF_ULP / p_scale) * (visible @ av) / l[:, None]
    out[seen] = rel + absolute
    return out
