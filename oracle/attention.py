"""Exact attention, the plain definition, in float64 -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module; the product path never imports it.

What is computed (per batch b and head h; Q is Sq x D, K and V are Sk x D):

    X     = scale * Q K^T                     (Sq x Sk logits, materialised)
    X_ij  = -inf  where causal and j > i + (Sk - Sq)
                                              (key j visible iff j <= i + Sk - Sq:
                                               the mask aligned to the last query
                                               and the last key; with Sq == Sk,
                                               j <= i)
    m_i   = max_j X_ij
    P_ij  = exp(X_ij - m_i),   l_i = sum_j P_ij
    O_i   = (sum_j P_ij V_j) / l_i
    lse_i = m_i + ln(l_i)                     (natural-log logsumexp of the
                                               scaled logits of row i)

Sources:
* The formula softmax(Q K^T / sqrt(d_k) + mask) V and "the causal mask keeps
  the lower triangle": xdnf.cn, "CUDA手写masked multi-head attention性能优化
  实战", section 3.1 (masked attention math).
* Row statistics m (max) and l (sum) of the softmax: hotdry.top,
  "FlashAttention的Triton性能考古学", section "核心算法回顾".
* The row logsumexp output is not defined on the pages; it is taken here as
  the natural-log logsumexp of the scaled logits (a reading, not a quote).
* The pages' causal mask is square. For Sq != Sk the mask is read as aligned
  to the bottom-right corner (the last query sees every key), and a query
  that sees no key (possible when Sk < Sq) is given O = 0 and lse = -inf
  (readings; the pages are silent). Sequences of different lengths (the
  dynamic-shape dispatch of the xdnf.cn page, section 6.3) are each the
  definition applied to their own rows.

Each step of the definition is its own small function so that a reader can
check it against the formula above, and so that the pin tests can plant a
mistake in exactly one step.

Inputs are float64 arrays holding exactly the 16-bit values given to the GPU
(decode them with ``workloads.decode``); ``scale`` should be the float32
value the GPU receives, widened to float64.
"""
from __future__ import annotations

import math

import numpy as np


def _logits(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """X = scale * Q K^T for the given query rows against all keys."""
    return scale * (q @ k.T)


def _causal_mask(x: np.ndarray, rows: np.ndarray, offset: int = 0) -> np.ndarray:
    """Key j is visible to query row i iff j <= i + offset; hidden logits become -inf."""
    j = np.arange(x.shape[1])
    return np.where(j[None, :] > rows[:, None] + offset, -np.inf, x)


def _row_max(x: np.ndarray) -> np.ndarray:
    """m_i = max_j X_ij."""
    return x.max(axis=1)


def _exp_shifted(x: np.ndarray, m: np.ndarray) -> np.ndarray:
    """P_ij = exp(X_ij - m_i) (natural base)."""
    return np.exp(x - m[:, None])


def _row_sum(p: np.ndarray) -> np.ndarray:
    """l_i = sum_j P_ij."""
    return p.sum(axis=1)


def _normalise(acc: np.ndarray, l: np.ndarray) -> np.ndarray:
    """O_i = (P V)_i / l_i."""
    return acc / l[:, None]


def _lse(m: np.ndarray, l: np.ndarray) -> np.ndarray:
    """lse_i = m_i + ln(l_i)."""
    return m + np.log(l)


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows,
                   causal: bool, scale: float, offset: int | None = None):
    """O and LSE for selected query rows of one head (q: Sq x D, k, v: Sk x D).

    Each row of attention depends only on its own query, so a subset of rows is
    the definition restricted to those rows. ``offset`` is the causal
    alignment (key j visible to row i iff j <= i + offset); by default
    Sk - Sq. Rows that see no key get O = 0 and lse = -inf.
    Returns (O[R, D], lse[R]).
    """
    rows = np.asarray(rows, dtype=np.int64)
    if offset is None:
        offset = k.shape[0] - q.shape[0]
    D = q.shape[1]
    if k.shape[0] == 0:
        return np.zeros((len(rows), D)), np.full(len(rows), -np.inf)
    x = _logits(q[rows], k, scale)
    if causal:
        x = _causal_mask(x, rows, offset)
    seen = np.isfinite(x).any(axis=1)  # rows that see at least one key
    o = np.zeros((len(rows), D))
    lse = np.full(len(rows), -np.inf)
    if seen.any():
        xs = x[seen]
        m = _row_max(xs)
        p = _exp_shifted(xs, m)
        l = _row_sum(p)
        o[seen] = _normalise(p @ v, l)
        lse[seen] = _lse(m, l)
    return o, lse


def attention_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool,
                  scale: float):
    """O and LSE for all rows; q of shape (..., Sq, D), k and v (..., Sk, D), float64.

    Returns O of shape (..., Sq, D) and lse of shape (..., Sq), float64.
    One head at a time is materialised (an Sq x Sk float64 matrix).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lead = q.shape[:-2]
    Sq, D = q.shape[-2:]
    Sk = k.shape[-2]
    n = int(np.prod(lead, dtype=np.int64))
    qf = q.reshape(n, Sq, D)
    kf = k.reshape(n, Sk, D)
    vf = v.reshape(n, Sk, D)
    o = np.empty_like(qf)
    lse = np.empty(qf.shape[:2], dtype=np.float64)
    for n in range(qf.shape[0]):
        o[n], lse[n] = attention_rows(qf[n], kf[n], vf[n], np.arange(Sq), causal, scale)
    return o.reshape(*lead, Sq, D), lse.reshape(*lead, Sq)


def attention_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_q, cu_k,
                     causal: bool, scale: float):
    """Sequences packed along a token axis, each attending only to itself.

    q: [total_q, H, D], k and v: [total_k, H, D] float64; cu_q, cu_k: B+1
    token offsets. Sequence b is query tokens cu_q[b] .. cu_q[b+1]-1 against
    key tokens cu_k[b] .. cu_k[b+1]-1, each head the definition above (causal
    masks aligned bottom-right within the sequence). Returns O [total_q, H, D]
    and lse [H, total_q].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    total_q, H, D = q.shape
    o = np.zeros((total_q, H, D))
    lse = np.full((H, total_q), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 == q0:
            continue
        for h in range(H):
            ob, lb = attention_rows(q[q0:q1, h], k[k0:k1, h], v[k0:k1, h],
                                    np.arange(q1 - q0), causal, scale)
            o[q0:q1, h] = ob
            lse[h, q0:q1] = lb
    return o, lse


def attention_probs(q: np.ndarray, k: np.ndarray, causal: bool, scale: float):
    """Normalised attention weights P / l for one head (S x S float64)."""
    rows = np.arange(q.shape[0])
    x = _logits(q, k, scale)
    if causal:
        x = _causal_mask(x, rows)
    m = _row_max(x)
    p = _exp_shifted(x, m)
    return p / _row_sum(p)[:, None]


def attention_bruteforce(q, k, v, causal: bool, scale: float):
    """Pure-Python loops with math.exp / math.log, for tiny single-head inputs.

    q is a sequence of Sq rows, k and v of Sk rows (D values each). Follows
    the definition one scalar at a time: logits, max, exponentials, sum,
    weighted sum of values, logsumexp. A causal query i sees key j iff
    j - i <= Sk - Sq; a query that sees no key gives a zero row and -inf.
    Returns (O as a list of rows, lse as a list).
    """
    Sq, Sk = len(q), len(k)
    D = len(q[0])
    O, LSE = [], []
    for i in range(Sq):
        logits = []
        for j in range(Sk):
            if causal and j - i > Sk - Sq:
                continue
            dot = 0.0
            for d in range(D):
                dot += float(q[i][d]) * float(k[j][d])
            logits.append((j, scale * dot))
        if not logits:
            O.append([0.0] * D)
            LSE.append(-math.inf)
            continue
        m = max(x for _, x in logits)
        w = [(j, math.exp(x - m)) for j, x in logits]
        l = sum(p for _, p in w)
        row = []
        for d in range(D):
            acc = 0.0
            for j, p in w:
                acc += p * float(v[j][d])
            row.append(acc / l)
        O.append(row)
        LSE.append(m + math.log(l))
    return O, LSE
