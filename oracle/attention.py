"""Exact attention, the plain definition, in float64 -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module; the product path never imports it.

What is computed (per batch b and head h; Q, K, V are S x D):

    X     = scale * Q K^T                     (S x S logits, materialised)
    X_ij  = -inf  where causal and j > i      (key j visible iff j <= i)
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


def _causal_mask(x: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Key j is visible to query row i iff j <= i; hidden logits become -inf."""
    j = np.arange(x.shape[1])
    return np.where(j[None, :] > rows[:, None], -np.inf, x)


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
                   causal: bool, scale: float):
    """O and LSE for selected query rows of one head (q, k, v: S x D float64).

    Each row of attention depends only on its own query, so a subset of rows is
    the definition restricted to those rows. Returns (O[R, D], lse[R]).
    """
    rows = np.asarray(rows, dtype=np.int64)
    x = _logits(q[rows], k, scale)
    if causal:
        x = _causal_mask(x, rows)
    m = _row_max(x)
    p = _exp_shifted(x, m)
    l = _row_sum(p)
    o = _normalise(p @ v, l)
    return o, _lse(m, l)


def attention_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool,
                  scale: float):
    """O and LSE for all rows; q, k, v of shape (..., S, D) in float64.

    Returns O of shape (..., S, D) and lse of shape (..., S), float64.
    One head at a time is materialised (an S x S float64 matrix).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lead = q.shape[:-2]
    S, D = q.shape[-2:]
    qf = q.reshape(-1, S, D)
    kf = k.reshape(-1, S, D)
    vf = v.reshape(-1, S, D)
    o = np.empty_like(qf)
    lse = np.empty(qf.shape[:2], dtype=np.float64)
    for n in range(qf.shape[0]):
        o[n], lse[n] = attention_rows(qf[n], kf[n], vf[n], np.arange(S), causal, scale)
    return o.reshape(*lead, S, D), lse.reshape(*lead, S)


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

    q, k, v are sequences of rows (S x D). Follows the definition one scalar at
    a time: logits, max, exponentials, sum, weighted sum of values, logsumexp.
    Returns (O as a list of rows, lse as a list).
    """
    S = len(q)
    D = len(q[0])
    O, LSE = [], []
    for i in range(S):
        logits = []
        for j in range(S):
            if causal and j > i:
                continue
            dot = 0.0
            for d in range(D):
                dot += float(q[i][d]) * float(k[j][d])
            logits.append((j, scale * dot))
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
