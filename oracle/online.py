"""Streaming attention with a lagging running max -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module; the product path never imports it.

This is the algorithm, not the definition: float64, one head, the steps in
the order the pages give them. It exists to pin two facts about the method
independently of the GPU: (1) letting the running max lag by a threshold
does not change the exact result, and (2) how many times per row the
rescale actually fires for a given input (an expectation for the kernel's
diagnostic counter).

Algorithm (FA2 loop order: one block of query rows stays resident, key/value
blocks stream past it, normalisation happens once at the end -- hotdry.top,
"FlashAttention的Triton性能考古学", section "FlashAttention v2：循环重构与寄存
器积累"; running max m and sum l -- same page, "核心算法回顾"):

For each key block, with c = scale * log2(e) and the per-row base b kept in
log2 units (hjcheng0602.cn, "Flash Attention CUDA Kernel 优化 ... G6", section
"V41: Conditional Scale", steps 1-8):

1. s = raw dot products q . k for the block (not yet scaled); masked -> -inf.
2. tile_max = max_j s.
3. candidate = max(b_old, tile_max * c).
4. Rebase test: if candidate <= b_old + threshold the base stays and the
   history factor is 1; otherwise b_new = candidate and the history factor is
   2^(b_old - b_new).
5. p = 2^(s * c - b) for every score; with the base lagging by at most the
   threshold, p lies in (0, 2^threshold].
6. row_sum = row_sum * history + sum_j p.
7. The output accumulator rows are multiplied by history (the rescale; only
   needed when some row rebased) and then accumulate p @ V.

At the end O = acc / row_sum and the natural-log logsumexp is
(b + log2(row_sum)) * ln 2.

Readings where the pages are silent: the base starts at -inf, so the first
block always rebases with history 2^-inf = 0 (not counted as a rescale
event); the threshold is in log2 units of the scaled logit and the test is
"<=" (no rebase at exactly b_old + threshold).
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)


def _rebase(b: np.ndarray, scaled_max: np.ndarray, threshold_log2: float):
    """Steps 3-4 for one tile: the candidate base max(b, scaled tile max); the
    base moves only when the candidate exceeds b + threshold. Returns the new
    base, the history factor 2^(b_old - b_new) (1 where the base stays; 0 on a
    row's first tile, whose base was -inf) and whether the move counts as a
    rescale (not on the first tile, where the accumulator is still zero)."""
    cand = np.maximum(b, scaled_max)
    rebase = cand > b + threshold_log2
    with np.errstate(invalid="ignore"):
        history = np.where(rebase, np.exp2(b - cand), 1.0)
    counted = rebase & np.isfinite(b)
    return np.where(rebase, cand, b), history, counted


def online_softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                             causal: bool, scale: float, block_n: int = 64,
                             threshold_log2: float = 8.0):
    """One head (q, k, v: S x D float64).

    Returns a dict with O (S x D), lse (S), rescales (per-row count of rebases
    after the first block), max_p (largest p seen) and min_history (smallest
    history factor applied by a counted rebase, or 1.0 if none).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    S, D = q.shape
    c = scale * LOG2E
    b = np.full(S, -np.inf)
    row_sum = np.zeros(S)
    acc = np.zeros((S, D))
    rescales = np.zeros(S, dtype=np.int64)
    max_p = 0.0
    min_history = 1.0
    rows = np.arange(S)
    for kv0 in range(0, S, block_n):
        kv1 = min(S, kv0 + block_n)
        s = q @ k[kv0:kv1].T                                   # step 1
        if causal:
            j = np.arange(kv0, kv1)
            s = np.where(j[None, :] > rows[:, None], -np.inf, s)
        tile_max = s.max(axis=1)                               # step 2
        b_new, history, counted = _rebase(b, tile_max * c, threshold_log2)  # steps 3-4
        rescales += counted
        if counted.any():
            min_history = min(min_history, float(history[counted].min()))
        b = b_new
        with np.errstate(invalid="ignore"):
            p = np.exp2(s * c - b[:, None])                    # step 5
        p = np.where(np.isneginf(s), 0.0, p)
        if p.size:
            max_p = max(max_p, float(p.max()))
        row_sum = row_sum * history + p.sum(axis=1)            # step 6
        acc = acc * history[:, None] + p @ v[kv0:kv1]          # step 7
    o = acc / row_sum[:, None]
    lse = (b + np.log2(row_sum)) * math.log(2.0)
    return {"o": o, "lse": lse, "rescales": rescales, "max_p": max_p,
            "min_history": min_history}
