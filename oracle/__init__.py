"""CPU oracle for the fused attention forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package. The product path
(the HIP library and its Python binding) never imports it, and this package
imports nothing from the product path: the two share no code. The only module
both sides use is ``workloads`` (seeded input generation, no attention
arithmetic).

Contents:

* :mod:`oracle.attention` -- the plain definition of exact attention in
  float64, materialising the full score matrix (also for query and key
  lengths that differ and for sequences packed along a token axis), plus a
  pure-Python brute force for tiny inputs.
* :mod:`oracle.fp8` -- exact attention of 8-bit float (E4M3) inputs with
  per-tensor descales, and the bound on how far rounding the probabilities
  to E4M3 before the P V product can move O.
* :mod:`oracle.online` -- the streaming (tiled, online-softmax) algorithm with
  the lagging-max conditional rescale, in float64, step by step in the pages'
  order. It is used to check that the lagging-max algebra reaches the plain
  definition and to predict how often the rescale fires.
"""
from .attention import (attention_fwd, attention_rows, attention_probs,
                        attention_bruteforce, attention_varlen)
from .fp8 import attention_fp8, pv_rounding_bound
from .online import online_softmax_attention

__all__ = ["attention_fwd", "attention_rows", "attention_probs",
           "attention_bruteforce", "attention_varlen", "online_softmax_attention",
           "attention_fp8", "pv_rounding_bound"]
