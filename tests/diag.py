"""ctypes binding of the diagnostic library (libfa_fwd_diag.so, declared in
include/fa_fwd_diag.h), used by the tests only: the production kernels with
a rescale-event counter, the lag threshold at 8 or 0, and a forced kernel
choice. Argument marshalling only; the library has no fallback."""
from __future__ import annotations

import ctypes
import os

import exact_attention_16_amd as fa
from exact_attention_16_amd import _lib

DIAG_PATH = os.path.join(os.path.dirname(fa.LIB_PATH), "libfa_fwd_diag.so")

# kernel choice (the variant argument)
VARIANT_AUTO = 0
VARIANT_FOUR_WAVE = 1
VARIANT_PING_PONG = 2
VARIANT_PERSISTENT = 5
VARIANT_SPLIT = 7
VARIANT_OCC4 = 8

SIGNATURES = {"fa_fwd_diag": (ctypes.c_int, _lib._FWD_ARGS + [ctypes.c_int] * 3 + [ctypes.c_void_p])}

_diag = None


def load_diag() -> ctypes.CDLL:
    global _diag
    if _diag is None:
        if not os.path.exists(DIAG_PATH):
            raise RuntimeError(f"{DIAG_PATH} is not built; run `python -m exact_attention_16_amd.build`")
        lib = ctypes.CDLL(DIAG_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _diag = lib
    return _diag


def fa_fwd_diag(q, k, v, o, lse, B, H, S, D, causal, scale, stream, dtype, threshold_log2,
                variant, rescale_events, check=True):
    st = load_diag().fa_fwd_diag(q, k, v, o, lse, B, H, S, D, int(causal), scale, stream, dtype,
                                 threshold_log2, variant, rescale_events)
    if check and st != 0:
        raise fa.FaError(st, "fa_fwd_diag")
    return st
