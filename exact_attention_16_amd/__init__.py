"""MI355X-native fused attention forward (gfx950 HIP kernels behind a C ABI).

The library (libfa_fwd.so, built in-tree by ``exact_attention_16_amd.build``)
is loaded lazily on first use; :mod:`exact_attention_16_amd._lib` holds the
ctypes binding with the C entry points' names.
"""
from ._lib import (FA_BF16, FA_F16, FaError, attention, attention_fp8, attention_kt,
                   attention_varlen, fa_fwd, fa_fwd_bf16, fa_fwd_f16, fa_fwd_fp8, fa_fwd_kt,
                   fa_fwd_strided, fa_fwd_tile, fa_fwd_varlen, fa_strerror, fa_version, load,
                   LIB_PATH)

__all__ = ["FA_BF16", "FA_F16", "FaError", "attention", "attention_fp8", "attention_kt",
           "attention_varlen", "fa_fwd", "fa_fwd_bf16", "fa_fwd_f16", "fa_fwd_fp8", "fa_fwd_kt",
           "fa_fwd_strided", "fa_fwd_tile", "fa_fwd_varlen", "fa_strerror", "fa_version", "load",
           "LIB_PATH"]
