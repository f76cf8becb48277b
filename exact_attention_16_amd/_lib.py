"""ctypes binding of the C ABI declared in include/fa_fwd.h.

Argument marshalling only: every step of the attention forward runs in the
HIP kernels of libfa_fwd.so. The functions below carry the C names and take
raw device pointers (ints) and sizes; :func:`attention` is a convenience that
takes torch tensors (torch supplies device memory and the stream, nothing
else).

There is no fallback: if the library is not built, or no GPU is present when
a kernel is launched, the call fails loudly.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa_fwd.so")

FA_F16 = 0
FA_BF16 = 1

# kernel choice of fa_fwd_diag
VARIANT_AUTO = 0
VARIANT_FOUR_WAVE = 1
VARIANT_PING_PONG = 2
VARIANT_TWO_BLOCK = 3

STATUS = {
    0: "FA_OK", -1: "FA_ERR_NULL", -2: "FA_ERR_DIM", -3: "FA_ERR_UNSUPPORTED",
    -4: "FA_ERR_ALIGN", -5: "FA_ERR_SCALE", -6: "FA_ERR_ALIAS", -7: "FA_ERR_HIP",
    -8: "FA_ERR_ARG",
}

# exported symbol -> (restype, argtypes)
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_FWD_ARGS = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]
SIGNATURES = {
    "fa_fwd": (_I, _FWD_ARGS + [_I]),
    "fa_fwd_f16": (_I, _FWD_ARGS),
    "fa_fwd_bf16": (_I, _FWD_ARGS),
    "fa_fwd_diag": (_I, _FWD_ARGS + [_I, _I, _I, _P]),
    "fa_fwd_tile": (_I, [_I, _I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I),
                         ctypes.POINTER(_I), ctypes.POINTER(ctypes.c_longlong)]),
    "fa_strerror": (ctypes.c_char_p, [_I]),
    "fa_version": (_I, []),
}

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = load().fa_strerror(status).decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg})")


def load() -> ctypes.CDLL:
    """Load libfa_fwd.so (built by exact_attention_16_amd.build); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m exact_attention_16_amd.build` "
                "(or __graft_entry__.build()). There is no non-HIP fallback.")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int, where: str) -> int:
    if status != 0:
        raise FaError(status, where)
    return status


def fa_fwd(q, k, v, o, lse, B, H, S, D, causal, scale, stream, dtype, check=True):
    st = load().fa_fwd(q, k, v, o, lse, B, H, S, D, int(causal), scale, stream, dtype)
    return _check(st, "fa_fwd") if check else st


def fa_fwd_f16(q, k, v, o, lse, B, H, S, D, causal, scale, stream, check=True):
    st = load().fa_fwd_f16(q, k, v, o, lse, B, H, S, D, int(causal), scale, stream)
    return _check(st, "fa_fwd_f16") if check else st


def fa_fwd_bf16(q, k, v, o, lse, B, H, S, D, causal, scale, stream, check=True):
    st = load().fa_fwd_bf16(q, k, v, o, lse, B, H, S, D, int(causal), scale, stream)
    return _check(st, "fa_fwd_bf16") if check else st


def fa_fwd_diag(q, k, v, o, lse, B, H, S, D, causal, scale, stream, dtype,
                threshold_log2, variant, rescale_events, check=True):
    st = load().fa_fwd_diag(q, k, v, o, lse, B, H, S, D, int(causal), scale, stream,
                            dtype, threshold_log2, variant, rescale_events)
    return _check(st, "fa_fwd_diag") if check else st


def fa_fwd_tile(D, B=0, H=0, S=0):
    """(block_m, block_n, threads, work_groups) for head dim D."""
    bm, bn, th = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    wg = ctypes.c_longlong()
    _check(load().fa_fwd_tile(D, B, H, S, ctypes.byref(bm), ctypes.byref(bn),
                              ctypes.byref(th), ctypes.byref(wg)), "fa_fwd_tile")
    return bm.value, bn.value, th.value, wg.value


def fa_strerror(status: int) -> str:
    return load().fa_strerror(status).decode()


def fa_version() -> int:
    return load().fa_version()


# ------------------------------------------------------------ torch helpers

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return FA_F16
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def attention(q, k, v, causal: bool, scale: float | None = None, out=None, lse=None,
              stream=None):
    """Attention forward on torch device tensors of shape [B, H, S, D].

    Returns (o, lse). `out`/`lse` may be given to avoid allocation. The kernel
    is enqueued on `stream` (default: torch's current stream) and the call
    returns without synchronising.
    """
    import torch
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if q.shape != k.shape or q.shape != v.shape or q.dim() != 4:
        raise ValueError("q, k, v must share one [B, H, S, D] shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, S, D = q.shape
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
           B, H, S, D, causal, float(scale), stream.cuda_stream, _dtype_code(q))
    return out, lse
