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

STATUS = {
    0: "FA_OK", -1: "FA_ERR_NULL", -2: "FA_ERR_DIM", -3: "FA_ERR_UNSUPPORTED",
    -4: "FA_ERR_ALIGN", -5: "FA_ERR_SCALE", -6: "FA_ERR_ALIAS", -7: "FA_ERR_HIP",
    -8: "FA_ERR_ARG", -9: "FA_ERR_LAYOUT",
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
    "fa_fwd_strided": (_I, [_P] * 5 + [_I] * 6 + [_F, _P, _I, _P]),
    "fa_fwd_varlen": (_I, [_P] * 7 + [_I] * 8 + [_F, _P, _I, _P]),
    "fa_fwd_kt": (_I, _FWD_ARGS + [_I]),
    "fa_fwd_fp8": (_I, [_P] * 5 + [_I] * 5 + [_F] * 4 + [_P]),
    "fa_fwd_tile": (_I, [_I, _I, _I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I),
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


def _strides(values, n):
    if len(values) != n:
        raise ValueError(f"expected {n} strides, got {len(values)}")
    return (ctypes.c_longlong * n)(*[int(x) for x in values])


def fa_fwd_strided(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale, stream, dtype, strides,
                   check=True):
    """strides: 14 element strides, q/k/v/o (batch, head, row) then lse (batch, head)."""
    st = load().fa_fwd_strided(q, k, v, o, lse, B, H, Sq, Sk, D, int(causal), scale, stream,
                               dtype, _strides(strides, 14))
    return _check(st, "fa_fwd_strided") if check else st


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, H, max_seqlen_q,
                  max_seqlen_k, total_q, total_k, D, causal, scale, stream, dtype, strides,
                  check=True):
    """strides: 9 element strides, q/k/v/o (head, row) then lse (head)."""
    st = load().fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, H, max_seqlen_q,
                              max_seqlen_k, total_q, total_k, D, int(causal), scale, stream,
                              dtype, _strides(strides, 9))
    return _check(st, "fa_fwd_varlen") if check else st


def fa_fwd_kt(q, kt, v, o, lse, B, H, S, D, causal, scale, stream, dtype, check=True):
    st = load().fa_fwd_kt(q, kt, v, o, lse, B, H, S, D, int(causal), scale, stream, dtype)
    return _check(st, "fa_fwd_kt") if check else st


def fa_fwd_fp8(q, k, v, o, lse, B, H, S, D, causal, scale, descale_q, descale_k, descale_v,
               stream, check=True):
    st = load().fa_fwd_fp8(q, k, v, o, lse, B, H, S, D, int(causal), scale, descale_q,
                           descale_k, descale_v, stream)
    return _check(st, "fa_fwd_fp8") if check else st


def fa_fwd_tile(D, B=0, H=0, S=0, causal=False):
    """(block_m, block_n, threads, work_groups) for head dim D."""
    bm, bn, th = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    wg = ctypes.c_longlong()
    _check(load().fa_fwd_tile(D, B, H, S, int(causal), ctypes.byref(bm), ctypes.byref(bn),
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


def _check_outputs(q, out, lse, o_shape, lse_shape, o_dtype):
    """out and lse as the kernel writes them: out of o_dtype and o_shape, lse
    float32 of lse_shape, both on q's device. Checked before any launch: the
    kernel derives the byte sizes it writes from the element types, which the
    C-side span checks cannot see."""
    import torch
    if out is not None:
        if out.dtype != o_dtype:
            raise ValueError(f"out must be {o_dtype}, not {out.dtype}")
        if tuple(out.shape) != tuple(o_shape):
            raise ValueError(f"out must have shape {tuple(o_shape)}, not {tuple(out.shape)}")
        if out.device != q.device:
            raise ValueError(f"out must be on {q.device}, not {out.device}")
        if out.dim() and out.stride(-1) != 1:
            raise ValueError("out's last dimension (D) must be contiguous")
    if lse is not None:
        if lse.dtype != torch.float32:
            raise ValueError(f"lse must be float32, not {lse.dtype}")
        if tuple(lse.shape) != tuple(lse_shape):
            raise ValueError(f"lse must have shape {tuple(lse_shape)}, not {tuple(lse.shape)}")
        if lse.device != q.device:
            raise ValueError(f"lse must be on {q.device}, not {lse.device}")


def _check_devices(q, *others):
    if not q.is_cuda:
        raise ValueError("q, k, v must be device tensors")
    for t in others:
        if t.device != q.device:
            raise ValueError(f"every tensor must be on {q.device}, not {t.device}")


def _check_structure(q, k, v, dims):
    if not (q.dim() == k.dim() == v.dim() == dims):
        raise ValueError(f"q, k, v must have {dims} dimensions")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    for t in (q, k, v):
        if t.stride(-1) != 1:
            raise ValueError("the last dimension (D) must be contiguous")


def attention(q, k, v, causal: bool, scale: float | None = None, out=None, lse=None,
              stream=None, layout: str = "bhsd"):
    """Attention forward on torch device tensors.

    layout "bhsd": q [B, H, Sq, D], k and v [B, H, Sk, D]; "bshd": q
    [B, Sq, H, D], k and v [B, Sk, H, D]. Any strides with a contiguous last
    dimension (views, slices, transposes); a causal mask with Sq != Sk is
    aligned bottom-right. Returns (o, lse): o in q's shape and layout (a new
    contiguous tensor unless `out` is given), lse [B, H, Sq] float32. The
    kernel is enqueued on `stream` (default: torch's current stream) and the
    call returns without synchronising.
    """
    import torch
    _check_structure(q, k, v, 4)
    if layout == "bhsd":
        B, H, Sq, D = q.shape
        Sk = k.shape[2]
        if k.shape[0] != B or k.shape[1] != H or k.shape[3] != D:
            raise ValueError("k, v must be [B, H, Sk, D] with q's B, H, D")
        perm = (0, 1, 2)
    elif layout == "bshd":
        B, Sq, H, D = q.shape
        Sk = k.shape[1]
        if k.shape[0] != B or k.shape[2] != H or k.shape[3] != D:
            raise ValueError("k, v must be [B, Sk, H, D] with q's B, H, D")
        perm = (0, 2, 1)
    else:
        raise ValueError(f"unknown layout {layout!r}")
    _check_outputs(q, out, lse, q.shape, (B, H, Sq), q.dtype)
    _check_devices(q, k, v)
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    dense = (layout == "bhsd" and Sq == Sk and q.is_contiguous() and k.is_contiguous()
             and v.is_contiguous() and out.is_contiguous() and lse.is_contiguous()
             and out.shape == q.shape and lse.shape == (B, H, Sq))
    if dense:
        fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
               B, H, Sq, D, causal, float(scale), stream.cuda_stream, _dtype_code(q))
        return out, lse
    strides = []
    for t in (q, k, v, out):
        strides += [t.stride(i) for i in perm]
    if lse.dim() != 3 or lse.stride(2) != 1:
        raise ValueError("lse must be [B, H, Sq] with contiguous rows")
    strides += [lse.stride(0), lse.stride(1)]
    fa_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                   B, H, Sq, Sk, D, causal, float(scale), stream.cuda_stream, _dtype_code(q),
                   strides)
    return out, lse


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                     max_seqlen_k: int, causal: bool, scale: float | None = None, out=None,
                     lse=None, stream=None):
    """Attention forward over sequences of different lengths packed along a token axis.

    q [total_q, H, D], k and v [total_k, H, D] (any strides with a
    contiguous last dimension); cu_seqlens_q / cu_seqlens_k: int32 device
    tensors of B+1 non-decreasing token offsets (sequence b owns query tokens
    cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1, key tokens likewise). Returns
    (o, lse): o [total_q, H, D], lse [H, total_q] float32. Causal masks are
    aligned bottom-right within each sequence.
    """
    import torch
    _check_structure(q, k, v, 3)
    total_q, H, D = q.shape
    total_k = k.shape[0]
    if k.shape[1] != H or k.shape[2] != D:
        raise ValueError("k, v must be [total_k, H, D] with q's H and D")
    for cu in (cu_seqlens_q, cu_seqlens_k):
        if cu.dtype != torch.int32 or cu.dim() != 1 or not cu.is_contiguous():
            raise ValueError("cu_seqlens must be contiguous int32 device tensors")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B+1 offsets")
    B = cu_seqlens_q.numel() - 1
    _check_outputs(q, out, lse, (total_q, H, D), (H, total_q), q.dtype)
    _check_devices(q, k, v, cu_seqlens_q, cu_seqlens_k)
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty((total_q, H, D), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    if lse.dim() != 2 or lse.stride(1) != 1:
        raise ValueError("lse must be [H, total_q] with contiguous rows")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    strides = []
    for t in (q, k, v, out):
        strides += [t.stride(1), t.stride(0)]
    strides += [lse.stride(0)]
    fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                  cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, H, int(max_seqlen_q),
                  int(max_seqlen_k), total_q, total_k, D, causal, float(scale),
                  stream.cuda_stream, _dtype_code(q), strides)
    return out, lse


def attention_fp8(q, k, v, descale_q: float, descale_k: float, descale_v: float, causal: bool,
                  scale: float | None = None, out=None, lse=None, stream=None):
    """Attention forward on 8-bit float inputs with per-tensor descales.

    q, k, v: contiguous [B, H, S, D] device tensors of E4M3 codes
    (torch.float8_e4m3fn, or uint8 holding the codes), D = 64 or 128; the value of
    a code is its E4M3 value times the tensor's descale. Returns (o, lse):
    o [B, H, S, D] bfloat16, lse [B, H, S] float32, enqueued on `stream`
    (default: torch's current stream) without synchronising.
    """
    import torch
    _check_structure(q, k, v, 4)
    if q.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError(f"8-bit inputs must be float8_e4m3fn or uint8 codes, not {q.dtype}")
    if q.shape != k.shape:
        raise ValueError("q, k, v must have one shape [B, H, S, D]")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("8-bit inputs must be contiguous [B, H, S, D]")
    B, H, S, D = q.shape
    _check_outputs(q, out, lse, (B, H, S, D), (B, H, S), torch.bfloat16)
    _check_devices(q, k, v)
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty((B, H, S, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if (out.dtype != torch.bfloat16 or out.shape != q.shape or not out.is_contiguous()
            or lse.dtype != torch.float32 or lse.shape != (B, H, S) or not lse.is_contiguous()):
        raise ValueError("out must be contiguous bf16 [B, H, S, D], lse contiguous fp32 [B, H, S]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
               B, H, S, D, causal, float(scale), float(descale_q), float(descale_k),
               float(descale_v), stream.cuda_stream)
    return out, lse


def attention_kt(q, kt, v, causal: bool, scale: float | None = None, out=None, lse=None,
                 stream=None):
    """Attention forward with K given transposed.

    q, v: contiguous [B, H, S, D] 16-bit device tensors; kt: contiguous
    [B, H, D, S] (S a multiple of 8). Returns (o, lse) as :func:`attention`.
    """
    import torch
    if not (q.dtype == kt.dtype == v.dtype):
        raise ValueError("q, kt, v must share one dtype")
    B, H, S, D = q.shape
    if tuple(kt.shape) != (B, H, D, S) or v.shape != q.shape:
        raise ValueError("kt must be [B, H, D, S] and v [B, H, S, D] for q [B, H, S, D]")
    if not (q.is_contiguous() and kt.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, kt, v must be contiguous")
    _check_outputs(q, out, lse, q.shape, (B, H, S), q.dtype)
    _check_devices(q, kt, v)
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if not (out.is_contiguous() and out.shape == q.shape and lse.is_contiguous()
            and lse.shape == (B, H, S)):
        raise ValueError("out must be contiguous [B, H, S, D], lse contiguous [B, H, S]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    fa_fwd_kt(q.data_ptr(), kt.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
              B, H, S, D, causal, float(scale), stream.cuda_stream, _dtype_code(q))
    return out, lse
