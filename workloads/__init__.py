"""Seeded synthetic inputs for the fused attention forward.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It holds no attention arithmetic: it draws Gaussian Q/K/V from a
seeded generator, rounds them to the 16-bit storage type, and decodes 16-bit
storage back to float64 so that the oracle sees exactly the values the GPU
receives.

Workloads (all Q/K/V iid N(0,1), scale = 1/sqrt(D), layout [B, H, S, D]):

====  ================================  =====  ======  ==========================
name  shape (B, H, S, D)                dtype  causal  source of the shape
====  ================================  =====  ======  ==========================
tiny  1, 1, 128, 64                     fp16   both    small case for brute checks
dec   1, 16, 1024, 64                   fp16   yes     causal decoder layer
bat   10, 64, 1024, 64                  fp16   no      the Triton FA2 study's shape
                                                       (hotdry.top, "FlashAttention
                                                       的Triton性能考古学", grid section)
long  2, 16, 8192, 128                  bf16   yes     long-context causal
ramp  1, 8, 16384, 128                  bf16   yes     rescale stress (key ramp)
long8 2, 16, 8192, 128                  e4m3   yes     the long workload in 8-bit
                                                       floats, per-tensor scales
bat8  10, 64, 1024, 64                  e4m3   no      the bat workload in 8-bit
====  ================================  =====  ======  ==========================

Recipe: ``numpy.random.default_rng(seed)`` draws Q, then K, then V as float32
``standard_normal``; the ``ramp`` workload then draws a unit vector ``u``
(float64 normal, normalised), adds ``0.002*j*u`` to key row ``j`` and ``u`` to
every query row, summed in float32.  Rounding to fp16 is numpy's
round-to-nearest-even ``astype``; rounding to bf16 is the bit-exact
round-to-nearest-even of the float32 pattern.

8-bit inputs (``make_fp8_inputs``): the same float32 draws, then per tensor a
descale d = float32(max|x| / 448) and codes E4M3(x / d) (nearest, ties to
even), so that each tensor spans E4M3's range; the value of a code is
decode(code) * d.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

F16 = "f16"
BF16 = "bf16"
E4M3 = "e4m3"  # OCP 8-bit float E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits,
               # no infinities, S.1111.111 = NaN, largest finite 448

# numeric codes shared with the C ABI's dtype enum (FA_F16 = 0, FA_BF16 = 1)
DTYPE_CODE = {F16: 0, BF16: 1}
ELEM_BYTES = {F16: 2, BF16: 2, E4M3: 1}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    dtype: str
    causal: bool
    seed: int
    ramp: float = 0.0  # per-key additive ramp coefficient (0 = none)

    @property
    def scale(self) -> float:
        """float32(1/sqrt(D)), the value passed to the kernel."""
        return float(np.float32(1.0 / math.sqrt(self.D)))

    @property
    def flops(self) -> float:
        """Metric FLOPs: 4*B*H*S^2*D, halved when causal."""
        f = 4.0 * self.B * self.H * self.S * self.S * self.D
        return f / 2 if self.causal else f

    @property
    def algorithmic_bytes(self) -> int:
        """Q, K, V read once (their element size), O written once (16-bit), LSE (4 B/row)."""
        n = self.B * self.H * self.S * self.D
        return (3 * ELEM_BYTES[self.dtype] + 2) * n + 4 * self.B * self.H * self.S

    def with_causal(self, causal: bool) -> "Workload":
        return Workload(self.name, self.B, self.H, self.S, self.D, self.dtype,
                        causal, self.seed, self.ramp)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 128, 64, F16, False, 1),
    "tiny_causal": Workload("tiny_causal", 1, 1, 128, 64, F16, True, 1),
    "dec": Workload("dec", 1, 16, 1024, 64, F16, True, 2),
    "bat": Workload("bat", 10, 64, 1024, 64, F16, False, 3),
    "long": Workload("long", 2, 16, 8192, 128, BF16, True, 4),
    "ramp": Workload("ramp", 1, 8, 16384, 128, BF16, True, 5, ramp=0.002),
    "long8": Workload("long8", 2, 16, 8192, 128, E4M3, True, 4),
    "bat8": Workload("bat8", 10, 64, 1024, 64, E4M3, False, 3),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = (u + np.uint32(0x7FFF) + lsb) >> 16
    # NaN stays NaN (quiet); not produced by these generators
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, (u >> 16) | 0x40, r)
    return r.astype(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE binary16 (round to nearest even); uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _e4m3_table() -> np.ndarray:
    """Values of the finite non-negative E4M3FN codes 0x00 .. 0x7E, ascending."""
    c = np.arange(0x7F, dtype=np.int64)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m * 2.0 ** -9, (8 + m) * 2.0 ** (e - 10))


_E4M3 = _e4m3_table()


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round to E4M3FN (nearest, ties to even), saturating at +-448; uint8 bits."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(_E4M3, a), 1, len(_E4M3) - 1)  # first code >= a
    lo = hi - 1
    dlo, dhi = a - _E4M3[lo], _E4M3[hi] - a
    code = np.where((dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0)), hi, lo)
    code = np.where(a <= _E4M3[0], 0, code)
    out = code | np.where(np.signbit(x), 0x80, 0)
    return np.where(np.isnan(x), 0x7F, out).astype(np.uint8)


def round_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F16:
        return f32_to_f16_bits(x)
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    if dtype == E4M3:
        return f32_to_e4m3_bits(x)
    raise ValueError(dtype)


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of 16-bit (or, for E4M3, 8-bit) storage."""
    if dtype == E4M3:
        b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
        mag = np.where((b & 0x7F) == 0x7F, np.nan, _E4M3[np.minimum(b & 0x7F, 0x7E)])
        return np.where(b & 0x80, -mag, mag)
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float64)
    if dtype == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def make_inputs(w: Workload, ramp_override: float | None = None):
    """Seeded Q, K, V as uint16 bit arrays of shape (B, H, S, D)."""
    rng = np.random.default_rng(w.seed)
    shape = (w.B, w.H, w.S, w.D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    ramp = w.ramp if ramp_override is None else ramp_override
    if ramp:
        u = rng.standard_normal(w.D)
        u = u / np.linalg.norm(u)
        j = np.arange(w.S, dtype=np.float64)
        k += (ramp * j[:, None] * u[None, :]).astype(np.float32)
        q += u.astype(np.float32)
    return (round_bits(q, w.dtype), round_bits(k, w.dtype), round_bits(v, w.dtype))


def quantize_e4m3(x: np.ndarray):
    """Per-tensor scaled E4M3: (codes, descale) with descale = float32(max|x| / 448)."""
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    d = float(np.float32(amax / 448.0)) if amax > 0 else 1.0
    return f32_to_e4m3_bits(np.asarray(x, dtype=np.float64) / d), d


def make_fp8_inputs(w: Workload):
    """Seeded Q, K, V as E4M3 codes (uint8, (B, H, S, D)) and their descales (dq, dk, dv)."""
    rng = np.random.default_rng(w.seed)
    shape = (w.B, w.H, w.S, w.D)
    xs = [rng.standard_normal(shape, dtype=np.float32) for _ in range(3)]
    out = [quantize_e4m3(x) for x in xs]
    return tuple(c for c, _ in out), tuple(d for _, d in out)


def random_bits(shape, dtype: str, seed: int, mean: float = 0.0, std: float = 1.0):
    """Gaussian values rounded to 16-bit storage (for edge-case tests)."""
    rng = np.random.default_rng(seed)
    x = (mean + std * rng.standard_normal(shape)).astype(np.float32)
    return round_bits(x, dtype)



# Variable-length batch: sequences of different lengths packed along a token
# axis ([total, H, D]), the situation of the dynamic-shape section (6.3) of
# the xdnf.cn page (lengths that vary per request). Lengths are drawn
# uniformly from [lo, hi] with their own seed; Q, K, V are N(0,1) like the
# fixed-length workloads.
@dataclass(frozen=True)
class VarlenWorkload:
    name: str
    B: int
    H: int
    D: int
    lo: int
    hi: int
    dtype: str
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.D)))

    def lengths(self) -> np.ndarray:
        rng = np.random.default_rng(self.seed)
        return rng.integers(self.lo, self.hi + 1, size=self.B).astype(np.int64)

    def flops(self) -> float:
        """Metric convention per sequence: 4*H*L^2*D, halved when causal."""
        L = self.lengths().astype(np.float64)
        f = 4.0 * self.H * float((L * L).sum()) * self.D
        return f / 2 if self.causal else f


VARLEN = VarlenWorkload("varlen", B=16, H=16, D=128, lo=256, hi=8192, dtype=BF16, causal=True,
                        seed=8)


def make_varlen_inputs(w: VarlenWorkload):
    """Token offsets (B+1, int32) and Q, K, V bits of shape (total, H, D)."""
    L = w.lengths()
    cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    rng = np.random.default_rng(w.seed + 1)
    shape = (int(cu[-1]), w.H, w.D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    return cu, round_bits(q, w.dtype), round_bits(k, w.dtype), round_bits(v, w.dtype)
