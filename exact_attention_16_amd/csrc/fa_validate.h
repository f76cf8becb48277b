// Host-side argument checks of every entry point, and the Problem each one
// fills. Plain C++: no HIP call, no device access, no allocation, so the
// checks run (and are tested, also under AddressSanitizer and
// UndefinedBehaviorSanitizer) on a machine without a GPU.
//
// Every size product is computed with overflow checks: strides and counts
// come from the caller, and a product that wrapped could make a huge tensor
// look small and pass the range checks.
#pragma once
#include <math.h>
#include <stdint.h>

#include "../../include/fa_fwd.h"
#include "fa_layout.h"
#include "fa_layout8.h"
#include "fa_problem.h"

namespace fa {

// Largest element stride accepted; anything larger is FA_ERR_DIM before any
// arithmetic on it.
constexpr long long kMaxStride = 1LL << 40;
// Largest element count of one tensor.
constexpr long long kMaxElems = 1LL << 40;
// One (sequence, head) of a tensor is addressed with 32-bit byte offsets.
constexpr long long kMaxHeadBytes = 1LL << 31;

// a * b, false on overflow (inputs >= 0)
static inline bool mul_ok(long long a, long long b, long long* r) {
  return !__builtin_mul_overflow(a, b, r);
}
// a * b * c < lim, all >= 0, without overflow
static inline bool product_below(long long a, long long b, long long c, long long lim) {
  long long ab, abc;
  return mul_ok(a, b, &ab) && mul_ok(ab, c, &abc) && abc < lim;
}

// Byte span [lo, hi) of a strided tensor: dims n[i] >= 1 with strides st[i]
// (elements, 0 <= st[i] <= kMaxStride), the innermost extent `inner`
// elements, element size es. False when the span does not fit the address
// space.
struct Span {
  uintptr_t lo, hi;
};
static inline bool span_of(const void* base, const long long* n, const long long* st, int nd,
                           long long inner, int es, Span* out) {
  long long last = inner;  // one past the last element, relative to base
  for (int i = 0; i < nd; ++i) {
    long long t;
    if (n[i] < 1 || !mul_ok(n[i] - 1, st[i], &t) || __builtin_add_overflow(last, t, &last))
      return false;
  }
  long long bytes;
  uintptr_t hi;
  if (!mul_ok(last, es, &bytes) || __builtin_add_overflow((uintptr_t)base, (uintptr_t)bytes, &hi))
    return false;
  *out = Span{(uintptr_t)base, hi};
  return true;
}
static inline bool spans_overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// True when no two index tuples of dims n (strides st, all >= 0) with an
// innermost block of `inner` contiguous elements share an element: sorted by
// stride, each stride must clear the whole extent of the smaller ones.
static inline bool no_self_overlap(const long long* n, const long long* st, int nd,
                                   long long inner) {
  long long dn[4], ds[4];
  int m = 0;
  for (int i = 0; i < nd && i < 4; ++i)
    if (n[i] > 1) {
      dn[m] = n[i];
      ds[m] = st[i];
      ++m;
    }
  for (int i = 1; i < m; ++i)  // insertion sort by stride
    for (int j = i; j > 0 && ds[j] < ds[j - 1]; --j) {
      const long long t = ds[j]; ds[j] = ds[j - 1]; ds[j - 1] = t;
      const long long u = dn[j]; dn[j] = dn[j - 1]; dn[j - 1] = u;
    }
  long long extent = inner;
  for (int i = 0; i < m; ++i) {
    long long t;
    if (ds[i] < extent) return false;
    if (!mul_ok(ds[i], dn[i] - 1, &t) || __builtin_add_overflow(t, extent, &extent)) return false;
  }
  return true;
}

// Scalar checks shared by every 16-bit entry point.
static inline int validate_args(int B, int H, int Sq, int Sk, int D, int causal, float scale,
                                int dtype) {
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (B < 0 || H < 0 || Sq < 0 || Sk < 0) return FA_ERR_DIM;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  // the grid of the kernel with the smallest query tile stays below 2^31
  if (!product_below(B, H, num_q_tiles(Sq, Cfg4<64>::BM), 1LL << 31)) return FA_ERR_DIM;
  return FA_OK;
}

// Checks on a filled 16-bit Problem (at least one query row). nq / nk: the
// outer dims (counts) of the query-side and key-side tensors, with the
// matching strides of q, k, v and o; nl / sl those of lse.
static inline int validate_problem(const Problem& P, int D, const long long* nq,
                                   const long long* sq_, const long long* sk_,
                                   const long long* sv_, const long long* so_,
                                   const long long* nk, int nd, const long long* nl,
                                   const long long* sl, int ndl) {
  if (!P.q || !P.k || !P.v || !P.o || !P.lse) return FA_ERR_NULL;
  const uintptr_t al = (uintptr_t)P.q | (uintptr_t)P.k | (uintptr_t)P.v | (uintptr_t)P.o |
                       (uintptr_t)P.lse;
  if (al & 15) return FA_ERR_ALIGN;
  const long long all[] = {P.qb, P.qh, P.qs, P.kb, P.kh, P.ks, P.vb,
                           P.vh, P.vs, P.ob, P.oh, P.os, P.lb, P.lh};
  for (long long x : all)
    if (x < 0) return FA_ERR_LAYOUT;
  for (long long x : all)
    if (x > kMaxStride) return FA_ERR_DIM;
  for (int i = 0; i < 12; ++i)
    if (all[i] % 8) return FA_ERR_ALIGN;  // every row starts 16-byte aligned
  if (P.qs < D || P.ks < D || P.vs < D || P.os < D) return FA_ERR_LAYOUT;
  // offsets within one (sequence, head) are 32-bit bytes
  if (!product_below(P.Sq, P.qs, 2, kMaxHeadBytes) || !product_below(P.Sk, P.ks, 2, kMaxHeadBytes) ||
      !product_below(P.Sk, P.vs, 2, kMaxHeadBytes) || !product_below(P.Sq, P.os, 2, kMaxHeadBytes) ||
      !product_below(P.Sq, 4, 1, kMaxHeadBytes))
    return FA_ERR_DIM;
  if (!no_self_overlap(nq, so_, nd, D) || !no_self_overlap(nl, sl, ndl, 1)) return FA_ERR_LAYOUT;
  Span q, k, v, o, l;
  if (!span_of(P.q, nq, sq_, nd, D, 2, &q) || !span_of(P.k, nk, sk_, nd, D, 2, &k) ||
      !span_of(P.v, nk, sv_, nd, D, 2, &v) || !span_of(P.o, nq, so_, nd, D, 2, &o) ||
      !span_of(P.lse, nl, sl, ndl, 1, 4, &l))
    return FA_ERR_DIM;
  if (spans_overlap(o, q) || spans_overlap(o, k) || spans_overlap(o, v) || spans_overlap(l, q) ||
      spans_overlap(l, k) || spans_overlap(l, v) || spans_overlap(l, o))
    return FA_ERR_ALIAS;
  if ((o.hi - o.lo) / 2 > (uint64_t)kMaxElems || (q.hi - q.lo) / 2 > (uint64_t)kMaxElems)
    return FA_ERR_DIM;
  return FA_OK;
}

// Fixed-length problem from strides (14: q, k, v, o as batch, head, row; lse
// as batch, head). *empty is set when there is no query row to compute.
static inline int make_fixed(Problem* P, const void* q, const void* k, const void* v, void* o,
                             float* lse, int B, int H, int Sq, int Sk, int D, int causal,
                             float scale, int dtype, const long long* st, bool* empty) {
  *empty = false;
  int r = validate_args(B, H, Sq, Sk, D, causal, scale, dtype);
  if (r != FA_OK) return r;
  if ((long long)B * H * Sq == 0) {
    *empty = true;
    return FA_OK;
  }
  if (!st) return FA_ERR_NULL;
  *P = Problem{q, k, v, o, lse, st[0], st[1], st[2], st[3], st[4], st[5], st[6],
               st[7], st[8], st[9], st[10], st[11], st[12], st[13], nullptr, nullptr,
               0, 0, B, H, Sq, Sk, 0, scale * kLog2e, nullptr, 0.f, kHeadGroup};
  const long long nq[] = {B, H, Sq}, nk[] = {B, H, Sk > 0 ? Sk : 1};
  const long long sq_[] = {st[0], st[1], st[2]}, sk_[] = {st[3], st[4], st[5]},
                  sv_[] = {st[6], st[7], st[8]}, so_[] = {st[9], st[10], st[11]};
  const long long nl[] = {B, H, Sq}, sl[] = {st[12], st[13], 1};
  return validate_problem(*P, D, nq, sq_, sk_, sv_, so_, nk, 3, nl, sl, 3);
}

static inline void dense_strides(long long* st, int H, int S, int D) {
  const long long hs = (long long)S * D;
  const long long v[] = {H * hs, hs, D, H * hs, hs, D, H * hs, hs, D, H * hs, hs, D,
                         (long long)H * S, S};
  for (int i = 0; i < 14; ++i) st[i] = v[i];
}

// Dense problem: q, k, v, o [B,H,S,D], lse [B,H,S].
static inline int make_dense(Problem* P, const void* q, const void* k, const void* v, void* o,
                             float* lse, int B, int H, int S, int D, int causal, float scale,
                             int dtype, bool* empty) {
  *empty = false;
  const int r = validate_args(B, H, S, S, D, causal, scale, dtype);
  if (r != FA_OK) return r;
  if ((long long)B * H * S == 0) {
    *empty = true;
    return FA_OK;
  }
  // the dense strides themselves must not overflow (H*S*D <= 2^40)
  if (!product_below(H, S, D, kMaxStride + 1)) return FA_ERR_DIM;
  long long st[14];
  dense_strides(st, H, S, D);
  return make_fixed(P, q, k, v, o, lse, B, H, S, S, D, causal, scale, dtype, st, empty);
}

// Byte spans of contiguous q, k, v, o (n elements each, es / oes bytes per
// element) and lse (nl floats); FA_ERR_ALIAS if o or lse overlaps another.
static inline int dense_alias_check(const void* q, const void* k, const void* v, const void* o,
                                    const float* lse, long long n, int es, int oes,
                                    long long nl) {
  const Span sq{(uintptr_t)q, (uintptr_t)q + (uintptr_t)(es * n)},
      sk{(uintptr_t)k, (uintptr_t)k + (uintptr_t)(es * n)},
      sv{(uintptr_t)v, (uintptr_t)v + (uintptr_t)(es * n)},
      so{(uintptr_t)o, (uintptr_t)o + (uintptr_t)(oes * n)},
      sl{(uintptr_t)lse, (uintptr_t)lse + (uintptr_t)(4 * nl)};
  if (spans_overlap(so, sq) || spans_overlap(so, sk) || spans_overlap(so, sv) ||
      spans_overlap(sl, sq) || spans_overlap(sl, sk) || spans_overlap(sl, sv) ||
      spans_overlap(sl, so))
    return FA_ERR_ALIAS;
  return FA_OK;
}

// Dense problem with K given transposed: q, v, o [B,H,S,D], k [B,H,D,S].
static inline int make_kt(Problem* P, const void* q, const void* k, const void* v, void* o,
                          float* lse, int B, int H, int S, int D, int causal, float scale,
                          int dtype, bool* empty) {
  *empty = false;
  int r = validate_args(B, H, S, S, D, causal, scale, dtype);
  if (r != FA_OK) return r;
  if ((long long)B * H * S == 0) {
    *empty = true;
    return FA_OK;
  }
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse) & 15)
    return FA_ERR_ALIGN;
  if (S % 8) return FA_ERR_ALIGN;  // every row of k (S keys of one d) starts 16-byte aligned
  if (!product_below(S, D, 2, kMaxHeadBytes)) return FA_ERR_DIM;
  long long bh, n;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, (long long)S * D, &n) || n > kMaxElems) return FA_ERR_DIM;
  r = dense_alias_check(q, k, v, o, lse, n, 2, 2, bh * S);
  if (r != FA_OK) return r;
  const long long hs = (long long)S * D;
  // k's third stride is the distance between its d rows (S elements)
  *P = Problem{q, k, v, o, lse, H * hs, hs, D, H * hs, hs, S, H * hs, hs, D, H * hs, hs, D,
               (long long)H * S, S, nullptr, nullptr, 0, 0, B, H, S, S, 0, scale * kLog2e,
               nullptr, 0.f, kHeadGroup};
  return FA_OK;
}

static inline bool positive_finite(float x) { return x > 0.f && isfinite(x); }

// Dense [B,H,S,D] problem on E4M3 inputs (one byte per element) with a bf16
// output (two bytes per element).
static inline int make_fp8(Problem* P, const void* q, const void* k, const void* v, void* o,
                           float* lse, int B, int H, int S, int D, int causal, float scale,
                           float dq, float dk, float dv, bool* empty) {
  *empty = false;
  if (B < 0 || H < 0 || S < 0) return FA_ERR_DIM;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  if (!positive_finite(scale) || !positive_finite(dq) || !positive_finite(dk) ||
      !positive_finite(dv))
    return FA_ERR_SCALE;
  // the folded base-2 logit multiplier must be a normal float
  const double c = (double)scale * dq * dk * (double)kLog2e;
  if (!(c >= 1.17549435e-38 && c <= 3.40282347e38)) return FA_ERR_SCALE;
  if (!product_below(B, H, num_q_tiles(S, CfgF8::BM), 1LL << 31)) return FA_ERR_DIM;
  if ((long long)B * H * S == 0) {
    *empty = true;
    return FA_OK;
  }
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse) & 15)
    return FA_ERR_ALIGN;
  // one head's O rows addressed with 32-bit byte offsets; at most 2^40 elements
  if (!product_below(S, D, 2, kMaxHeadBytes)) return FA_ERR_DIM;
  long long bh, n;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, (long long)S * D, &n) || n > kMaxElems) return FA_ERR_DIM;
  const int r = dense_alias_check(q, k, v, o, lse, n, 1, 2, bh * S);
  if (r != FA_OK) return r;
  const long long hs = (long long)S * D;
  *P = Problem{q, k, v, o, lse, H * hs, hs, D, H * hs, hs, D, H * hs, hs, D, H * hs, hs, D,
               (long long)H * S, S, nullptr, nullptr, 0, 0, B, H, S, S, 0, (float)c, nullptr, dv,
               kHeadGroup};
  return FA_OK;
}

// Sequences packed along a token axis (9 strides: q, k, v, o as head, row;
// lse as head). *empty is set when there is no query row to compute.
static inline int make_varlen(Problem* P, const void* q, const void* k, const void* v, void* o,
                              float* lse, const int* cuq, const int* cuk, int B, int H,
                              int max_q, int max_k, int total_q, int total_k, int D, int causal,
                              float scale, int dtype, const long long* st, bool* empty) {
  *empty = false;
  int r = validate_args(B, H, max_q, max_k, D, causal, scale, dtype);
  if (r != FA_OK) return r;
  if (total_q < 0 || total_k < 0) return FA_ERR_DIM;
  if ((long long)B * H * max_q == 0 || total_q == 0) {
    *empty = true;
    return FA_OK;
  }
  if (!cuq || !cuk || !st) return FA_ERR_NULL;
  if (((uintptr_t)cuq | (uintptr_t)cuk) & 3) return FA_ERR_ALIGN;
  *P = Problem{q, k, v, o, lse, 0, st[0], st[1], 0, st[2], st[3], 0, st[4], st[5], 0,
               st[6], st[7], 0, st[8], cuq, cuk, total_q, total_k,
               B, H, max_q, max_k, 0, scale * kLog2e, nullptr, 0.f,
               // one sequence's heads on an XCD at a time (sequences differ in length)
               H % 8 == 0 ? H / 8 : 1};
  const long long nq[] = {H, total_q}, nk[] = {H, total_k > 0 ? total_k : 1};
  const long long sq_[] = {st[0], st[1]}, sk_[] = {st[2], st[3]}, sv_[] = {st[4], st[5]},
                  so_[] = {st[6], st[7]};
  const long long nl[] = {H, total_q}, sl[] = {st[8], 1};
  return validate_problem(*P, D, nq, sq_, sk_, sv_, so_, nk, 2, nl, sl, 2);
}

}  // namespace fa
