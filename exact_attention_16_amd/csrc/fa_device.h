// Device building blocks shared by the gfx950 attention-forward kernels:
// vector types, lane exchanges, buffer descriptors, LDS pointer types,
// barriers and waits, scheduling patterns, the rows of a Problem (fa_problem.h)
// and the per-row softmax state every wave type shares.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_layout.h"
#include "fa_problem.h"

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Word 3 of a raw (untyped, stride 0) gfx9 buffer descriptor.
constexpr int kBufferWord3 = 0x00020000;

template <int N> struct IC { static constexpr int value = N; };
template <int P, class X> __device__ __forceinline__ X& pick(X& one, X& zero) {
  if constexpr (P != 0) return one; else return zero;
}

typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// Value combined with the same register of lane l^32 (the other k-half of
// the same query row): v_permlane32_swap exchanges the upper half-wave of
// one copy with the lower half-wave of the other, so the two results hold
// both values in every lane and a symmetric op combines them.
// The maxima use the NaN-propagating maximum (v_maximum3_f32 on gfx950):
// fmaxf's NaN-ignoring form costs an extra quieting op per operand that
// does not come from plain arithmetic (MFMA results, lane exchanges). A NaN
// score makes its row NaN through the exponential either way.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max_xor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return vmax(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Raw buffer descriptor over `bytes` bytes at `base`. A macro rather than a
// function: a function or lambda returning the descriptor type makes the
// host compilation pass drop the kernel launch stubs.
// Base and size are wave-uniform; they pass through readfirstlane so that
// the descriptor is built in scalar registers even where the compiler has
// kept them in vector registers (it would otherwise loop over the lanes'
// values around every use). On values already scalar this costs nothing.
#define FA_RSRC(base, bytes)                                                      \
  __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>((const void*)fa::uniform_ptr(base)), 0, \
                                    (int)__builtin_amdgcn_readfirstlane((uint32_t)(bytes)), \
                                    kBufferWord3)
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

// Byte count of a DMA source range: `bytes` when `live`, else 0 (an empty
// range, which the DMA turns into zeros). A product rather than a select:
// the compiler turns the select of a uniform condition into branches that
// split the DMA issue into blocks of its own. The 8-bit kernel runs about 1%
// faster this way; the 16-bit kernels' time is unchanged.
// The count is wave-uniform (it comes from sizes and the tile index); the
// readfirstlane says so to the compiler, which otherwise may derive it from a
// lane-varying expression that shares terms with it (the mask's bound) and
// then wraps every DMA issue in a loop over the lanes' values.
__device__ __forceinline__ uint32_t dma_bytes(bool live, uint32_t bytes) {
  return __builtin_amdgcn_readfirstlane(bytes * (uint32_t)live);
}

// LDS pointers stay in address space 3 from the point where each shared
// array is declared (a cast of a generic pointer to address space 3 would
// make the host compilation pass drop the kernel launch stubs).
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ u32x4 lds16(const lds_char* p) { return *(lds_u32x4*)p; }

// Hardware work-group barrier fenced against compiler reordering. Unlike
// __syncthreads() it implies no wait for outstanding memory operations: the
// caller waits for exactly what it needs first.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
// s_waitcnt vmcnt(N) lgkmcnt(0) (no export wait), 0 <= N <= 15.
template <int N> __device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N <= 15, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0070 | N);
}

// Scheduling pattern for one MFMA loop: DS0 LDS reads up front, then N
// times {one MFMA, DS LDS reads}, so that each MFMA's operands are read
// several MFMAs ahead of it. (Left to itself the scheduler reads them just
// before their MFMA, which then waits for the LDS round trip.)
template <int DS0, int N, int DS>
__device__ __forceinline__ void read_ahead() {
  __builtin_amdgcn_sched_group_barrier(0x100, DS0, 0);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, DS, 0);
  }
}

// Scheduling pattern for one region of independent MFMA and vector work:
// DS0 LDS reads up front, then N times {one MFMA, DS LDS reads, V VALU}.
template <int DS0, int N, int DS, int V>
__device__ __forceinline__ void mix() {
  __builtin_amdgcn_sched_group_barrier(0x100, DS0, 0);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, DS, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
  }
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Lengths and row-0 element offsets of sequence bb, head h of a Problem:
// query rows Lq and key rows Lk (with per-sequence offsets: clamped to the
// tensors' token rows and to Sq / Sk), and where row 0 of q, k, v, o and lse
// starts.
struct HeadRows {
  int Lq, Lk;
  long long q0, k0, v0, o0, l0;
  int cut_q;   // variable lengths: query rows past the stated maximum
  bool cut_k;  // variable lengths: more keys than the stated maximum
};
// The offsets are read through the constant address space: they do not
// change during a launch, so the reads are scalar loads of wave-uniform
// values, also in code after the kernel's first stores (the persistent
// form's later items), where a plain global read becomes a vector load whose
// result the compiler treats as lane-varying.
typedef __attribute__((address_space(4))) const int const_int;
__device__ __forceinline__ HeadRows head_rows(const Problem& P, int bb, int h) {
  HeadRows r;
  if (P.cuq) {
    const_int* cq = (const_int*)P.cuq;
    const_int* ck = (const_int*)P.cuk;
    const int sq = clampi(cq[bb], 0, P.totq), eq = clampi(cq[bb + 1], sq, P.totq);
    const int sk = clampi(ck[bb], 0, P.totk), ek = clampi(ck[bb + 1], sk, P.totk);
    r.Lq = min(eq - sq, P.Sq);
    r.Lk = min(ek - sk, P.Sk);
    r.cut_q = (eq - sq) - r.Lq;
    r.cut_k = ek - sk > P.Sk;
    r.q0 = sq * P.qs + h * P.qh;
    r.k0 = sk * P.ks + h * P.kh;
    r.v0 = sk * P.vs + h * P.vh;
    r.o0 = sq * P.os + h * P.oh;
    r.l0 = h * P.lh + sq;
  } else {
    r.Lq = P.Sq;
    r.Lk = P.Sk;
    r.cut_q = 0;
    r.cut_k = false;
    r.q0 = bb * P.qb + h * P.qh;
    r.k0 = bb * P.kb + h * P.kh;
    r.v0 = bb * P.vb + h * P.vh;
    r.o0 = bb * P.ob + h * P.oh;
    r.l0 = bb * P.lb + h * P.lh;
  }
  return r;
}

// Compacted variable-length launch (varlen_tile in fa_layout.h): the
// sequence g holding rank k, the rank r within it and its tile count nt.
// Every wave scans the offsets itself, lane l taking sequences 4l .. 4l+3
// (at most kCompactMaxSeqs): per-lane item counts, an inclusive sum over the
// lanes, and the first lane whose sum exceeds k. *dec: some offset is below
// the one before it (the same for every work-group). False when k is at or
// past the last item (a work-group of the bound's slack).
template <int BM>
__device__ __forceinline__ bool varlen_find(const Problem& P, int m, int k, int* g, int* r,
                                            int* nt, bool* dec) {
  const int lane = threadIdx.x & 63;
  int s[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int idx = 4 * lane + i;
    s[i] = idx <= P.B ? P.cuq[idx] : 0;
  }
  int n[4], tot = 0;
  bool d = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    n[i] = 0;
    if (4 * lane + i < P.B) {
      d |= s[i + 1] < s[i];
      const int sq = clampi(s[i], 0, P.totq), eq = clampi(s[i + 1], sq, P.totq);
      n[i] = num_q_tiles(min(eq - sq, P.Sq), BM);
    }
    tot += m * n[i];
  }
  *dec = __builtin_amdgcn_ballot_w64(d) != 0;
  int incl = tot;
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) {
    const int t = __shfl_up(incl, (unsigned)sh, 64);
    if (lane >= sh) incl += t;
  }
  const uint64_t hit = __builtin_amdgcn_ballot_w64(k < incl);
  if (hit == 0) return false;
  const int L = (int)__builtin_ctzll(hit);
  int rr = k - (incl - tot), gg = 0, nn = 0;
  bool found = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!found) {
      if (rr < m * n[i]) {
        gg = 4 * lane + i;
        nn = n[i];
        found = true;
      } else {
        rr -= m * n[i];
      }
    }
  }
  *g = __builtin_amdgcn_readlane(gg, L);
  *r = __builtin_amdgcn_readlane(rr, L);
  *nt = __builtin_amdgcn_readlane(nn, L);
  return true;
}

// What every wave type knows about its rows (configuration C, causal mask,
// base lag THR in log2 units): which 32 query rows it owns, its sequence's
// lengths, the running base b of the online softmax and its share of the
// row sum, and the decisions that follow from them (tile counts, whether a
// tile needs index compares, the base update).
template <class C, bool CAUSAL, int THR> struct RowState {
  int lane, wave, hh, q0w, qrow, qt;
  int Lq, Lk, off;  // this sequence's query and key rows; off = Lk - Lq (causal alignment)
  float c;          // base-2 multiplier of the raw dot products
  float b, lsum;    // running base (log2 units, lags the true max by <= THR);
                    // this lane's partial row sum (its k-half of the keys)

  // Finds this wave's rows (sub: which 32-row block of the wave's C::RPW
  // rows) and its sequence; false when the work-group's query tile lies
  // wholly past the sequence's end (the same for every wave of the
  // work-group, which then returns before any DMA or barrier).
  // id: the work item (Q tile, head) in launch order; the work-group's
  // own id unless a persistent work-group passes the one it is on.
  __device__ __forceinline__ bool locate(const Problem& P, int sub, HeadRows* hr, int id) {
    // every field the set-up reads, loaded together here (one round trip to
    // the kernel arguments; left to itself the compiler loads the strides
    // only after the work-group's tile is known, a second round trip:
    // tiny 5.0 -> 4.7 us)
    asm volatile("" ::"s"(P.q), "s"(P.k), "s"(P.v), "s"(P.o), "s"(P.lse));
    asm volatile("" ::"s"(P.qb), "s"(P.qh), "s"(P.qs), "s"(P.kb), "s"(P.kh), "s"(P.ks));
    asm volatile("" ::"s"(P.vb), "s"(P.vh), "s"(P.vs), "s"(P.ob), "s"(P.oh), "s"(P.os));
    asm volatile("" ::"s"(P.lb), "s"(P.lh), "s"(P.cuq), "s"(P.B), "s"(P.H), "s"(P.Sq), "s"(P.Sk));
    asm volatile("" ::"s"(P.nqt), "s"(P.c), "s"(P.hgroup), "s"(P.compact), "s"(P.items), "s"(P.totq));
    const int tid = threadIdx.x;
    lane = tid & 63;
    // (the key-split kernel runs several groups of C::NW waves on the same rows)
    wave = __builtin_amdgcn_readfirstlane((tid >> 6) % C::NW);
    hh = lane >> 5;
    c = P.c;
    int bh;
    if (P.compact) {
      const bool xcd = (P.H & 7) == 0;
      const int m = xcd ? P.H >> 3 : P.H;
      int g, r, nt, j;
      bool dec;
      const bool any = varlen_find<C::BM>(P, m, xcd ? id >> 3 : id, &g, &r, &nt, &dec);
      if (dec) {  // offsets out of order: nothing is computed
        flag_all_rows(P, id);
        return false;
      }
      if (!any) return false;
      varlen_tile(r, m, nt, CAUSAL, &qt, &j);
      bh = g * P.H + (xcd ? (id & 7) + 8 * j : j);
    } else {
      block_to_tile(id, P.B * P.H, P.nqt, CAUSAL, &qt, &bh, P.hgroup);
    }
    const int bb = bh / P.H, h = bh - bb * P.H;
    *hr = head_rows(P, bb, h);
    Lq = hr->Lq;
    Lk = hr->Lk;
    if (hr->cut_q > 0 || hr->cut_k) {  // rare: a sequence longer than the maxima
      flag_cut_rows(P, *hr);
      return false;
    }
    if (qt * C::BM >= Lq) return false;
    off = Lk - Lq;
    q0w = qt * C::BM + wave * C::RPW + sub * kRowsPerWave;
    qrow = q0w + (lane & 31);
    return true;
  }
  // Variable lengths, a sequence longer than the stated maxima: its rows past
  // the maximum query length lie in no work-group's tile, with more keys than
  // the maximum key length its rows would see only a prefix of them, and
  // either way the causal alignment (j <= i + Lk - Lq) would use cut
  // lengths. Such a sequence is not computed: all its rows get NaN in O
  // (16-bit all-ones: a NaN in fp16 and bf16) and in lse, so the violated
  // bound shows. Each work-group of the sequence marks its own tile's rows;
  // the one with the last query tile also marks the rows past the maximum.
  // Every thread of the work-group takes a share (thread index and block
  // size).
  __device__ void flag_cut_rows(const Problem& P, const HeadRows& hr) const {
    auto mark = [&](int a, int b) {
      if (b <= a) return;
      unsigned short* const o = (unsigned short*)P.o + hr.o0;
      const long long n = (long long)(b - a) * C::D;
      for (long long i = threadIdx.x; i < n; i += blockDim.x)
        o[(long long)(a + (int)(i / C::D)) * P.os + (int)(i % C::D)] = 0xFFFFu;
      for (int r = a + (int)threadIdx.x; r < b; r += (int)blockDim.x)
        P.lse[hr.l0 + r] = __builtin_nanf("");
    };
    mark(qt * C::BM, min(hr.Lq, (qt + 1) * C::BM));
    if (qt == num_q_tiles(hr.Lq, C::BM) - 1) mark(hr.Lq, hr.Lq + hr.cut_q);
  }
  // Variable lengths (compacted launch) with offsets that decrease somewhere,
  // against the stated order: the launch's bound no longer covers every
  // tile, so no sequence is computed and every token row of every head gets
  // NaN in O and lse. Work item id of the P.items marks token rows
  // [t0, t1), its share of the totq, in every head.
  __device__ void flag_all_rows(const Problem& P, int id) const {
    const unsigned G = (unsigned)P.items, n = (unsigned)P.totq;
    const unsigned per = n / G, rem = n % G, u = (unsigned)id;
    const int t0 = (int)(u * per + (u < rem ? u : rem));
    const int t1 = t0 + (int)per + (u < rem);
    unsigned short* const o = (unsigned short*)P.o;
    const long long cnt = (long long)(t1 - t0) * C::D;  // a few work-groups may hold many rows
    for (int h = 0; h < P.H; ++h) {
      for (long long i = threadIdx.x; i < cnt; i += blockDim.x)
        o[(t0 + i / C::D) * P.os + h * P.oh + (int)(i % C::D)] = 0xFFFFu;
      for (int t = t0 + (int)threadIdx.x; t < t1; t += (int)blockDim.x)
        P.lse[h * P.lh + t] = __builtin_nanf("");
    }
  }

  __device__ __forceinline__ void reset_softmax() {
    b = -INFINITY;
    lsum = 0.f;
  }

  // KV tiles this wave computes (0 for a wave wholly past the end), and the
  // work-group's KV tile count.
  __device__ __forceinline__ int wave_tiles() const {
    return q0w < Lq ? (wave_kv_end(q0w, Lq, Lk, CAUSAL) + C::BN - 1) / C::BN : 0;
  }
  __device__ __forceinline__ int group_tiles() const {
    return (tile_kv_end(qt, Lq, Lk, CAUSAL, C::BM) + C::BN - 1) / C::BN;
  }
  // Leading KV tiles that need no index compares for these rows
  __device__ __forceinline__ int unmasked_tiles() const {
    return fa::unmasked_tiles(q0w, Lq, Lk, CAUSAL, C::BN);
  }
  // the tile starting at key kv0 needs index compares (diagonal or ragged end)
  __device__ __forceinline__ bool needs_mask(int kv0) const {
    return (CAUSAL && kv0 + C::BN - 1 > q0w + off) || kv0 + C::BN > Lk;
  }
  // running max with lag over one tile's scores (each lane holds 16 per
  // 32-key block): new base b and history factor 2^(b_old - b_new)
  template <int NKB> __device__ __forceinline__ float softmax_max(const f32x16 (&s)[NKB]) {
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = vmax(mx, s[kb][r]);
    mx = max_xor32(mx);
    const float cand = vmax(b, mx * c);
    const bool rebase = cand > b + (float)THR;
    const float hist = rebase ? __builtin_amdgcn_exp2f(b - cand) : 1.f;  // 0 on the first tile
    b = rebase ? cand : b;
    lsum *= hist;
    return hist;
  }
};

template <int R, class X> __device__ __forceinline__ X pick3(X a, X b, X c) {
  if constexpr (R == 0) return a;
  else if constexpr (R == 1) return b;
  else return c;
}

}  // namespace fa
