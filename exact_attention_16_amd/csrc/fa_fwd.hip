// Fused attention forward for AMD Instinct MI355X (gfx950, CDNA4).
//
// Each wave owns 32 query rows of one (batch, head) for the whole kernel,
// with its Q rows held in registers as MFMA operands, and streams the K/V
// tiles of that head through LDS. Per KV tile j a wave computes
//   S(j) = K(j) Q^T          (v_mfma_f32_32x32x16, raw dot products in fp32)
//   softmax(S(j)) -> P(j)    (VALU: tile max, lagging base, exp2, row sum)
//   O^T += V(j)^T P(j)^T     (v_mfma_f32_32x32x16)
// and at the end normalises once and writes O and the row logsumexp.
//
// Data movement: K and V tiles go from HBM to LDS by buffer loads with the
// LDS bit (direct DMA, 16 bytes per lane; no staging registers, no VALU),
// whose range check zero-fills rows past the end of the sequence. K is read
// back as 16-byte S^T operand fragments (no transpose); V^T operand
// fragments come from the row-major V tile through ds_read_b64_tr_b16,
// which transposes in the LDS crossbar. Both tiles are XOR-swizzled per row
// so that the operand reads are free of bank conflicts.
//
// Softmax: base 2 with a lagging running base b per row (log2 units of the
// scaled logit). The tile max of the raw dot products is exchanged between
// the two lanes of a row with v_permlane32_swap; b moves only when the
// candidate exceeds b + THR, with history factor 2^(b_old - b_new); p =
// 2^(s*c - b) with c = scale*log2(e), so p <= 2^THR. Row sums accumulate the
// unrounded fp32 p; P is rounded once to the input type for the MFMA. The
// O rescale is skipped, wave-uniformly, unless a ballot finds a row with
// history < 1. Causal tiles wholly above the diagonal are never visited;
// only tiles crossing the diagonal or the ragged end compare indices.
//
// Two kernels overlap the matrix cores and the vector ALU differently:
//  * fa_fwd_pp (eight waves, 256 query rows): the waves form two groups
//    whose slots alternate between an MFMA phase (P(j-1).V(j-1) and
//    K(j).Q^T) and a softmax phase, offset by one slot, so each SIMD always
//    holds one multiplying and one exponentiating wave; K/V use three LDS
//    stages, issued two tiles ahead.
//  * fa_fwd_k4 (four waves, 128 query rows), for grids too small to fill the
//    chip with 256-row tiles: each wave overlaps the next tile's K.Q^T (and,
//    at D=64, the previous tile's P.V) with its own current softmax; two LDS
//    stages.
//
// Method sources: exact attention softmax(QK^T/sqrt(d)+mask)V with a
// lower-triangle causal mask (xdnf.cn, "CUDA手写masked multi-head attention
// 性能优化实战", 3.1); tiling with running max/sum, v2 loop order, deferred
// normalisation and the (Q tile, head) grid (hotdry.top, "FlashAttention的
// Triton性能考古学", sections "核心算法回顾" and "FlashAttention v2：循环重构与
// 寄存器积累"); the conditional rescale with a lag of 8 and p in (0, 256], the
// warp-vote skip of the rescale, the rescale done by the softmax workers
// themselves, and issuing the next tile's Q.K^T ahead of the current P.V
// (hjcheng0602.cn, "Flash Attention CUDA Kernel 优化 ... G6", V39, V41, V44).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/fa_fwd.h"
#include "fa_layout.h"

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

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;
// Word 3 of a raw (untyped, stride 0) gfx9 buffer descriptor.
constexpr int kBufferWord3 = 0x00020000;

template <int N> struct IC { static constexpr int value = N; };
template <int P, class X> __device__ __forceinline__ X& pick(X& one, X& zero) {
  if constexpr (P != 0) return one; else return zero;
}

template <typename T> struct Ops;

template <> struct Ops<__bf16> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // two fp32 -> packed pair, round to nearest even
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
  }
};

template <> struct Ops<_Float16> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
  }
};

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
#define FA_RSRC(base, bytes) \
  __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>((const void*)(base)), 0, (int)(bytes), kBufferWord3)

// LDS pointers stay in address space 3 from the point where each shared
// array is declared (a cast of a generic pointer to address space 3 would
// make the host compilation pass drop the kernel launch stubs).
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ u32x4 lds16(const lds_char* p) { return *(lds_u32x4*)p; }

// V^T operand: two transposed 8-byte reads (keys +0..3 and +4..7)
__device__ __forceinline__ u32x4 lds_tr_pair(const lds_char* p, uint32_t second) {
  const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + second));
  const u32x2 x = __builtin_bit_cast(u32x2, x0), y = __builtin_bit_cast(u32x2, x1);
  return (u32x4){x[0], x[1], y[0], y[1]};
}

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

// Scheduling pattern for one region: DS0 LDS reads up front, then REPS
// times {one MFMA, V1 VALU, DS LDS reads, one MFMA, V2 VALU}.
template <int DS0, int REPS, int V1, int DS, int V2>
__device__ __forceinline__ void interleave() {
  __builtin_amdgcn_sched_group_barrier(0x100, DS0, 0);
#pragma unroll
  for (int i = 0; i < REPS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, V1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, DS, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, V2, 0);
  }
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

// One wave's share of a work-group: its query rows, accumulators and the
// per-tile operations on them.
template <typename T, class C, bool CAUSAL, int THR, bool DIAG>
struct Wave {
  static constexpr int D = C::D;
  static constexpr int BN = C::BN;
  static constexpr int NKB = BN / 32;  // 32-key blocks per KV tile
  static constexpr int NDC = D / 16;   // Q.K^T contraction steps (16 d each)
  static constexpr int NDB = D / 32;   // 32-row d blocks of O^T
  static constexpr int NKC = BN / 16;  // P.V contraction steps (16 keys each)
  static constexpr int DPW = C::dmaPerWave;
  static constexpr uint32_t RB = C::rowBytes;

  int lane, wave, hh, S, q0w, qrow, qt, bh;
  float c;  // scale * log2(e)
  const T* Kh;
  const T* Vh;
  uint32_t koff0, voff0, kdo0, vdo0;
  u32x4 qf[NDC];
  f32x16 o[NDB];
  float b, lsum;
  unsigned n_events;

  // sub: which 32-row block of the wave's C::RPW rows this object holds
  __device__ __forceinline__ void init(const T* Q, const T* K, const T* V, int BH, int S_, int nqt,
                                       float c_, int sub = 0) {
    const int tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    hh = lane >> 5;
    S = S_;
    c = c_;
    block_to_tile(blockIdx.x, BH, nqt, CAUSAL, &qt, &bh);
    const size_t head = (size_t)bh * (size_t)S * D;
    Kh = K + head;
    Vh = V + head;
    q0w = qt * C::BM + wave * C::RPW + sub * kRowsPerWave;
    qrow = q0w + (lane & 31);
    // Q operand fragments (rows past S read as zeros)
    const auto rq = FA_RSRC(Q + head, (uint32_t)S * RB);
#pragma unroll
    for (int j = 0; j < NDC; ++j)
      qf[j] = __builtin_amdgcn_raw_buffer_load_b128(rq, q_frag_off<D>(qrow, j, hh), 0, 0);
    // per-lane LDS / DMA base offsets; the rest are XOR / immediate offsets
    koff0 = k_read_off<D>(0, 0, lane);
    voff0 = v_tr_off<D>(0, 0, 0, lane);
    kdo0 = dma_src_k<C>(wave, 0, lane);
    vdo0 = dma_src_v<C>(wave, 0, lane);
#pragma unroll
    for (int j = 0; j < NDB; ++j) o[j] = (f32x16){};
    b = -INFINITY;  // running base, log2 units (lags the true max by <= THR)
    lsum = 0.f;     // this lane's partial row sum (its k-half of the keys)
    n_events = 0;
  }

  // KV tiles this wave computes (0 for a wave wholly past the end), and the
  // work-group's KV tile count.
  __device__ __forceinline__ int wave_tiles() const {
    return q0w < S ? (wave_kv_end(q0w, S, CAUSAL) + BN - 1) / BN : 0;
  }
  __device__ __forceinline__ int group_tiles() const {
    return (tile_kv_end(qt, S, CAUSAL, C::BM) + BN - 1) / BN;
  }

  // Leading KV tiles that need no index compares for these rows: tiles
  // before the one holding key q0w (causal) and before the ragged end.
  __device__ __forceinline__ int unmasked_tiles() const {
    const int r = S / BN;
    const int d = q0w / BN;
    return CAUSAL ? (d < r ? d : r) : r;
  }

  // this wave's share of the DMA of K or V tile t into an LDS stage; a tile
  // at or past `limit` is an empty range (the DMA then writes zeros)
  __device__ __forceinline__ void dma_k(lds_char* dst, int t, int limit = 0x7fffffff) const {
    const int kv0 = t * BN;
    const uint32_t bytes = t < limit ? (uint32_t)(S - kv0) * RB : 0u;
    const auto r = FA_RSRC(Kh + (size_t)kv0 * D, bytes);
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      // (the LDS pointer goes through a local: written inline as the builtin's
      // argument, the host compilation pass drops the kernel launch stubs)
      lds_char* const lp = dst + dma_lds_k<C>(wave, i);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lp, 16, kdo0 + i * C::dmaStrideK, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void dma_v(lds_char* dst, int t, int limit = 0x7fffffff) const {
    const int kv0 = t * BN;
    const uint32_t bytes = t < limit ? (uint32_t)(S - kv0) * RB : 0u;
    const auto r = FA_RSRC(Vh + (size_t)kv0 * D, bytes);
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      lds_char* const lp = dst + dma_lds_v<C>(wave, i);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lp, 16, vdo0 + i * C::dmaStrideV, 0, 0, 0);
    }
  }

  // S^T = K Q^T for the tile at kt (step 0 starts from a zero accumulator)
  __device__ __forceinline__ void qk(f32x16 (&s)[NKB], const lds_char* kt) const {
#pragma unroll
    for (int j = 0; j < NDC; ++j) {
      const lds_char* base = kt + (koff0 ^ (uint32_t)(j << 5));
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        s[kb] = Ops<T>::mfma(lds16(base + kb * 32 * RB), qf[j], j == 0 ? (f32x16){} : s[kb]);
    }
  }
  // O^T += V^T P^T for the tile at vt
  __device__ __forceinline__ void pv(const u32x4 (&p)[NKC], const lds_char* vt) {
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
      for (int jd = 0; jd < NDB; ++jd)
        o[jd] = Ops<T>::mfma(lds_tr_pair(vt + (voff0 ^ (uint32_t)(jd << 6)) + kc * 16 * RB, 4 * RB),
                             p[kc], o[jd]);
  }
  // the tile starting at key kv0 needs index compares (diagonal or ragged end)
  __device__ __forceinline__ bool needs_mask(int kv0) const {
    return (CAUSAL && kv0 + BN - 1 > q0w) || kv0 + BN > S;
  }
  __device__ __forceinline__ void mask(f32x16 (&s)[NKB], int kv0) const {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 32 * kb + acc_key32(r, hh);
        const bool vis = key < S && (!CAUSAL || key <= qrow);
        s[kb][r] = vis ? s[kb][r] : -INFINITY;
      }
  }
  // running max with lag: new base b and history factor 2^(b_old - b_new)
  __device__ __forceinline__ float softmax_max(const f32x16 (&s)[NKB]) {
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
  // p = 2^(s*c - b), row sum of the unrounded p, P packed for the P.V MFMA
  __device__ __forceinline__ void softmax_exp(const f32x16 (&s)[NKB], u32x4 (&p)[NKC]) {
    const float nb = (b == -INFINITY) ? 0.f : -b;  // fully hidden row: p = 0
    float ls[4] = {0.f, 0.f, 0.f, 0.f};  // four sum chains, so no add waits on the one before
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float e[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          e[x] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * g + x], c, nb));
          ls[x & 3] += e[x];
        }
        p[2 * kb + g] = (u32x4){Ops<T>::pack2(e[0], e[1]), Ops<T>::pack2(e[2], e[3]),
                                Ops<T>::pack2(e[4], e[5]), Ops<T>::pack2(e[6], e[7])};
      }
    lsum += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  }
  // rare path: some row of the wave moved its base -> rescale O
  __device__ __forceinline__ void rescale(int j, float hist) {
    if (DIAG && j >= 1 && hh == 0 && qrow < S && hist < 1.f) ++n_events;
    if (j >= 1 && __builtin_amdgcn_ballot_w64(hist < 1.f) != 0) {
#pragma unroll
      for (int jd = 0; jd < NDB; ++jd) o[jd] *= hist;
    }
  }
  // softmax of tile j in place: mask, base update, rescale of O, P(j)
  __device__ __forceinline__ void softmax_tile(f32x16 (&s)[NKB], u32x4 (&p)[NKC], int j) {
    const int kv0 = j * BN;
    if (needs_mask(kv0)) mask(s, kv0);
    const float hist = softmax_max(s);
    rescale(j, hist);
    softmax_exp(s, p);
  }

  // normalise once, write O and lse (rows past S dropped by the range check)
  __device__ __forceinline__ void epilogue(T* O, float* LSE, unsigned long long* events) {
    const float ltot = sum_xor32(lsum);
    if (q0w < S) {
      const size_t head = (size_t)bh * (size_t)S * D;
      const auto ro = FA_RSRC(O + head, (uint32_t)S * RB);
      const auto rl = FA_RSRC(LSE + (size_t)bh * S, (uint32_t)S * 4u);
      const float inv = 1.f / ltot;
#pragma unroll
      for (int jd = 0; jd < NDB; ++jd)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const f32x16& a = o[jd];
          const int r0 = 8 * g;
          const u32x4 w = {Ops<T>::pack2(a[r0 + 0] * inv, a[r0 + 1] * inv),
                           Ops<T>::pack2(a[r0 + 2] * inv, a[r0 + 3] * inv),
                           Ops<T>::pack2(a[r0 + 4] * inv, a[r0 + 5] * inv),
                           Ops<T>::pack2(a[r0 + 6] * inv, a[r0 + 7] * inv)};
          // accumulator element r0+e of lane (i, hh) is d = 32jd + 16g + 8hh + e
          __builtin_amdgcn_raw_buffer_store_b128(w, ro, o_frag_off<D>(qrow, jd, g, hh), 0, 0);
        }
      if (hh == 0) {
        const float l2 = (b + __builtin_amdgcn_logf(ltot)) * kLn2;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, l2), rl,
                                              (uint32_t)qrow * 4u, 0, 0);
      }
    }
    if (DIAG && n_events) atomicAdd(events, (unsigned long long)n_events);
  }
};

// ------------------------------------------------- eight-wave ping-pong
template <int R, class X> __device__ __forceinline__ X pick3(X a, X b, X c) {
  if constexpr (R == 0) return a;
  else if constexpr (R == 1) return b;
  else return c;
}

template <typename T, int D, bool CAUSAL, int THR, bool DIAG>
__global__ void __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd_pp(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
          T* __restrict__ O, float* __restrict__ LSE, int BH, int S, int nqt, float c,
          unsigned long long* __restrict__ events) {
  using C = Cfg8<D>;
  using W = Wave<T, C, CAUSAL, THR, DIAG>;
  constexpr int TB = C::tileBytes;
  constexpr int DPW = C::dmaPerWave;
  constexpr bool ONE = pp_one_barrier<D>;  // one barrier per step, else two
  static_assert(kStages == 3, "the step below is unrolled over three stages");
  // One array per stage: with the stage fixed at compile time the compiler
  // sees that an LDS read never aliases the DMA in flight into another stage
  // and inserts no wait for it. The compiler lays the arrays out in name
  // order; the V stages are named to come first, so that their transposed
  // reads (two per P.V MFMA, the part of the MFMA phase with the most
  // instructions per MFMA) mostly fit the 16-bit offset field of the LDS
  // instruction and need no address arithmetic. This affects speed only.
  __shared__ __attribute__((aligned(1024))) char a_vstage0[TB];
  __shared__ __attribute__((aligned(1024))) char a_vstage1[TB];
  __shared__ __attribute__((aligned(1024))) char a_vstage2[TB];
  __shared__ __attribute__((aligned(1024))) char b_kstage0[TB];
  __shared__ __attribute__((aligned(1024))) char b_kstage1[TB];
  __shared__ __attribute__((aligned(1024))) char b_kstage2[TB];
  lds_char* const lk0 = (lds_char*)b_kstage0;
  lds_char* const lk1 = (lds_char*)b_kstage1;
  lds_char* const lk2 = (lds_char*)b_kstage2;
  lds_char* const lv0 = (lds_char*)a_vstage0;
  lds_char* const lv1 = (lds_char*)a_vstage1;
  lds_char* const lv2 = (lds_char*)a_vstage2;

  W w;
  w.init(Q, K, V, BH, S, nqt, c);
  const int grp = w.wave >> 2;  // 0: waves 0-3, 1: waves 4-7 (one of each per SIMD)
  const int ntiles = w.group_tiles();
  const int nw = w.wave_tiles();
  f32x16 s[W::NKB];  // S(j), from its MFMA phase to its softmax phase
  u32x4 p[W::NKC];   // P(j), from its softmax phase to the next MFMA phase

  // DMA pair i (issued in slot 2i, R = i mod 3): K(i+2) and V(i+1), as
  // empty ranges where those tiles do not exist, so that every pair is the
  // same 2*DPW issues and each wait below is a constant count.
  auto dma_pair = [&](auto r, int i) {
    constexpr int R = decltype(r)::value;
    w.dma_k(pick3<(R + 2) % 3>(lk0, lk1, lk2), i + 2, ntiles);
    w.dma_v(pick3<(R + 1) % 3>(lv0, lv1, lv2), i + 1, ntiles);
  };
  // End of a slot: this wave's LDS reads are done and all its DMA except the
  // latest pair has landed; then the work-group barrier.
  auto end_slot = [&]() {
    wait_vm_lgkm0<2 * DPW>();
    wg_barrier();
  };

  // prologue: K(0), K(1), V(0) in their stages; the other stages get empty
  // ranges so that the compiler tracks a DMA into every stage from the first
  // block on (an LDS read then waits only for DMA into its own stage).
  w.dma_k(lk0, 0);
  w.dma_k(lk1, 1, ntiles);
  w.dma_k(lk2, 2, 0);
  w.dma_v(lv0, 0);
  w.dma_v(lv1, 1, 0);
  w.dma_v(lv2, 2, 0);
  __builtin_amdgcn_s_waitcnt(0);
  wg_barrier();

  // With two barriers per step group A runs step j in slots (2j, 2j+1),
  // group B in (2j+1, 2j+2): B takes slot 0 alone first and A takes the last
  // slot alone at the end, so both groups pass the same number of barriers.
  // With one, slot j holds A's step j and B's softmax phase of step j-1 and
  // MFMA phase of step j. Each group has its own
  // copy of the loop, in which every DMA is unconditional: the compiler's
  // count of DMA in flight then matches the constant waits on every path.
  auto run = [&](auto g) {
    constexpr int G = decltype(g)::value;
    if constexpr (G == 1) {
      dma_pair(IC<0>{}, 0);
      if constexpr (!ONE) end_slot();
    }
    // step j (R = j mod 3): MFMA phase P(j-1).V(j-1) + S(j) = K(j) Q^T, then
    // the softmax phase of S(j). K(j) sits in stage R, V(j-1) in stage R-1.
    // The MFMA phase runs at raised wave priority, so that on each SIMD the
    // multiplying wave's MFMAs and LDS reads issue ahead of the other
    // wave's exponentials whenever both are ready.
    auto step = [&](auto r, int j) {
      constexpr int R = decltype(r)::value;
      __builtin_amdgcn_s_setprio(1);
      if constexpr (G == 0) dma_pair(r, j);
      __builtin_amdgcn_sched_barrier(0);
      if (j >= 1 && j - 1 < nw) {
        w.pv(p, pick3<(R + 2) % 3>(lv0, lv1, lv2));
        read_ahead<8, W::NKC * W::NDB, 2>();  // two reads per MFMA, four MFMAs ahead
      }
      if (j < nw) {
        w.qk(s, pick3<R>(lk0, lk1, lk2));
        read_ahead<4, W::NDC * W::NKB, 1>();  // one read per MFMA, four MFMAs ahead
      }
      if constexpr (ONE) {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (G == 1) end_slot();
      } else {
        end_slot();
      }
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      if (j < nw) w.softmax_tile(s, p, j);
      // group B's DMA share goes after its softmax work, clear of group A's
      // issues at the start of the slot
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (G == 1) dma_pair(IC<(R + 1) % 3>{}, j + 1);
      if constexpr (!ONE || G == 0) end_slot();
    };
    for (int j = 0;; j += 3) {
      step(IC<0>{}, j);
      if (j + 1 > ntiles) break;
      step(IC<1>{}, j + 1);
      if (j + 2 > ntiles) break;
      step(IC<2>{}, j + 2);
      if (j + 3 > ntiles) break;
    }
    if constexpr (G == 0 && !ONE) end_slot();
  };
  if (grp == 0) run(IC<0>{});
  else run(IC<1>{});
  __builtin_amdgcn_s_waitcnt(0);  // no DMA into LDS outlives the work-group
  w.epilogue(O, LSE, events);
}

// ------------------------------------------------- four waves x 64 rows
// Each wave holds two 32-row blocks A and B. Per 32-key tile j, in program
// order (one scheduling region each, so the compiler interleaves the two
// independent streams):
//   part a: S_A(j), S_B(j) = K(j) Q^T (each K fragment read once, two MFMAs)
//           with block B's exponentials of tile j-1 -> P_B(j-1)
//   part b: O_A += P_A(j-1) V(j-1), O_B += P_B(j-1) V(j-1) (each V fragment
//           read once) with block A's softmax of tile j -> P_A(j) and block
//           B's tile max of tile j (its new base applies from part a on)
//   then the rare O rescales, a wait for the DMA and one barrier.
// K and V tiles use three LDS stages, issued two tiles ahead as in the
// eight-wave kernel.
template <typename T, int D, bool CAUSAL, int THR, bool DIAG>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(1, 1)))
fa_fwd_w2(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
          T* __restrict__ O, float* __restrict__ LSE, int BH, int S, int nqt, float c,
          unsigned long long* __restrict__ events) {
  using C = CfgW2<D>;
  using W = Wave<T, C, CAUSAL, THR, DIAG>;
  constexpr int TB = C::tileBytes;
  constexpr int DPW = C::dmaPerWave;
  constexpr int NKB = W::NKB, NKC = W::NKC, NDC = W::NDC, NDB = W::NDB;
  constexpr uint32_t RB = C::rowBytes;
  static_assert(kStages == 3, "the step below is unrolled over three stages");
  // one array per stage, V stages first in name order (as in fa_fwd_pp)
  __shared__ __attribute__((aligned(1024))) char b_kstage0[TB];
  __shared__ __attribute__((aligned(1024))) char b_kstage1[TB];
  __shared__ __attribute__((aligned(1024))) char b_kstage2[TB];
  __shared__ __attribute__((aligned(1024))) char a_vstage0[TB];
  __shared__ __attribute__((aligned(1024))) char a_vstage1[TB];
  __shared__ __attribute__((aligned(1024))) char a_vstage2[TB];
  lds_char* const lk0 = (lds_char*)b_kstage0;
  lds_char* const lk1 = (lds_char*)b_kstage1;
  lds_char* const lk2 = (lds_char*)b_kstage2;
  lds_char* const lv0 = (lds_char*)a_vstage0;
  lds_char* const lv1 = (lds_char*)a_vstage1;
  lds_char* const lv2 = (lds_char*)a_vstage2;

  W wa, wb;
  wa.init(Q, K, V, BH, S, nqt, c, 0);
  wb.init(Q, K, V, BH, S, nqt, c, 1);
  const int ntiles = wa.group_tiles();
  // tiles either block computes (block B's rows can lie wholly past S)
  const int nlast = max(wa.wave_tiles(), wb.wave_tiles());
  const int nfull = wa.unmasked_tiles();  // tiles before this is < both blocks' first masked

  // Double buffers, alternating by iteration parity: S_B(j-1) / S_B(j) and
  // P_A(j-1) / P_A(j). Before the first tile S_B = -inf and P_A = 0, so that
  // iteration 0 runs the same code (its block-B exponentials give P_B = 0
  // and its P.V adds zeros from the zero-filled stage).
  f32x16 sA[NKB], sB0[NKB], sB1[NKB];
  u32x4 pA0[NKC], pA1[NKC], pB[NKC];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) sB0[kb] = (f32x16){} - INFINITY;
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) pA0[kc] = (u32x4){};

  // both blocks' S for the K tile at kt: one LDS read per fragment
  auto qk2 = [&](const lds_char* kt, f32x16 (&sb)[NKB]) {
#pragma unroll
    for (int j = 0; j < NDC; ++j) {
      const lds_char* base = kt + (wa.koff0 ^ (uint32_t)(j << 5));
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const u32x4 kf = lds16(base + kb * 32 * RB);
        sA[kb] = Ops<T>::mfma(kf, wa.qf[j], j == 0 ? (f32x16){} : sA[kb]);
        sb[kb] = Ops<T>::mfma(kf, wb.qf[j], j == 0 ? (f32x16){} : sb[kb]);
      }
    }
  };
  // both blocks' O for the V tile at vt: one LDS read per fragment
  auto pv2 = [&](const lds_char* vt, const u32x4 (&pa)[NKC]) {
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
      for (int jd = 0; jd < NDB; ++jd) {
        const u32x4 vf =
            lds_tr_pair(vt + (wa.voff0 ^ (uint32_t)(jd << 6)) + kc * 16 * RB, 4 * RB);
        wa.o[jd] = Ops<T>::mfma(vf, pa[kc], wa.o[jd]);
        wb.o[jd] = Ops<T>::mfma(vf, pB[kc], wb.o[jd]);
      }
  };
  auto dma_pair = [&](auto r, int i) {
    constexpr int R = decltype(r)::value;
    wa.dma_k(pick3<(R + 2) % 3>(lk0, lk1, lk2), i + 2, ntiles);
    wa.dma_v(pick3<(R + 1) % 3>(lv0, lv1, lv2), i + 1, ntiles);
  };

  // prologue: K(0), K(1), V(0); the other stages get empty ranges (zeros),
  // which also gives the compiler a DMA into every stage from the first
  // block on
  wa.dma_k(lk0, 0);
  wa.dma_k(lk1, 1, ntiles);
  wa.dma_k(lk2, 2, 0);
  wa.dma_v(lv0, 0);
  wa.dma_v(lv1, 1, 0);
  wa.dma_v(lv2, 2, 0);
  __builtin_amdgcn_s_waitcnt(0);
  wg_barrier();

  // Iteration j = 0 .. ntiles (R = j mod 3, P = j mod 2): K(j) in stage R,
  // V(j-1) in stage R-1. Tiles a block cannot see at all are masked to
  // -inf like any other, giving p = 0; a wave past its last tile only
  // issues its DMA share and meets the barrier.
  auto step = [&](auto r, auto par, int j) {
    constexpr int R = decltype(r)::value;
    constexpr int P = decltype(par)::value;
    f32x16(&sBo)[NKB] = pick<P>(sB1, sB0);  // S_B(j-1)
    f32x16(&sBn)[NKB] = pick<P>(sB0, sB1);  // S_B(j)
    u32x4(&pAo)[NKC] = pick<P>(pA1, pA0);   // P_A(j-1)
    u32x4(&pAn)[NKC] = pick<P>(pA0, pA1);   // P_A(j)
    dma_pair(r, j);
    __builtin_amdgcn_sched_barrier(0);
    if (j <= nlast) {
      // part a: S_A(j), S_B(j); block B's exponentials of tile j-1. P_B
      // and B's row sum are pinned here, beside the MFMAs they overlap.
      qk2(pick3<R>(lk0, lk1, lk2), sBn);
      wb.softmax_exp(sBo, pB);
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) asm volatile("" : "+v"(pB[kc]));
      asm volatile("" : "+v"(wb.lsum));
      interleave<2, NDC * NKB, 4, 1, 4>();
      if (j >= nfull) {
        const int kv0 = j * W::BN;
        wa.mask(sA, kv0);
        wb.mask(sBn, kv0);
      }
      // part b: P.V of tile j-1 for both blocks; block A's softmax of tile
      // j; block B's max of tile j
      pv2(pick3<(R + 2) % 3>(lv0, lv1, lv2), pAo);
      const float hA = wa.softmax_max(sA);
      wa.softmax_exp(sA, pAn);
      const float hB = wb.softmax_max(sBn);
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) asm volatile("" : "+v"(pAn[kc]));
      asm volatile("" : "+v"(wa.lsum));
      interleave<4, NKC * NDB, 6, 2, 6>();
      // rare: move O to the new bases (after this P.V, before the next)
      wa.rescale(j, hA);
      wb.rescale(j, hB);
    }
    wait_vm_lgkm0<2 * DPW>();
    wg_barrier();
  };
  for (int j = 0;; j += 6) {
    step(IC<0>{}, IC<0>{}, j);
    if (j + 1 > ntiles) break;
    step(IC<1>{}, IC<1>{}, j + 1);
    if (j + 2 > ntiles) break;
    step(IC<2>{}, IC<0>{}, j + 2);
    if (j + 3 > ntiles) break;
    step(IC<0>{}, IC<1>{}, j + 3);
    if (j + 4 > ntiles) break;
    step(IC<1>{}, IC<0>{}, j + 4);
    if (j + 5 > ntiles) break;
    step(IC<2>{}, IC<1>{}, j + 5);
    if (j + 6 > ntiles) break;
  }
  __builtin_amdgcn_s_waitcnt(0);  // no DMA into LDS outlives the work-group
  wa.epilogue(O, LSE, events);
  wb.epilogue(O, LSE, events);
}

// ------------------------------------------------------------ four-wave
// Register pipeline depth per head dimension. D=64: three stages (S(j+1),
// P(j-1).V(j-1) and softmax(j) in one block) fit two waves per SIMD. D=128:
// two stages (the history from the tile max alone, the rare rescale, then
// one block with the exponentials, P(j).V(j) and S(j+1)); the other wave on
// the SIMD covers the rest.
template <int D> struct Pipe { static constexpr bool three = D == 64; };

template <typename T, int D, bool CAUSAL, int THR, bool DIAG>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd_k4(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
          T* __restrict__ O, float* __restrict__ LSE, int BH, int S, int nqt, float c,
          unsigned long long* __restrict__ events) {
  using C = Cfg4<D>;
  using W = Wave<T, C, CAUSAL, THR, DIAG>;
  constexpr bool P3 = Pipe<D>::three;
  constexpr int NKB = W::NKB, NKC = W::NKC;
  constexpr int TB = C::tileBytes;
  // one array per stage, V stages first in name order (as in fa_fwd_pp)
  __shared__ __attribute__((aligned(1024))) char b_kstage0[TB];
  __shared__ __attribute__((aligned(1024))) char b_kstage1[TB];
  __shared__ __attribute__((aligned(1024))) char a_vstage0[TB];
  __shared__ __attribute__((aligned(1024))) char a_vstage1[TB];
  lds_char* const lk0 = (lds_char*)b_kstage0;
  lds_char* const lk1 = (lds_char*)b_kstage1;
  lds_char* const lv0 = (lds_char*)a_vstage0;
  lds_char* const lv1 = (lds_char*)a_vstage1;

  W w;
  w.init(Q, K, V, BH, S, nqt, c);
  const int ntiles = w.group_tiles();
  const int nw = w.wave_tiles();

  f32x16 sA[NKB], sB[NKB];  // S(j) lives in sA for even j, sB for odd j
  u32x4 pA[NKC], pB[NKC];   // P(j) likewise (only pA is used with two stages)
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) pB[kc] = (u32x4){};  // P(-1) = 0

  // ---- prologue: K(0), K(1) (and V(0) with two stages) in LDS; S(0) --------
  // With three stages iteration 0 runs the steady-state block with P(-1) = 0
  // against V buffer 1, so that buffer must hold finite values (0 * NaN
  // would poison O).
  w.dma_k(lk0, 0);
  if (ntiles > 1) w.dma_k(lk1, 1);
  if constexpr (P3) {
#pragma unroll
    for (int i = 0; i < TB / (16 * C::threads); ++i)
      *(__attribute__((address_space(3))) u32x4*)(lv1 + 16 * (threadIdx.x + i * C::threads)) =
          (u32x4){};
  } else {
    w.dma_v(lv0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (nw > 0) w.qk(sA, lk0);
  __syncthreads();  // b_kstage0 is refilled with K(2) in iteration 0

  // ---- iteration j (PH = j % 2). DMA first (K(j+2); V(j) with three stages,
  // V(j+1) with two). A wave that still has tile j then computes; at its
  // last tile the S(j+1) it computes is not used. With three stages
  // iteration nw only drains P(nw-1).V(nw-1). The wave keeps issuing its
  // share of the DMA and the barriers until the work-group's last tile.
  auto iter = [&](auto ph, int j) {
    constexpr int PH = decltype(ph)::value;
    f32x16(&scur)[NKB] = pick<PH>(sB, sA);
    f32x16(&snext)[NKB] = pick<PH>(sA, sB);
    u32x4(&pcur)[NKC] = P3 ? pick<PH>(pB, pA) : pA;
    u32x4(&pprev)[NKC] = pick<PH>(pA, pB);
    lds_char* k_next = PH ? lk0 : lk1;  // holds K(j+1)
    lds_char* k_dma = PH ? lk1 : lk0;   // receives K(j+2)
    lds_char* v_cur = PH ? lv1 : lv0;   // V(j) (two stages) / receives V(j) (three)
    lds_char* v_oth = PH ? lv0 : lv1;   // V(j-1) (three stages) / receives V(j+1) (two)
    if constexpr (P3) {
      if (j < ntiles) w.dma_v(v_cur, j);
    } else {
      if (j + 1 < ntiles) w.dma_v(v_oth, j + 1);
    }
    if (j + 2 < ntiles) w.dma_k(k_dma, j + 2);
    __builtin_amdgcn_sched_barrier(0);

    if (j < nw) {
      const int kv0 = j * W::BN;
      if (w.needs_mask(kv0)) w.mask(scur, kv0);
      if constexpr (P3) {
        // one block: P(j-1).V(j-1) and S(j+1) MFMAs under softmax(j); the
        // rescale of O by softmax(j)'s history follows P(j-1).V(j-1). P(j)
        // and the row sum are pinned in the block instead of sinking past
        // the rescale branch.
        w.pv(pprev, v_oth);
        const float hist = w.softmax_max(scur);
        w.softmax_exp(scur, pcur);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) asm volatile("" : "+v"(pcur[kc]));
        asm volatile("" : "+v"(w.lsum));
        w.qk(snext, k_next);
        w.rescale(j, hist);
      } else {
        // the history is known from the tile max alone: rescale O first,
        // then one block with the exponentials, P(j).V(j) (each 16-key chunk
        // as soon as its P is packed) and the S(j+1) MFMAs
        const float hist = w.softmax_max(scur);
        w.rescale(j, hist);
        w.softmax_exp(scur, pcur);
        w.pv(pcur, v_cur);
        w.qk(snext, k_next);
      }
    } else if (P3 && j == nw) {
      w.pv(pprev, v_oth);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  const int niter = P3 ? ntiles + 1 : ntiles;
  int j = 0;
  for (; j + 1 < niter; j += 2) {
    iter(IC<0>{}, j);
    iter(IC<1>{}, j + 1);
  }
  if (j < niter) iter(IC<0>{}, j);

  w.epilogue(O, LSE, events);
}

// ------------------------------------------------------------------- host

// Kernel choice: the ping-pong kernel when its 256-row tiles give at least
// one work-group per compute unit, else the four-wave kernel.
constexpr long long kPingPongMinGroups = 256;

enum Variant { kAuto = 0, kFourWave = 1, kPingPong = 2, kTwoBlock = 3 };

template <int D> static bool use_pingpong(int BH, int S, int variant) {
  if (variant == kFourWave) return false;
  if (variant == kPingPong) return true;
  return (long long)num_q_tiles(S, Cfg8<D>::BM) * BH >= kPingPongMinGroups;
}

template <typename T, int D, bool CAUSAL, int THR, bool DIAG>
static int launch_one(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int S, float scale, hipStream_t stream, unsigned long long* ev,
                      int variant) {
  const int BH = B * H;
  const float c = scale * kLog2e;
  if (variant == kTwoBlock) {
    const int nqt = num_q_tiles(S, CfgW2<D>::BM);
    hipLaunchKernelGGL((fa_fwd_w2<T, D, CAUSAL, THR, DIAG>), dim3((unsigned)nqt * (unsigned)BH),
                       dim3(CfgW2<D>::threads), 0, stream, (const T*)q, (const T*)k, (const T*)v,
                       (T*)o, lse, BH, S, nqt, c, ev);
  } else if (use_pingpong<D>(BH, S, variant)) {
    const int nqt = num_q_tiles(S, Cfg8<D>::BM);
    hipLaunchKernelGGL((fa_fwd_pp<T, D, CAUSAL, THR, DIAG>), dim3((unsigned)nqt * (unsigned)BH),
                       dim3(Cfg8<D>::threads), 0, stream, (const T*)q, (const T*)k, (const T*)v,
                       (T*)o, lse, BH, S, nqt, c, ev);
  } else {
    const int nqt = num_q_tiles(S, Cfg4<D>::BM);
    hipLaunchKernelGGL((fa_fwd_k4<T, D, CAUSAL, THR, DIAG>), dim3((unsigned)nqt * (unsigned)BH),
                       dim3(Cfg4<D>::threads), 0, stream, (const T*)q, (const T*)k, (const T*)v,
                       (T*)o, lse, BH, S, nqt, c, ev);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

template <typename T, int D, int THR, bool DIAG>
static int launch_c(int causal, const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int S, float scale, hipStream_t st, unsigned long long* ev,
                    int variant) {
  return causal
             ? launch_one<T, D, true, THR, DIAG>(q, k, v, o, lse, B, H, S, scale, st, ev, variant)
             : launch_one<T, D, false, THR, DIAG>(q, k, v, o, lse, B, H, S, scale, st, ev, variant);
}

template <typename T, int THR, bool DIAG>
static int launch_d(int D, int causal, const void* q, const void* k, const void* v, void* o,
                    float* lse, int B, int H, int S, float scale, hipStream_t st,
                    unsigned long long* ev, int variant) {
  return D == 64 ? launch_c<T, 64, THR, DIAG>(causal, q, k, v, o, lse, B, H, S, scale, st, ev,
                                              variant)
                 : launch_c<T, 128, THR, DIAG>(causal, q, k, v, o, lse, B, H, S, scale, st, ev,
                                               variant);
}

static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Host-side validation; touches no HIP API.
static int validate(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int H, int S, int D, int causal, float scale, int dtype, bool* empty) {
  *empty = false;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (B < 0 || H < 0 || S < 0) return FA_ERR_DIM;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  if ((long long)B * H * S == 0) {
    *empty = true;
    return FA_OK;
  }
  if ((long long)S * D * 2 >= (1LL << 31)) return FA_ERR_DIM;  // 32-bit buffer offsets
  const long long rows = (long long)B * H * S;
  if (rows * D > (1LL << 40)) return FA_ERR_DIM;
  if ((long long)B * H * num_q_tiles(S, Cfg4<64>::BM) >= (1LL << 31)) return FA_ERR_DIM;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  const uintptr_t al = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse;
  if (al & 15) return FA_ERR_ALIGN;
  const size_t nt = (size_t)rows * D * 2, nl = (size_t)rows * 4;
  if (overlaps(o, nt, q, nt) || overlaps(o, nt, k, nt) || overlaps(o, nt, v, nt) ||
      overlaps(lse, nl, q, nt) || overlaps(lse, nl, k, nt) || overlaps(lse, nl, v, nt) ||
      overlaps(lse, nl, o, nt))
    return FA_ERR_ALIAS;
  return FA_OK;
}

}  // namespace fa

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int S,
           int D, int causal, float scale, hipStream_t stream, int dtype) {
  bool empty;
  const int st = fa::validate(q, k, v, o, lse, B, H, S, D, causal, scale, dtype, &empty);
  if (st != FA_OK || empty) return st;
  return dtype == FA_BF16
             ? fa::launch_d<__bf16, 8, false>(D, causal, q, k, v, o, lse, B, H, S, scale, stream,
                                              nullptr, fa::kAuto)
             : fa::launch_d<_Float16, 8, false>(D, causal, q, k, v, o, lse, B, H, S, scale,
                                                stream, nullptr, fa::kAuto);
}

int fa_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int S, int D, int causal, float scale, hipStream_t stream) {
  return fa_fwd(q, k, v, o, lse, B, H, S, D, causal, scale, stream, FA_F16);
}

int fa_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int S, int D, int causal, float scale, hipStream_t stream) {
  return fa_fwd(q, k, v, o, lse, B, H, S, D, causal, scale, stream, FA_BF16);
}

int fa_fwd_diag(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int S, int D, int causal, float scale, hipStream_t stream, int dtype,
                int threshold_log2, int variant, unsigned long long* rescale_events) {
  bool empty;
  const int st = fa::validate(q, k, v, o, lse, B, H, S, D, causal, scale, dtype, &empty);
  if (st != FA_OK) return st;
  if (threshold_log2 != 0 && threshold_log2 != 8) return FA_ERR_ARG;
  if (variant < fa::kAuto || variant > fa::kTwoBlock) return FA_ERR_ARG;
  if (!rescale_events) return FA_ERR_NULL;
  if (((uintptr_t)rescale_events & 7) != 0) return FA_ERR_ALIGN;
  if (empty) return FA_OK;
  const bool bf = dtype == FA_BF16;
  if (threshold_log2 == 8)
    return bf ? fa::launch_d<__bf16, 8, true>(D, causal, q, k, v, o, lse, B, H, S, scale, stream,
                                              rescale_events, variant)
              : fa::launch_d<_Float16, 8, true>(D, causal, q, k, v, o, lse, B, H, S, scale,
                                                stream, rescale_events, variant);
  return bf ? fa::launch_d<__bf16, 0, true>(D, causal, q, k, v, o, lse, B, H, S, scale, stream,
                                            rescale_events, variant)
            : fa::launch_d<_Float16, 0, true>(D, causal, q, k, v, o, lse, B, H, S, scale, stream,
                                              rescale_events, variant);
}

int fa_fwd_tile(int D, int B, int H, int S, int* block_m, int* block_n, int* threads,
                long long* work_groups) {
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  const int BH = (B < 0 || H < 0) ? 0 : B * H;
  const int SS = S < 0 ? 0 : S;
  const bool pp = D == 64 ? fa::use_pingpong<64>(BH, SS, fa::kAuto)
                          : fa::use_pingpong<128>(BH, SS, fa::kAuto);
  const int bm = pp ? 256 : 128;
  if (block_m) *block_m = bm;
  if (block_n) *block_n = pp ? (D == 64 ? fa::Cfg8<64>::BN : fa::Cfg8<128>::BN) : 64;
  if (threads) *threads = pp ? 512 : 256;
  if (work_groups) *work_groups = (long long)BH * fa::num_q_tiles(SS, bm);
  return FA_OK;
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_DIM: return "B, H or S is negative or the sizes exceed the supported limits";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension (D must be 64 or 128) or dtype";
    case FA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case FA_ERR_SCALE: return "scale must be finite and > 0";
    case FA_ERR_ALIAS: return "o or lse overlaps another buffer";
    case FA_ERR_HIP: return "the HIP runtime rejected the kernel launch";
    case FA_ERR_ARG: return "causal must be 0 or 1 (or a diagnostic argument is invalid)";
    default: return "unknown status";
  }
}

int fa_version(void) { return 200; }

}  // extern "C"
