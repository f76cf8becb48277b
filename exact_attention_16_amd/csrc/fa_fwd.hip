// Fused attention forward for AMD Instinct MI355X (gfx950, CDNA4).
//
// One work-group = 4 waves = one Q tile of 128 query rows of one (batch,
// head); each wave owns 32 query rows for the whole kernel, with its Q rows
// held in registers as MFMA operands. K and V stream through LDS in tiles of
// 64 keys, two LDS buffers each.
//
// Data movement: K and V tiles go from HBM to LDS by buffer loads with the
// LDS bit (direct DMA, 16 bytes per lane; no staging registers, no VALU),
// whose range check zero-fills rows past the end of the sequence. K is read
// back as 16-byte S^T operand fragments (no transpose); V^T operand
// fragments come from the row-major V tile through ds_read_b64_tr_b16,
// which transposes in the LDS crossbar. Both tiles are XOR-swizzled per row
// so that the operand reads are free of bank conflicts.
//
// Per KV tile j, each wave runs a three-stage register pipeline in one
// scheduling block, so that the matrix cores and the vector ALU overlap:
//   S(j+1) = K(j+1) Q^T      (MFMA, v_mfma_f32_32x32x16)
//   O^T   += V(j-1)^T P(j-1)^T (MFMA)
//   softmax(S(j)) -> P(j)    (VALU: max, exp2, sum, convert)
// followed, only when some row's running max moved, by the O rescale.
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
// Method sources: exact attention softmax(QK^T/sqrt(d)+mask)V with a
// lower-triangle causal mask (xdnf.cn, "CUDA手写masked multi-head attention
// 性能优化实战", 3.1); tiling with running max/sum, v2 loop order, deferred
// normalisation and the (Q tile, head) grid (hotdry.top, "FlashAttention的
// Triton性能考古学", "核心算法回顾" and "FlashAttention v2"); the conditional
// rescale with a lag of 8 and p in (0, 256], the warp-vote skip of the
// rescale, the rescale done by the softmax workers themselves, and issuing
// the next tile's Q.K^T ahead of the current P.V (hjcheng0602.cn, "Flash
// Attention CUDA Kernel 优化 ... G6", V39, V41 and V44).
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
__device__ __forceinline__ float max_xor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
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

template <int D> struct Pipe { static constexpr bool three = D == 64; };

template <typename T, int D, bool CAUSAL, int THR, bool DIAG>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
              T* __restrict__ O, float* __restrict__ LSE, int BH, int S, int nqt, float c,
              unsigned long long* __restrict__ events) {
  using TL = Tile<D>;
  constexpr bool P3 = Pipe<D>::three;
  // V^T operand: two transposed 8-byte reads (keys +0..3 and +4..7)
  auto lds_tr_pair = [](const lds_char* p, uint32_t second) -> u32x4 {
    const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + second));
    const u32x2 x = __builtin_bit_cast(u32x2, x0), y = __builtin_bit_cast(u32x2, x1);
    return (u32x4){x[0], x[1], y[0], y[1]};
  };
  constexpr int BN = TL::BN;
  constexpr int NKB = BN / 32;   // 32-key blocks per KV tile
  constexpr int NDC = D / 16;    // Q.K^T contraction steps (16 d each)
  constexpr int NDB = D / 32;    // 32-row d blocks of O^T
  constexpr int NKC = BN / 16;   // P.V contraction steps (16 keys each)
  constexpr int DPW = TL::dmaPerWave;
  constexpr uint32_t RB = TL::rowBytes;
  __shared__ __attribute__((aligned(1024))) char ks0[TL::bytes];
  __shared__ __attribute__((aligned(1024))) char ks1[TL::bytes];
  __shared__ __attribute__((aligned(1024))) char vs0[TL::bytes];
  __shared__ __attribute__((aligned(1024))) char vs1[TL::bytes];
  lds_char* const lk0 = (lds_char*)ks0;
  lds_char* const lk1 = (lds_char*)ks1;
  lds_char* const lv0 = (lds_char*)vs0;
  lds_char* const lv1 = (lds_char*)vs1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i32 = lane & 31;
  const int hh = lane >> 5;

  int qt, bh;
  block_to_tile(blockIdx.x, BH, nqt, CAUSAL, &qt, &bh);
  const size_t head = (size_t)bh * (size_t)S * D;
  const T* Kh = K + head;
  const T* Vh = V + head;
  const uint32_t head_bytes = (uint32_t)S * RB;
  const auto rq = FA_RSRC(Q + head, head_bytes);
  const auto ro = FA_RSRC(O + head, head_bytes);
  const auto rl = FA_RSRC(LSE + (size_t)bh * S, (uint32_t)S * 4u);

  const int q0w = qt * kBM + wave * kRowsPerWave;  // first row of this wave
  const int qrow = q0w + i32;                      // this lane's row
  const bool wave_live = q0w < S;
  const int ntiles = (tile_kv_end(qt, S, CAUSAL) + BN - 1) / BN;
  const int nw = wave_live ? (wave_kv_end(q0w, S, CAUSAL) + BN - 1) / BN : 0;

  // Q operand fragments (rows past S read as zeros)
  u32x4 qf[NDC];
#pragma unroll
  for (int j = 0; j < NDC; ++j)
    qf[j] = __builtin_amdgcn_raw_buffer_load_b128(rq, q_frag_off<D>(qrow, j, hh), 0, 0);

  // per-lane LDS / DMA base offsets; the rest are XOR / immediate offsets
  const uint32_t koff0 = k_read_off<D>(0, 0, lane);
  const uint32_t voff0 = v_tr_off<D>(0, 0, 0, lane);
  const uint32_t kdo0 = dma_src_k<D>(wave, 0, lane);
  const uint32_t vdo0 = dma_src_v<D>(wave, 0, lane);

  f32x16 o[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j) o[j] = (f32x16){};
  float b = -INFINITY;  // running base, log2 units (lags the true max by <= THR)
  float lsum = 0.f;     // this lane's partial row sum (its k-half of the keys)
  unsigned n_events = 0;

  // ---- building blocks --------------------------------------------------
  auto dma_k = [&](lds_char* dst, int t) {
    const int kv0 = t * BN;
    const auto r = FA_RSRC(Kh + (size_t)kv0 * D, (uint32_t)(S - kv0) * RB);
#pragma unroll
    for (int i = 0; i < DPW; ++i)
    {
      // (the LDS pointer goes through a local: written inline as the builtin's
      // argument, the host compilation pass drops the kernel launch stubs)
      lds_char* const lp = dst + dma_lds_k<D>(wave, i);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lp, 16, kdo0 + i * kDmaStrideK, 0, 0, 0);
    }
  };
  auto dma_v = [&](lds_char* dst, int t) {
    const int kv0 = t * BN;
    const auto r = FA_RSRC(Vh + (size_t)kv0 * D, (uint32_t)(S - kv0) * RB);
#pragma unroll
    for (int i = 0; i < DPW; ++i)
    {
      // (the LDS pointer goes through a local: written inline as the builtin's
      // argument, the host compilation pass drops the kernel launch stubs)
      lds_char* const lp = dst + dma_lds_v<D>(wave, i);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lp, 16, vdo0 + i * kDmaStrideV, 0, 0, 0);
    }
  };
  auto qk = [&](f32x16 (&s)[NKB], const lds_char* kt) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = (f32x16){};
#pragma unroll
    for (int j = 0; j < NDC; ++j) {
      const lds_char* base = kt + (koff0 ^ (uint32_t)(j << 5));
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        s[kb] = Ops<T>::mfma(lds16(base + kb * 32 * RB), qf[j], s[kb]);
    }
  };
  auto pv = [&](const u32x4 (&p)[NKC], const lds_char* vt) {
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
      for (int jd = 0; jd < NDB; ++jd)
        o[jd] = Ops<T>::mfma(lds_tr_pair(vt + (voff0 ^ (uint32_t)(jd << 6)) + kc * 16 * RB, 4 * RB),
                             p[kc], o[jd]);
  };
  auto mask = [&](f32x16 (&s)[NKB], int kv0) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 32 * kb + acc_key32(r, hh);
        const bool vis = key < S && (!CAUSAL || key <= qrow);
        s[kb][r] = vis ? s[kb][r] : -INFINITY;
      }
  };
  // running max with lag, p = 2^(s*c - b), row sum, P packed; returns history
  auto softmax = [&](f32x16 (&s)[NKB], u32x4 (&p)[NKC]) -> float {
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = max_xor32(mx);
    const float cand = fmaxf(b, mx * c);
    const bool rebase = cand > b + (float)THR;
    const float hist = rebase ? __builtin_amdgcn_exp2f(b - cand) : 1.f;  // 0 on the first tile
    b = rebase ? cand : b;
    const float nb = (b == -INFINITY) ? 0.f : -b;  // fully hidden row: p = 0
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float e[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          e[x] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * g + x], c, nb));
          ls += e[x];
        }
        p[2 * kb + g] = (u32x4){Ops<T>::pack2(e[0], e[1]), Ops<T>::pack2(e[2], e[3]),
                                Ops<T>::pack2(e[4], e[5]), Ops<T>::pack2(e[6], e[7])};
      }
    lsum = lsum * hist + ls;
    // keep P(j) and the row sum in the block of the MFMAs they overlap,
    // instead of letting them sink past the rescale branch
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) asm volatile("" : "+v"(p[kc]));
    asm volatile("" : "+v"(lsum));
    return hist;
  };
  // rare path: some row of the wave moved its base -> rescale O
  auto rescale = [&](int j, float hist) {
    if (DIAG && j >= 1 && hh == 0 && qrow < S && hist < 1.f) ++n_events;
    if (j >= 1 && __builtin_amdgcn_ballot_w64(hist < 1.f) != 0) {
#pragma unroll
      for (int jd = 0; jd < NDB; ++jd) o[jd] *= hist;
    }
  };

  f32x16 sA[NKB], sB[NKB];  // S(j) lives in sA for even j, sB for odd j
  u32x4 pA[NKC], pB[NKC];   // P(j) likewise (only pA is used with two stages)
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) pB[kc] = (u32x4){};  // P(-1) = 0

  // ---- prologue: K(0), K(1) (and V(0) with two stages) in LDS; S(0) --------
  // With three stages iteration 0 runs the steady-state block with P(-1) = 0
  // against V buffer 1, so that buffer must hold finite values (0 * NaN
  // would poison O).
  dma_k(lk0, 0);
  if (ntiles > 1) dma_k(lk1, 1);
  if constexpr (P3) {
#pragma unroll
    for (int i = 0; i < TL::bytes / (16 * kThreads); ++i)
      *(__attribute__((address_space(3))) u32x4*)(lv1 + 16 * (tid + i * kThreads)) = (u32x4){};
  } else {
    dma_v(lv0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (nw > 0) qk(sA, lk0);
  __syncthreads();  // ks0 is refilled with K(2) in iteration 0

  // ---- iteration j (PH = j % 2). DMA first (K(j+2); V(j) with three stages,
  // V(j+1) with two). A wave that still has tile j then runs one scheduling
  // block: S(j+1) = QK and softmax(S(j)) -> P(j), plus P(j-1).V(j-1) with
  // three stages; with two stages the rescale and P(j).V(j) follow. At the
  // wave's last tile the S(j+1) it computes is not used. With three stages
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
      if (j < ntiles) dma_v(v_cur, j);
    } else {
      if (j + 1 < ntiles) dma_v(v_oth, j + 1);
    }
    if (j + 2 < ntiles) dma_k(k_dma, j + 2);
    __builtin_amdgcn_sched_barrier(0);

    if (j < nw) {
      const int kv0 = j * BN;
      if ((CAUSAL && kv0 + BN - 1 > q0w) || kv0 + BN > S) mask(scur, kv0);
      qk(snext, k_next);
      if constexpr (P3) pv(pprev, v_oth);
      const float hist = softmax(scur, pcur);
      rescale(j, hist);
      if constexpr (!P3) pv(pcur, v_cur);
    } else if (P3 && j == nw) {
      pv(pprev, v_oth);
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

  // ---- epilogue: normalise once, write O and lse ---------------------------
  // Rows past S are dropped by the buffer range check.
  const float ltot = sum_xor32(lsum);
  if (wave_live) {
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
        // accumulator element r0+e of lane (i32, hh) is d = 32jd + 16g + 8hh + e
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

// ------------------------------------------------------------------- host

template <typename T, int D, bool CAUSAL, int THR, bool DIAG>
static int launch_one(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int S, float scale, hipStream_t stream, unsigned long long* ev) {
  const int BH = B * H;
  const int nqt = num_q_tiles(S);
  const unsigned grid = (unsigned)nqt * (unsigned)BH;
  hipLaunchKernelGGL((fa_fwd_kernel<T, D, CAUSAL, THR, DIAG>), dim3(grid), dim3(kThreads), 0,
                     stream, (const T*)q, (const T*)k, (const T*)v, (T*)o, lse, BH, S, nqt,
                     scale * kLog2e, ev);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

template <typename T, int D, int THR, bool DIAG>
static int launch_c(int causal, const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int S, float scale, hipStream_t st, unsigned long long* ev) {
  return causal ? launch_one<T, D, true, THR, DIAG>(q, k, v, o, lse, B, H, S, scale, st, ev)
                : launch_one<T, D, false, THR, DIAG>(q, k, v, o, lse, B, H, S, scale, st, ev);
}

template <typename T, int THR, bool DIAG>
static int launch_d(int D, int causal, const void* q, const void* k, const void* v, void* o,
                    float* lse, int B, int H, int S, float scale, hipStream_t st,
                    unsigned long long* ev) {
  return D == 64 ? launch_c<T, 64, THR, DIAG>(causal, q, k, v, o, lse, B, H, S, scale, st, ev)
                 : launch_c<T, 128, THR, DIAG>(causal, q, k, v, o, lse, B, H, S, scale, st, ev);
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
  if ((long long)B * H * num_q_tiles(S) >= (1LL << 31)) return FA_ERR_DIM;
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
                                              nullptr)
             : fa::launch_d<_Float16, 8, false>(D, causal, q, k, v, o, lse, B, H, S, scale,
                                                stream, nullptr);
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
                int threshold_log2, unsigned long long* rescale_events) {
  bool empty;
  const int st = fa::validate(q, k, v, o, lse, B, H, S, D, causal, scale, dtype, &empty);
  if (st != FA_OK) return st;
  if (threshold_log2 != 0 && threshold_log2 != 8) return FA_ERR_ARG;
  if (!rescale_events) return FA_ERR_NULL;
  if (((uintptr_t)rescale_events & 7) != 0) return FA_ERR_ALIGN;
  if (empty) return FA_OK;
  const bool bf = dtype == FA_BF16;
  if (threshold_log2 == 8)
    return bf ? fa::launch_d<__bf16, 8, true>(D, causal, q, k, v, o, lse, B, H, S, scale, stream,
                                              rescale_events)
              : fa::launch_d<_Float16, 8, true>(D, causal, q, k, v, o, lse, B, H, S, scale,
                                                stream, rescale_events);
  return bf ? fa::launch_d<__bf16, 0, true>(D, causal, q, k, v, o, lse, B, H, S, scale, stream,
                                            rescale_events)
            : fa::launch_d<_Float16, 0, true>(D, causal, q, k, v, o, lse, B, H, S, scale, stream,
                                              rescale_events);
}

int fa_fwd_tile(int D, int B, int H, int S, int* block_m, int* block_n, int* threads,
                long long* work_groups) {
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  if (block_m) *block_m = fa::kBM;
  if (block_n) *block_n = fa::kBN;
  if (threads) *threads = fa::kThreads;
  if (work_groups)
    *work_groups = (B < 0 || H < 0 || S < 0) ? 0 : (long long)B * H * fa::num_q_tiles(S);
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

int fa_version(void) { return 100; }

}  // extern "C"
