// Fused attention forward for AMD Instinct MI355X (gfx950, CDNA4).
//
// One work-group = 4 waves = one Q tile of 128 query rows of one (batch,
// head); each wave owns 32 query rows for the whole kernel. Per KV tile:
//
//   1. K tile and V^T tile of the next KV tile are fetched from HBM into
//      registers (16-byte loads, consecutive lanes on consecutive bytes)
//      while the current tile is consumed from LDS (double buffer).
//   2. S^T = K Q^T on v_mfma_f32_32x32x16 (raw dot products in fp32; the
//      scale is folded into the exponent). Q stays in registers as MFMA
//      operands for the whole kernel; K rows are read from LDS as 16-byte
//      operand fragments, so K never needs a transpose.
//   3. Causal: tiles wholly above the diagonal are never visited, tiles
//      wholly below are not masked; only tiles that straddle the diagonal
//      (or the ragged end) compare indices.
//   4. Online softmax in base 2 with a lagging running max b: the tile max
//      is exchanged between the two lanes of a row with v_permlane32_swap;
//      b moves only when the candidate exceeds b + THR, and only then is the
//      O accumulator rescaled (wave-uniform branch on a ballot).
//      p = 2^(s*c - b) with c = scale*log2(e); row sums accumulate the
//      unrounded fp32 p.
//   5. O^T += V^T P^T on v_mfma_f32_32x32x16: P goes from the S accumulator
//      to the MFMA operand inside the lane; V^T fragments come from LDS.
//   6. Epilogue: one division per row, O rounded once to the 16-bit type,
//      lse = ln2 * (b + log2(l)).
//
// Method sources: exact attention softmax(QK^T/sqrt(d)+mask)V with a
// lower-triangle causal mask (xdnf.cn, "CUDA手写masked multi-head attention
// 性能优化实战", 3.1); tiling with running max/sum, v2 loop order, deferred
// normalisation and the (Q tile, head) grid (hotdry.top, "FlashAttention的
// Triton性能考古学", "核心算法回顾" and "FlashAttention v2"); the conditional
// rescale with a lag of 8 and p in (0, 256], the warp-vote skip of the
// rescale and the rescale done by the softmax workers themselves
// (hjcheng0602.cn, "Flash Attention CUDA Kernel 优化 ... G6", V41 and V44).
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
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

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

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }

template <typename T, int D, bool CAUSAL, int THR, bool DIAG>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
              T* __restrict__ O, float* __restrict__ LSE, int BH, int S, int nqt, float c,
              unsigned long long* __restrict__ events) {
  using L = Lds<D>;
  constexpr int BN = L::BN;
  constexpr int NKB = BN / 32;   // 32-key blocks per KV tile
  constexpr int NDC = D / 16;    // 16-wide d chunks (QK^T contraction steps)
  constexpr int NDB = D / 32;    // 32-row d blocks of O^T
  constexpr int NKC = BN / 16;   // 16-key chunks (P.V contraction steps)
  __shared__ __attribute__((aligned(1024))) char smem[L::totalBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i32 = lane & 31;
  const int hh = lane >> 5;

  int qt, bh;
  block_to_tile(blockIdx.x, BH, nqt, CAUSAL, &qt, &bh);
  const size_t head = (size_t)bh * (size_t)S * D;
  Q += head;
  K += head;
  V += head;
  O += head;
  LSE += (size_t)bh * S;

  const int q0w = qt * kBM + wave * kRowsPerWave;  // first row of this wave
  const int qrow = q0w + i32;                      // this lane's row
  const int qrow_c = qrow < S ? qrow : S - 1;
  const int ntiles = (tile_kv_end(qt, S, CAUSAL) + BN - 1) / BN;
  const int wkv_end = wave_kv_end(q0w, S, CAUSAL);
  const bool wave_live = q0w < S;

  // Q operand fragments: lane holds q[qrow, 16*j + 8*hh + 0..7]
  u32x4 qf[NDC];
#pragma unroll
  for (int j = 0; j < NDC; ++j) qf[j] = ld16(Q + q_frag_off<D>(qrow_c, j, hh));

  f32x16 o[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j) o[j] = (f32x16){};
  float b = -INFINITY;  // running base, log2 units (lags the true max by <= THR)
  float lsum = 0.f;     // this lane's partial row sum (its k-half of the keys)
  unsigned n_events = 0;

  u32x4 kreg[L::kChunksPerThread];
  u32x4 vreg[L::vUnitsPerThread][4];

  auto gload = [&](int t) {
    const int kv0 = t * BN;
#pragma unroll
    for (int n = 0; n < L::kChunksPerThread; ++n) {
      int key, ch;
      k_stage_map<D>(tid + n * kThreads, &key, &ch);
      kreg[n] = ld16(K + kv_chunk_off<D>(kv_row(kv0, key, S), ch));
    }
#pragma unroll
    for (int n = 0; n < L::vUnitsPerThread; ++n) {
      int kg, dc;
      v_stage_map<D>(tid + n * kThreads, &kg, &dc);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        vreg[n][q4] = ld16(V + kv_chunk_off<D>(kv_row(kv0, 4 * kg + q4, S), dc));
    }
  };
  auto swrite = [&](int stage) {
    char* sb = smem + stage * L::stageBytes;
#pragma unroll
    for (int n = 0; n < L::kChunksPerThread; ++n)
      *(u32x4*)(sb + k_write_off<D>(tid + n * kThreads)) = kreg[n];
    // V is written transposed: 4 keys of one d packed as 8 bytes.
#pragma unroll
    for (int n = 0; n < L::vUnitsPerThread; ++n) {
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t w0 = __builtin_amdgcn_perm(vreg[n][1][dd >> 1], vreg[n][0][dd >> 1], sel);
        const uint32_t w1 = __builtin_amdgcn_perm(vreg[n][3][dd >> 1], vreg[n][2][dd >> 1], sel);
        *(u32x2*)(sb + vt_write_off<D>(tid + n * kThreads, dd)) = (u32x2){w0, w1};
      }
    }
  };

  gload(0);
  swrite(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int stage = t & 1;
    const int kv0 = t * BN;
    if (t + 1 < ntiles) gload(t + 1);

    if (wave_live && kv0 < wkv_end) {
      const char* sb = smem + stage * L::stageBytes;

      // ---- S^T = K Q^T (raw dot products) --------------------------------
      f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = (f32x16){};
#pragma unroll
        for (int j = 0; j < NDC; ++j)
          s[kb] = Ops<T>::mfma(ld16(sb + k_read_off<D>(kb, j, lane)), qf[j], s[kb]);
      }

      // ---- mask: only tiles crossing the diagonal or the ragged end ------
      const bool need_mask = (CAUSAL && kv0 + BN - 1 > q0w) || (kv0 + BN > S);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * kb + acc_key32(r, hh);
            const bool vis = key < S && (!CAUSAL || key <= qrow);
            s[kb][r] = vis ? s[kb][r] : -INFINITY;
          }
      }

      // ---- running max with lag (conditional rescale) ---------------------
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = max_xor32(mx);
      const float cand = fmaxf(b, mx * c);
      float hist = 1.f;
      if (cand > b + (float)THR) {
        hist = __builtin_amdgcn_exp2f(b - cand);  // 2^(b_old - b_new); 0 on the first tile
        b = cand;
      }
      if (DIAG && t > 0 && hh == 0 && qrow < S && hist < 1.f) ++n_events;
      // rare path: some row of the wave moved its base -> rescale O rows
      if (t > 0 && __builtin_amdgcn_ballot_w64(hist < 1.f) != 0) {
        lsum *= hist;
#pragma unroll
        for (int j = 0; j < NDB; ++j) o[j] *= hist;
      }
      const float nb = (b == -INFINITY) ? 0.f : -b;  // fully hidden row: p = 0

      // ---- p = 2^(s*c - b), row sum (fp32, unrounded), pack P -------------
      u32x4 pf[NKC];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * g + e], c, nb));
            lsum += p[e];
          }
          pf[2 * kb + g] = (u32x4){Ops<T>::pack2(p[0], p[1]), Ops<T>::pack2(p[2], p[3]),
                                   Ops<T>::pack2(p[4], p[5]), Ops<T>::pack2(p[6], p[7])};
        }

      // ---- O^T += V^T P^T -------------------------------------------------
#pragma unroll
      for (int j = 0; j < NDB; ++j)
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
          o[j] = Ops<T>::mfma(ld16(sb + vt_read_off<D>(j, kc, lane)), pf[kc], o[j]);
    }

    if (t + 1 < ntiles) swrite(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise once, write O and lse ---------------------------
  const float ltot = sum_xor32(lsum);
  if (wave_live && qrow < S) {
    const float inv = 1.f / ltot;
#pragma unroll
    for (int j = 0; j < NDB; ++j)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const f32x16& a = o[j];
        const int r0 = 8 * g;
        u32x4 w = {Ops<T>::pack2(a[r0 + 0] * inv, a[r0 + 1] * inv),
                   Ops<T>::pack2(a[r0 + 2] * inv, a[r0 + 3] * inv),
                   Ops<T>::pack2(a[r0 + 4] * inv, a[r0 + 5] * inv),
                   Ops<T>::pack2(a[r0 + 6] * inv, a[r0 + 7] * inv)};
        // accumulator element r0+e of lane (i32, hh) is d = 32j + 16g + 8hh + e
        *(u32x4*)(O + o_frag_off<D>(qrow, j, g, hh)) = w;
      }
    if (hh == 0) LSE[qrow] = (b + __builtin_amdgcn_logf(ltot)) * kLn2;
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
  if (S > (1 << 30)) return FA_ERR_DIM;
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
  if (block_n) *block_n = D == 64 ? fa::TileCfg<64>::BN : fa::TileCfg<128>::BN;
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
