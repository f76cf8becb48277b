// Fused attention forward on 8-bit float inputs (E4M3, one descale per
// tensor) for MI355X (gfx950): Q, K and V are E4M3 codes, O is bf16 and the
// row logsumexp fp32.
//
// Work-group: eight waves of 32 query rows (fa_interleave.h), each
// overlapping the softmax of KV tile j with the MFMAs of tile j+1's scores,
// K/V in three LDS stages filled by direct DMA, 64-key tiles (128 at
// D = 64). Both products
// use the 8-bit matrix instruction v_mfma_f32_32x32x64_f8f6f4:
//   S^T = K Q^T   one 64-deep step per 32-key block per 64 of D
//   O^T += V^T P^T  one 64-key chunk per MFMA, P rounded to E4M3
// The operand layouts (fa_layout8.h) put each lane's 32 S values of a 64-key
// chunk in key order, so P packs straight into the P.V operand
// (v_cvt_pk_fp8_f32, round to nearest even); V^T comes from the row-major V
// tile through ds_read_b64_tr_b8.
//
// Scaling: the Q and K descales fold into the base-2 logit multiplier
// c = scale * dq * dk * log2(e); the V descale multiplies O once at the end.
// The running base lags the row max by at most THR = 2 binades and each
// probability is multiplied by 2^(8 - THR) before rounding, so the rounded
// values lie in (0, 256] (E4M3 reaches 448) and every probability at least
// 2^-14 of the row max stays a normal E4M3 number. Row sums use the
// unrounded fp32 values; the factor cancels in O and is taken out of lse.
//
// Method: exact attention with running max and sum and deferred
// normalisation as in the 16-bit kernels (hotdry.top, "FlashAttention的
// Triton性能考古学", sections "核心算法回顾" and "FlashAttention v2"); the
// 8-bit path is the FP8 support the same page lists for newer GPUs (section
// "架构感知优化策略").
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/fa_fwd.h"
#include "fa_device.h"
#include "fa_layout8.h"
#include "fa_interleave.h"
#include "fa_pingpong.h"

namespace fa {

__device__ __forceinline__ f32x16 mfma_f8(u32x8 a, u32x8 b, f32x16 c) {
  // format fields 0 (E4M3 for both operands), no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a),
                                                         __builtin_bit_cast(i32x8, b), c, 0, 0,
                                                         0, 0, 0, 0);
}

typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// one transposed 8-byte read (8 keys x one d per lane)
__device__ __forceinline__ u32x2 lds_tr8(const lds_char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p));
}

// four fp32 -> four E4M3 bytes (round to nearest even), lowest byte first
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  const uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// One wave's 32 query rows of the 8-bit kernel (the interface il_body and
// pp_body use).
template <bool CAUSAL, int THR, class C_ = CfgF8>
struct Wave8 : RowState<C_, CAUSAL, THR> {
  using Rows = RowState<C_, CAUSAL, THR>;
  using Rows::lane, Rows::wave, Rows::hh, Rows::q0w, Rows::qrow, Rows::qt, Rows::Lq, Rows::Lk,
      Rows::off, Rows::c, Rows::b, Rows::lsum;
  using C = C_;
  using Config = C_;
  static constexpr int D = C::D;
  static constexpr int BN = C::BN;
  static constexpr int NKB = BN / 32;  // 32-key MFMA blocks of S per tile
  static constexpr int NCH = BN / 64;  // 64-key chunks (P.V contraction steps)
  static constexpr int NDJ = D / 64;   // S contraction steps (64 d each)
  static constexpr int NDB = D / 32;   // 32-row d blocks of O^T
  static constexpr int DPW = C::dmaPerWave;
  static constexpr uint32_t RB = C::rowBytes;
  static constexpr int PSH = 8 - THR;  // probabilities are rounded times 2^PSH
  using STile = f32x16[NKB];
  using PTile = u32x8[NCH];

  float vscale;
  const char* Kh;
  const char* Vh;
  char* Oh;
  float* Lh;
  uint32_t rsk, rsv, rso;
  uint32_t dsk, dsv;
  uint32_t koff0, voff0, kdo0, vdo0;
  u32x8 qf[NDJ];
  f32x16 o[NDB];

  __device__ __forceinline__ bool init(const Problem& P, int id = -1) {
    HeadRows hr;
    if (!this->locate(P, 0, &hr, id < 0 ? (int)blockIdx.x : id)) return false;
    vscale = P.vscale;
    // one-byte Q, K, V elements; two-byte O elements
    Kh = (const char*)P.k + hr.k0;
    Vh = (const char*)P.v + hr.v0;
    Oh = (char*)P.o + hr.o0 * 2;
    Lh = P.lse + hr.l0;
    rsk = (uint32_t)P.ks;
    rsv = (uint32_t)P.vs;
    rso = (uint32_t)P.os * 2u;
    dsk = (uint32_t)C::dmaRowsK * rsk;
    dsv = (uint32_t)C::dmaRowsV * rsv;
    const uint32_t rsq = (uint32_t)P.qs;
    const auto rq = FA_RSRC((const char*)P.q + hr.q0, (uint32_t)Lq * rsq);
#pragma unroll
    for (int j = 0; j < NDJ; ++j) {
      const u32x4 x0 = __builtin_amdgcn_raw_buffer_load_b128(rq, q8_frag_off(qrow, j, hh, 0, rsq), 0, 0);
      const u32x4 x1 = __builtin_amdgcn_raw_buffer_load_b128(rq, q8_frag_off(qrow, j, hh, 1, rsq), 0, 0);
      qf[j] = (u32x8){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    }
    koff0 = k8_read_off<D>(0, 0, 0, lane);
    voff0 = v8_tr_off<D>(0, 0, 0, lane);
    kdo0 = dma_src_k8<C>(wave, 0, lane, rsk);
    vdo0 = dma_src_v8<C>(wave, 0, lane, rsv);
#pragma unroll
    for (int j = 0; j < NDB; ++j) o[j] = (f32x16){};
    this->reset_softmax();
    return true;
  }

  __device__ __forceinline__ void dma_k(lds_char* dst, int t, int limit = 0x7fffffff) const {
    const int kv0 = t * BN;
    const uint32_t bytes = dma_bytes((t < limit) & (kv0 < Lk), (uint32_t)(Lk - kv0) * rsk);
    const auto r = FA_RSRC(Kh + (size_t)kv0 * rsk, bytes);
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      lds_char* const lp = dst + dma_lds_k<C>(wave, i);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lp, 16, kdo0 + i * dsk, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void dma_v(lds_char* dst, int t, int limit = 0x7fffffff) const {
    const int kv0 = t * BN;
    const uint32_t bytes = dma_bytes((t < limit) & (kv0 < Lk), (uint32_t)(Lk - kv0) * rsv);
    const auto r = FA_RSRC(Vh + (size_t)kv0 * rsv, bytes);
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      lds_char* const lp = dst + dma_lds_v<C>(wave, i);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lp, 16, vdo0 + i * dsv, 0, 0, 0);
    }
  }

  // S^T = K Q^T for the tile at kt
  __device__ __forceinline__ void qk(f32x16 (&s)[NKB], const lds_char* kt) const {
#pragma unroll
    for (int j = 0; j < NDJ; ++j) {
      const lds_char* b0 = kt + (koff0 ^ (uint32_t)(j << 6));
      const lds_char* b1 = kt + (koff0 ^ (uint32_t)(j << 6 | 16));
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const uint32_t rows = k8_block_rows(kb) * RB;
        const u32x4 x0 = lds16(b0 + rows), x1 = lds16(b1 + rows);
        const u32x8 a = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        s[kb] = mfma_f8(a, qf[j], j == 0 ? (f32x16){} : s[kb]);
      }
    }
  }
  // O^T += V^T P^T for the tile at vt
  __device__ __forceinline__ void pv(const u32x8 (&p)[NCH], const lds_char* vt) {
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
      for (int jd = 0; jd < NDB; ++jd) {
        const lds_char* base = vt + (voff0 ^ (uint32_t)(jd << 5)) + ch * 64 * RB;
        const u32x2 t0 = lds_tr8(base), t1 = lds_tr8(base + 8 * RB);
        const u32x2 t2 = lds_tr8(base + 16 * RB), t3 = lds_tr8(base + 24 * RB);
        const u32x8 a = {t0[0], t0[1], t1[0], t1[1], t2[0], t2[1], t3[0], t3[1]};
        o[jd] = mfma_f8(a, p[ch], o[jd]);
      }
  }
  // operands read ahead of their MFMA: four transposed reads per P.V MFMA,
  // two reads per S MFMA, two MFMAs ahead
  static __device__ __forceinline__ void pv_schedule() { read_ahead<8, NCH * NDB, 4>(); }
  static __device__ __forceinline__ void qk_schedule() { read_ahead<4, NDJ * NKB, 2>(); }
  // softmax of one tile (about 4 vector instructions per score, 2 BN / 64
  // scores per lane) spread over the next tile's S MFMAs
  static __device__ __forceinline__ void il_schedule() {
    mix<4, NDJ * NKB, 2, (4 * BN / 2) / (NDJ * NKB)>();
  }

  __device__ __forceinline__ void mask(f32x16 (&s)[NKB], int kv0) const {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + acc_key8(kb, r, hh);
        const bool vis = key < Lk && (!CAUSAL || key <= qrow + off);
        s[kb][r] = vis ? s[kb][r] : -INFINITY;
      }
  }
  // p = 2^(s*c - b + PSH) in (0, 256]; row sum of the unrounded p; P as
  // E4M3 bytes in key order: byte 16*(kb%2) + r of chunk kb/2 is element r
  // of block kb
  __device__ __forceinline__ void softmax_exp(const f32x16 (&s)[NKB], u32x8 (&p)[NCH]) {
    const float nb = (b == -INFINITY) ? 0.f : (float)PSH - b;
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float e[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          e[x] = __builtin_amdgcn_exp2f(fmaf(s[kb][4 * g + x], c, nb));
          ls[x] += e[x];
        }
        p[kb >> 1][4 * (kb & 1) + g] = pack4_fp8(e[0], e[1], e[2], e[3]);
      }
    lsum += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  }
  __device__ __forceinline__ void rescale(int j, float hist) {
    if (j >= 1 && __builtin_amdgcn_ballot_w64(hist < 1.f) != 0) {
#pragma unroll
      for (int jd = 0; jd < NDB; ++jd) o[jd] *= hist;
    }
  }
  __device__ __forceinline__ void softmax_tile(f32x16 (&s)[NKB], u32x8 (&p)[NCH], int j) {
    const int kv0 = j * BN;
    if (this->needs_mask(kv0)) mask(s, kv0);
    const float hist = this->softmax_max(s);
    rescale(j, hist);
    softmax_exp(s, p);
  }

  // normalise (times the V descale), write O as bf16 and lse; a row that
  // sees no key gets O = 0 and lse = -inf
  __device__ __forceinline__ void epilogue(unsigned long long*) {
    const float ltot = sum_xor32(lsum);
    if (q0w >= Lq) return;
    const auto ro = FA_RSRC(Oh, (uint32_t)Lq * rso);
    const auto rl = FA_RSRC(Lh, (uint32_t)Lq * 4u);
    const float inv = ltot > 0.f ? vscale / ltot : 0.f;
    // As in the 16-bit wave's store_rows: everything packed first, and no
    // store's data registers written after it.
    static_assert(NDB == 2 || NDB == 4, "head dimension 64 or 128");
    u32x2 w[NDB][4];
#pragma unroll
    for (int jd = 0; jd < NDB; ++jd)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x16& a = o[jd];
        w[jd][u] = (u32x2){pack2_bf16(a[4 * u + 0] * inv, a[4 * u + 1] * inv),
                           pack2_bf16(a[4 * u + 2] * inv, a[4 * u + 3] * inv)};
      }
    const float l2 =
        ltot > 0.f ? (b - (float)PSH + __builtin_amdgcn_logf(ltot)) * kLn2 : -INFINITY;
    const uint32_t lbits = __builtin_bit_cast(uint32_t, l2);
    if (hh == 0) __builtin_amdgcn_raw_buffer_store_b32(lbits, rl, (uint32_t)qrow * 4u, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int jd = 0; jd < NDB; ++jd)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        __builtin_amdgcn_raw_buffer_store_b64(w[jd][u], ro, o8_frag_off(qrow, jd, u, hh, rso), 0, 0);
    if constexpr (NDB == 4)
      asm volatile("" ::"v"(w[0][0]), "v"(w[0][1]), "v"(w[0][2]), "v"(w[0][3]), "v"(w[1][0]),
                   "v"(w[1][1]), "v"(w[1][2]), "v"(w[1][3]), "v"(w[2][0]), "v"(w[2][1]),
                   "v"(w[2][2]), "v"(w[2][3]), "v"(w[3][0]), "v"(w[3][1]), "v"(w[3][2]),
                   "v"(w[3][3]), "v"(lbits));
    else
      asm volatile("" ::"v"(w[0][0]), "v"(w[0][1]), "v"(w[0][2]), "v"(w[0][3]), "v"(w[1][0]),
                   "v"(w[1][1]), "v"(w[1][2]), "v"(w[1][3]), "v"(lbits));
  }
};

// 64-key tiles at D = 128; at D = 64 a 64-key tile would be less than one
// 1-KiB DMA issue per wave, so 128-key tiles
template <int D> using CfgF8il = typename std::conditional<D == 64, CfgF8h, CfgF8i>::type;

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd_il8(const Problem P) {
  il_body<Wave8<CAUSAL, 2, CfgF8il<D>>>(P);
}

// Launches the 8-bit kernel for a filled, validated Problem. (The same wave
// type also runs under the ping-pong body, pp_body<Wave8<CAUSAL, 2>> with
// 128-key tiles; on the long causal workload at D = 128 that took 5%
// longer.)
template <int D> static int launch_fp8_d(Problem P, int causal, hipStream_t stream) {
  P.nqt = num_q_tiles(P.Sq, CfgF8il<D>::BM);
  P.items = P.nqt * P.B * P.H;
  const dim3 grid((unsigned)P.items), block(CfgF8il<D>::threads);
  if (causal)
    hipLaunchKernelGGL((fa_fwd_il8<D, true>), grid, block, 0, stream, P);
  else
    hipLaunchKernelGGL((fa_fwd_il8<D, false>), grid, block, 0, stream, P);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int launch_fp8(Problem P, int D, int causal, hipStream_t stream) {
  return D == 64 ? launch_fp8_d<64>(P, causal, stream) : launch_fp8_d<128>(P, causal, stream);
}

}  // namespace fa
