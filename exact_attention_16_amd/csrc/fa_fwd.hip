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
// fa_fwd picks one of two kernels, which overlap the matrix cores and the
// vector ALU differently:
//  * fa_fwd_pp (eight waves, 256 query rows; work-group body in
//    fa_pingpong.h): the waves form two groups whose slots alternate between
//    an MFMA phase (P(j-1).V(j-1) and K(j).Q^T) and a softmax phase, offset
//    by one slot, so each SIMD always holds one multiplying and one
//    exponentiating wave; K/V use three LDS stages, issued two tiles ahead.
//  * fa_fwd_k4 (four waves, 128 query rows), for grids too small to fill the
//    chip with 256-row tiles: each wave overlaps the next tile's K.Q^T (and,
//    at D=64, the previous tile's P.V) with its own current softmax; two LDS
//    stages.
// fa_fwd_diag can also run fa_fwd_w2 (four waves of two 32-row blocks) and
// fa_fwd_il (eight waves, each interleaving its softmax with its next
// tile's MFMAs; fa_interleave.h). fa_fwd_kt runs the ping-pong body on a K
// given transposed ([D, S] per head), read like a V tile. The 8-bit kernel
// is in fa_fwd_fp8.hip.
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
#include "fa_device.h"
#include "fa_layout8.h"
#include "fa_interleave.h"
#include "fa_pingpong.h"

namespace fa {

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

// V^T operand: two transposed 8-byte reads (keys +0..3 and +4..7)
__device__ __forceinline__ u32x4 lds_tr_pair(const lds_char* p, uint32_t second) {
  const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + second));
  const u32x2 x = __builtin_bit_cast(u32x2, x0), y = __builtin_bit_cast(u32x2, x1);
  return (u32x4){x[0], x[1], y[0], y[1]};
}

// One wave's share of a work-group: its query rows, accumulators and the
// per-tile operations on them. KT: the caller passes K transposed, [D, S]
// per head (k's "row" stride is then the stride between d rows); a K tile
// in LDS is then D rows of BN keys, laid out and read like a V tile with
// the roles of rows and columns swapped (config CK below).
template <typename T, class C, bool CAUSAL, int THR, bool DIAG, bool KT = false>
struct Wave : RowState<C, CAUSAL, THR> {
  using Rows = RowState<C, CAUSAL, THR>;
  using Rows::lane, Rows::wave, Rows::hh, Rows::q0w, Rows::qrow, Rows::qt, Rows::Lq, Rows::Lk,
      Rows::off, Rows::c, Rows::b, Rows::lsum;
  static constexpr int D = C::D;
  static constexpr int BN = C::BN;
  static constexpr int NKB = BN / 32;  // 32-key blocks per KV tile
  static constexpr int NDC = D / 16;   // Q.K^T contraction steps (16 d each)
  static constexpr int NDB = D / 32;   // 32-row d blocks of O^T
  static constexpr int NKC = BN / 16;  // P.V contraction steps (16 keys each)
  static constexpr int DPW = C::dmaPerWave;
  static constexpr uint32_t RB = C::rowBytes;
  // a transposed K tile: D rows (d) of BN 16-bit keys, as a V tile of a
  // configuration with head dimension BN and BN' = D
  using CK = Cfg<BN, C::NW, D>;
  static constexpr uint32_t RBK = CK::rowBytes;
  static_assert(!KT || CK::dmaPerWave == DPW, "a transposed K tile is the same size");
  using Config = C;
  using STile = f32x16[NKB];  // S^T of one KV tile
  using PTile = u32x4[NKC];   // P of one KV tile as P.V operands

  const char* Kh;  // row 0 of this (sequence, head) in k, v, o, lse
  const char* Vh;
  char* Oh;
  float* Lh;
  uint32_t rsk, rsv, rso;  // row strides in bytes
  uint32_t dsk, dsv;       // source bytes between successive DMA issues
  uint32_t koff0, voff0, kdo0, vdo0;
  u32x4 qf[NDC];
  f32x16 o[NDB];
  unsigned n_events;

  // Sets up this wave's rows of the work-group's query tile (see
  // RowState::locate); false when the tile lies wholly past its sequence's
  // end. sub: which 32-row block of the wave's C::RPW rows this object holds
  __device__ __forceinline__ bool init(const Problem& P, int sub = 0, int id = -1) {
    HeadRows hr;
    if (!this->locate(P, sub, &hr, id < 0 ? (int)blockIdx.x : id)) return false;
    const long long q0 = hr.q0, k0 = hr.k0, v0 = hr.v0, o0 = hr.o0, l0 = hr.l0;
    Kh = (const char*)P.k + k0 * 2;
    Vh = (const char*)P.v + v0 * 2;
    Oh = (char*)P.o + o0 * 2;
    Lh = P.lse + l0;
    rsk = (uint32_t)P.ks * 2u;
    rsv = (uint32_t)P.vs * 2u;
    rso = (uint32_t)P.os * 2u;
    dsk = (uint32_t)(KT ? CK::dmaRowsV : C::dmaRowsK) * rsk;
    dsv = (uint32_t)C::dmaRowsV * rsv;
    // Q operand fragments (rows past Lq read as zeros)
    const uint32_t rsq = (uint32_t)P.qs * 2u;
    const auto rq = FA_RSRC((const char*)P.q + q0 * 2, (uint32_t)Lq * rsq);
#pragma unroll
    for (int j = 0; j < NDC; ++j)
      qf[j] = __builtin_amdgcn_raw_buffer_load_b128(rq, q_frag_off<D>(qrow, j, hh, rsq), 0, 0);
    // per-lane LDS / DMA base offsets; the rest are XOR / immediate offsets
    koff0 = KT ? v_tr_off<BN>(0, 0, 0, lane) : k_read_off<D>(0, 0, lane);
    voff0 = v_tr_off<D>(0, 0, 0, lane);
    kdo0 = KT ? dma_src_v<CK>(wave, 0, lane, rsk) : dma_src_k<C>(wave, 0, lane, rsk);
    vdo0 = dma_src_v<C>(wave, 0, lane, rsv);
#pragma unroll
    for (int j = 0; j < NDB; ++j) o[j] = (f32x16){};
    this->reset_softmax();
    n_events = 0;
    return true;
  }

  // this wave's share of the DMA of K or V tile t into an LDS stage; a tile
  // at or past `limit` is an empty range (the DMA then writes zeros)
  __device__ __forceinline__ void dma_k(lds_char* dst, int t, int limit = 0x7fffffff) const {
    const int kv0 = t * BN;
    if constexpr (KT) {
      // D rows of keys kv0 .. kv0+BN-1; the range runs to the end of this
      // head's [D, S] block. Keys past Lk read the next row's values (or
      // zeros past the block): finite, and masked like any key past the end.
      const uint32_t bytes = dma_bytes((t < limit) & (kv0 < Lk), (uint32_t)D * rsk - (uint32_t)kv0 * 2u);
      const auto r = FA_RSRC(Kh + (size_t)kv0 * 2, bytes);
#pragma unroll
      for (int i = 0; i < DPW; ++i) {
        lds_char* const lp = dst + dma_lds_v<CK>(wave, i);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lp, 16, kdo0 + i * dsk, 0, 0, 0);
      }
    } else {
      const uint32_t bytes = dma_bytes((t < limit) & (kv0 < Lk), (uint32_t)(Lk - kv0) * rsk);
      const auto r = FA_RSRC(Kh + (size_t)kv0 * rsk, bytes);
#pragma unroll
      for (int i = 0; i < DPW; ++i) {
        // (the LDS pointer goes through a local: written inline as the builtin's
        // argument, the host compilation pass drops the kernel launch stubs)
        lds_char* const lp = dst + dma_lds_k<C>(wave, i);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lp, 16, kdo0 + i * dsk, 0, 0, 0);
      }
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

  // S^T = K Q^T for the tile at kt (step 0 starts from a zero accumulator)
  __device__ __forceinline__ void qk(f32x16 (&s)[NKB], const lds_char* kt) const {
#pragma unroll
    for (int j = 0; j < NDC; ++j) {
      if constexpr (KT) {
        // K operand of block kb, step j from the transposed tile: the V^T
        // read of fa_layout.h with d as the row and the key block as jd
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          s[kb] = Ops<T>::mfma(lds_tr_pair(kt + (koff0 ^ (uint32_t)(kb << 6)) + j * 16 * RBK, 4 * RBK),
                               qf[j], j == 0 ? (f32x16){} : s[kb]);
      } else {
        const lds_char* base = kt + (koff0 ^ (uint32_t)(j << 5));
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          s[kb] = Ops<T>::mfma(lds16(base + kb * 32 * RB), qf[j], j == 0 ? (f32x16){} : s[kb]);
      }
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
  // scheduling patterns of the two products: operands read several MFMAs
  // ahead (two reads per P.V MFMA and one per S MFMA, four MFMAs ahead)
  static __device__ __forceinline__ void pv_schedule() { read_ahead<8, NKC * NDB, 2>(); }
  static __device__ __forceinline__ void qk_schedule() {
    if constexpr (KT) read_ahead<8, NDC * NKB, 2>();
    else read_ahead<4, NDC * NKB, 1>();
  }
  // softmax of one tile (about 4.5 vector instructions per score, BN / 2
  // scores per lane) spread over the next tile's S MFMAs
  static __device__ __forceinline__ void il_schedule() {
    mix<4, NDC * NKB, 1, (9 * BN / 4) / (NDC * NKB) + 1>();
  }
  __device__ __forceinline__ void mask(f32x16 (&s)[NKB], int kv0) const {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 32 * kb + acc_key32(r, hh);
        const bool vis = key < Lk && (!CAUSAL || key <= qrow + off);
        s[kb][r] = vis ? s[kb][r] : -INFINITY;
      }
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
    if (DIAG && j >= 1 && hh == 0 && qrow < Lq && hist < 1.f) ++n_events;
    if (j >= 1 && __builtin_amdgcn_ballot_w64(hist < 1.f) != 0) {
#pragma unroll
      for (int jd = 0; jd < NDB; ++jd) o[jd] *= hist;
    }
  }
  // softmax of tile j in place: mask, base update, rescale of O, P(j)
  __device__ __forceinline__ void softmax_tile(f32x16 (&s)[NKB], u32x4 (&p)[NKC], int j) {
    const int kv0 = j * BN;
    if (this->needs_mask(kv0)) mask(s, kv0);
    const float hist = this->softmax_max(s);
    rescale(j, hist);
    softmax_exp(s, p);
  }

  // normalise once, write O and lse (rows past Lq dropped by the range
  // check). A row that sees no key (possible when Lk < Lq under the causal
  // mask, or Lk = 0) gets O = 0 and lse = -inf.
  __device__ __forceinline__ void epilogue(unsigned long long* events) {
    const float ltot = sum_xor32(lsum);
    if (q0w < Lq) {
      const auto ro = FA_RSRC(Oh, (uint32_t)Lq * rso);
      const auto rl = FA_RSRC(Lh, (uint32_t)Lq * 4u);
      const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
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
          __builtin_amdgcn_raw_buffer_store_b128(w, ro, o_frag_off<D>(qrow, jd, g, hh, rso), 0, 0);
        }
      if (hh == 0) {
        const float l2 = ltot > 0.f ? (b + __builtin_amdgcn_logf(ltot)) * kLn2 : -INFINITY;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, l2), rl,
                                              (uint32_t)qrow * 4u, 0, 0);
      }
    }
    if (DIAG && n_events) atomicAdd(events, (unsigned long long)n_events);
  }
};

// ------------------------------------------------- eight-wave ping-pong
template <typename T, int D, bool CAUSAL, int THR, bool DIAG>
__global__ void __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd_pp(const Problem P) {
  pp_body<Wave<T, Cfg8<D>, CAUSAL, THR, DIAG>>(P);
}

// ------------------------------------------------- persistent ping-pong
template <typename T, int D, bool CAUSAL, int THR, bool DIAG>
__global__ void __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd_pp_persist(const Problem P) {
  pp_persistent<Wave<T, Cfg8<D>, CAUSAL, THR, DIAG>>(P);
}

// ------------------------------------------------- K given transposed
// The ping-pong work-group on a [D, S] K: 64-key tiles at D = 128 and
// 128-key tiles at D = 64, so that a transposed K tile has 128- or 256-byte
// rows like a V tile.
template <int D> using CfgKT = Cfg<D, 8, (D == 64 ? 128 : 64)>;

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd_pp_kt(const Problem P) {
  pp_body<Wave<T, CfgKT<D>, CAUSAL, 8, false, true>>(P);
}

// ------------------------------------------------- eight waves, interleaved
template <typename T, int D, bool CAUSAL, int THR, bool DIAG>
__global__ void __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd_il(const Problem P) {
  il_body<Wave<T, CfgIL<D>, CAUSAL, THR, DIAG>>(P);
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
fa_fwd_w2(const Problem P) {
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
  if (!wa.init(P, 0)) return;
  wb.init(P, 1);
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
  wa.epilogue(P.events);
  wb.epilogue(P.events);
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
fa_fwd_k4(const Problem P) {
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
  if (!w.init(P)) return;
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

  w.epilogue(P.events);
}

// ------------------------------------------------------------------- host

// Kernel choice: the ping-pong kernel when its 256-row tiles give at least
// one work-group per compute unit, else the four-wave kernel.
constexpr long long kPingPongMinGroups = 256;

enum Variant { kAuto = 0, kFourWave = 1, kPingPong = 2, kTwoBlock = 3, kInterleave = 4,
               kPersistent = 5 };

// Work-groups of the persistent kernel: one per CU of the current device,
// rounded down to a multiple of the 8 XCDs.
static int persistent_groups() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus / 8 * 8;
}

template <int D> static bool use_pingpong(int BH, int S, int variant) {
  if (variant == kFourWave) return false;
  if (variant == kPingPong) return true;
  return (long long)num_q_tiles(S, Cfg8<D>::BM) * BH >= kPingPongMinGroups;
}

template <typename T, int D, bool CAUSAL, int THR, bool DIAG>
static int launch_one(Problem P, hipStream_t stream, int variant) {
  const int BH = P.B * P.H;
  if (variant == kPersistent) {
    P.nqt = num_q_tiles(P.Sq, Cfg8<D>::BM);
    const int g = persistent_groups();
    if (g <= 0) return FA_ERR_HIP;
    hipLaunchKernelGGL((fa_fwd_pp_persist<T, D, CAUSAL, THR, DIAG>), dim3((unsigned)g),
                       dim3(Cfg8<D>::threads), 0, stream, P);
  } else if (variant == kInterleave) {
    P.nqt = num_q_tiles(P.Sq, CfgIL<D>::BM);
    hipLaunchKernelGGL((fa_fwd_il<T, D, CAUSAL, THR, DIAG>), dim3((unsigned)P.nqt * (unsigned)BH),
                       dim3(CfgIL<D>::threads), 0, stream, P);
  } else if (variant == kTwoBlock) {
    P.nqt = num_q_tiles(P.Sq, CfgW2<D>::BM);
    hipLaunchKernelGGL((fa_fwd_w2<T, D, CAUSAL, THR, DIAG>), dim3((unsigned)P.nqt * (unsigned)BH),
                       dim3(CfgW2<D>::threads), 0, stream, P);
  } else if (use_pingpong<D>(BH, P.Sq, variant)) {
    P.nqt = num_q_tiles(P.Sq, Cfg8<D>::BM);
    hipLaunchKernelGGL((fa_fwd_pp<T, D, CAUSAL, THR, DIAG>), dim3((unsigned)P.nqt * (unsigned)BH),
                       dim3(Cfg8<D>::threads), 0, stream, P);
  } else {
    P.nqt = num_q_tiles(P.Sq, Cfg4<D>::BM);
    hipLaunchKernelGGL((fa_fwd_k4<T, D, CAUSAL, THR, DIAG>), dim3((unsigned)P.nqt * (unsigned)BH),
                       dim3(Cfg4<D>::threads), 0, stream, P);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

template <typename T, int THR, bool DIAG>
static int launch(const Problem& P, int D, int causal, hipStream_t st, int variant) {
  if (D == 64)
    return causal ? launch_one<T, 64, true, THR, DIAG>(P, st, variant)
                  : launch_one<T, 64, false, THR, DIAG>(P, st, variant);
  return causal ? launch_one<T, 128, true, THR, DIAG>(P, st, variant)
                : launch_one<T, 128, false, THR, DIAG>(P, st, variant);
}

template <typename T> static int launch_kt(Problem P, int D, int causal, hipStream_t st) {
  P.nqt = num_q_tiles(P.Sq, 256);
  const dim3 grid((unsigned)P.nqt * (unsigned)(P.B * P.H)), block(512);
  if (D == 64) {
    if (causal) hipLaunchKernelGGL((fa_fwd_pp_kt<T, 64, true>), grid, block, 0, st, P);
    else hipLaunchKernelGGL((fa_fwd_pp_kt<T, 64, false>), grid, block, 0, st, P);
  } else {
    if (causal) hipLaunchKernelGGL((fa_fwd_pp_kt<T, 128, true>), grid, block, 0, st, P);
    else hipLaunchKernelGGL((fa_fwd_pp_kt<T, 128, false>), grid, block, 0, st, P);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

static int launch_dtype(const Problem& P, int D, int causal, int dtype, hipStream_t st) {
  return dtype == FA_BF16 ? launch<__bf16, 8, false>(P, D, causal, st, kAuto)
                          : launch<_Float16, 8, false>(P, D, causal, st, kAuto);
}

// ------------------------------------------------------- host validation
// Touches no HIP API.

// Byte span [lo, hi) of a strided tensor: dims n[i] with strides st[i]
// (elements), the innermost extent `inner` elements, element size es.
struct Span {
  uintptr_t lo, hi;
};
static Span span_of(const void* base, const long long* n, const long long* st, int nd,
                    long long inner, int es) {
  long long last = inner;  // one past the last element, relative to base
  for (int i = 0; i < nd; ++i) last += (n[i] - 1) * st[i];
  return {(uintptr_t)base, (uintptr_t)base + (uintptr_t)(last * es)};
}
static bool spans_overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// True when no two index tuples of dims n (strides st, all >= 0) with an
// innermost block of `inner` contiguous elements share an element: sorted by
// stride, each stride must clear the whole extent of the smaller ones.
static bool no_self_overlap(const long long* n, const long long* st, int nd, long long inner) {
  long long dn[4], ds[4];
  int m = 0;
  for (int i = 0; i < nd; ++i)
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
    if (ds[i] < extent) return false;
    extent = ds[i] * (dn[i] - 1) + extent;
  }
  return true;
}

// Scalar checks shared by every entry point.
static int validate_args(int B, int H, int Sq, int Sk, int D, int causal, float scale, int dtype) {
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (B < 0 || H < 0 || Sq < 0 || Sk < 0) return FA_ERR_DIM;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  if ((long long)B * H * num_q_tiles(Sq, Cfg4<64>::BM) >= (1LL << 31)) return FA_ERR_DIM;
  return FA_OK;
}

// Checks on a filled Problem (non-empty). rows_q / rows_k: the query and key
// row counts of each tensor's outer dims, as (n, stride) pairs per dim.
static int validate_problem(const Problem& P, int D, const long long* nq, const long long* sq_,
                            const long long* sk_, const long long* sv_, const long long* so_,
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
  for (int i = 0; i < 12; ++i)
    if (all[i] % 8) return FA_ERR_ALIGN;  // every row starts 16-byte aligned
  if (P.qs < D || P.ks < D || P.vs < D || P.os < D) return FA_ERR_LAYOUT;
  // offsets within one (sequence, head) are 32-bit bytes
  const long long lim = 1LL << 31;
  if ((long long)P.Sq * P.qs * 2 >= lim || (long long)P.Sk * P.ks * 2 >= lim ||
      (long long)P.Sk * P.vs * 2 >= lim || (long long)P.Sq * P.os * 2 >= lim ||
      (long long)P.Sq * 4 >= lim)
    return FA_ERR_DIM;
  if (!no_self_overlap(nq, so_, nd, D) || !no_self_overlap(nl, sl, ndl, 1)) return FA_ERR_LAYOUT;
  const Span q = span_of(P.q, nq, sq_, nd, D, 2), k = span_of(P.k, nk, sk_, nd, D, 2),
             v = span_of(P.v, nk, sv_, nd, D, 2), o = span_of(P.o, nq, so_, nd, D, 2),
             l = span_of(P.lse, nl, sl, ndl, 1, 4);
  if (spans_overlap(o, q) || spans_overlap(o, k) || spans_overlap(o, v) || spans_overlap(l, q) ||
      spans_overlap(l, k) || spans_overlap(l, v) || spans_overlap(l, o))
    return FA_ERR_ALIAS;
  if ((uint64_t)(o.hi - o.lo) >> 41 || (uint64_t)(q.hi - q.lo) >> 41) return FA_ERR_DIM;  // 2^40 elements
  return FA_OK;
}

// Fixed-length problem from strides (14: q, k, v, o as batch, head, row; lse
// as batch, head). *empty is set when there is no query row to compute.
static int make_fixed(Problem* P, const void* q, const void* k, const void* v, void* o,
                      float* lse, int B, int H, int Sq, int Sk, int D, int causal, float scale,
                      int dtype, const long long* st, bool* empty) {
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

// Dense problem with K given transposed: q, v, o [B,H,S,D], k [B,H,D,S].
static int make_kt(Problem* P, const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int S, int D, int causal, float scale, int dtype, bool* empty) {
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
  if ((long long)S * D * 2 >= (1LL << 31)) return FA_ERR_DIM;
  const long long n = (long long)B * H * S * D;
  if (n > (1LL << 40)) return FA_ERR_DIM;
  const Span sq{(uintptr_t)q, (uintptr_t)q + (uintptr_t)(2 * n)},
      sk{(uintptr_t)k, (uintptr_t)k + (uintptr_t)(2 * n)},
      sv{(uintptr_t)v, (uintptr_t)v + (uintptr_t)(2 * n)},
      so{(uintptr_t)o, (uintptr_t)o + (uintptr_t)(2 * n)},
      sl{(uintptr_t)lse, (uintptr_t)lse + (uintptr_t)(4LL * B * H * S)};
  if (spans_overlap(so, sq) || spans_overlap(so, sk) || spans_overlap(so, sv) ||
      spans_overlap(sl, sq) || spans_overlap(sl, sk) || spans_overlap(sl, sv) ||
      spans_overlap(sl, so))
    return FA_ERR_ALIAS;
  const long long hs = (long long)S * D;
  // k's third stride is the distance between its d rows (S elements)
  *P = Problem{q, k, v, o, lse, H * hs, hs, D, H * hs, hs, S, H * hs, hs, D, H * hs, hs, D,
               (long long)H * S, S, nullptr, nullptr, 0, 0, B, H, S, S, 0, scale * kLog2e,
               nullptr, 0.f, kHeadGroup};
  return FA_OK;
}

// 8-bit inputs (fa_fwd_fp8.hip)
int launch_fp8(Problem P, int D, int causal, hipStream_t stream);

static bool positive_finite(float x) { return x > 0.f && isfinite(x); }

// Dense [B,H,S,D] problem on E4M3 inputs (one byte per element) with a bf16
// output (two bytes per element).
static int make_fp8(Problem* P, const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int S, int D, int causal, float scale, float dq, float dk,
                    float dv, bool* empty) {
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
  if ((long long)B * H * num_q_tiles(S, CfgF8::BM) >= (1LL << 31)) return FA_ERR_DIM;
  if ((long long)B * H * S == 0) {
    *empty = true;
    return FA_OK;
  }
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse) & 15)
    return FA_ERR_ALIGN;
  // one head's O rows addressed with 32-bit byte offsets; at most 2^40 elements
  if ((long long)S * D * 2 >= (1LL << 31)) return FA_ERR_DIM;
  const long long n = (long long)B * H * S * D;
  if (n > (1LL << 40)) return FA_ERR_DIM;
  const Span sq{(uintptr_t)q, (uintptr_t)q + (uintptr_t)n}, sk{(uintptr_t)k, (uintptr_t)k + (uintptr_t)n},
      sv{(uintptr_t)v, (uintptr_t)v + (uintptr_t)n}, so{(uintptr_t)o, (uintptr_t)o + (uintptr_t)(2 * n)},
      sl{(uintptr_t)lse, (uintptr_t)lse + (uintptr_t)(4LL * B * H * S)};
  if (spans_overlap(so, sq) || spans_overlap(so, sk) || spans_overlap(so, sv) ||
      spans_overlap(sl, sq) || spans_overlap(sl, sk) || spans_overlap(sl, sv) ||
      spans_overlap(sl, so))
    return FA_ERR_ALIAS;
  const long long hs = (long long)S * D;
  *P = Problem{q, k, v, o, lse, H * hs, hs, D, H * hs, hs, D, H * hs, hs, D, H * hs, hs, D,
               (long long)H * S, S, nullptr, nullptr, 0, 0, B, H, S, S, 0, (float)c, nullptr, dv,
               kHeadGroup};
  return FA_OK;
}

static void dense_strides(long long* st, int H, int S, int D) {
  const long long hs = (long long)S * D;
  const long long v[] = {H * hs, hs, D, H * hs, hs, D, H * hs, hs, D, H * hs, hs, D,
                         (long long)H * S, S};
  for (int i = 0; i < 14; ++i) st[i] = v[i];
}

}  // namespace fa

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int S,
           int D, int causal, float scale, hipStream_t stream, int dtype) {
  long long st[14];
  fa::dense_strides(st, H, S, D);
  fa::Problem P;
  bool empty;
  const int r = fa::make_fixed(&P, q, k, v, o, lse, B, H, S, S, D, causal, scale, dtype, st, &empty);
  if (r != FA_OK || empty) return r;
  return fa::launch_dtype(P, D, causal, dtype, stream);
}

int fa_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int S, int D, int causal, float scale, hipStream_t stream) {
  return fa_fwd(q, k, v, o, lse, B, H, S, D, causal, scale, stream, FA_F16);
}

int fa_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int S, int D, int causal, float scale, hipStream_t stream) {
  return fa_fwd(q, k, v, o, lse, B, H, S, D, causal, scale, stream, FA_BF16);
}

int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int H, int Sq, int Sk, int D, int causal, float scale, hipStream_t stream,
                   int dtype, const long long* strides) {
  fa::Problem P;
  bool empty;
  const int r =
      fa::make_fixed(&P, q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale, dtype, strides, &empty);
  if (r != FA_OK || empty) return r;
  return fa::launch_dtype(P, D, causal, dtype, stream);
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H,
                  int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int D,
                  int causal, float scale, hipStream_t stream, int dtype,
                  const long long* strides) {
  int r = fa::validate_args(B, H, max_seqlen_q, max_seqlen_k, D, causal, scale, dtype);
  if (r != FA_OK) return r;
  if (total_q < 0 || total_k < 0) return FA_ERR_DIM;
  if ((long long)B * H * max_seqlen_q == 0 || total_q == 0) return FA_OK;
  if (!cu_seqlens_q || !cu_seqlens_k || !strides) return FA_ERR_NULL;
  if (((uintptr_t)cu_seqlens_q | (uintptr_t)cu_seqlens_k) & 3) return FA_ERR_ALIGN;
  const long long* st = strides;  // q, k, v, o as head, row; lse as head
  fa::Problem P{q, k, v, o, lse, 0, st[0], st[1], 0, st[2], st[3], 0, st[4], st[5], 0,
                st[6], st[7], 0, st[8], cu_seqlens_q, cu_seqlens_k, total_q, total_k,
                B, H, max_seqlen_q, max_seqlen_k, 0, scale * fa::kLog2e, nullptr, 0.f,
                // one sequence's heads on an XCD at a time (sequences differ in length)
                H % 8 == 0 ? H / 8 : 1};
  const long long nq[] = {H, total_q}, nk[] = {H, total_k > 0 ? total_k : 1};
  const long long sq_[] = {st[0], st[1]}, sk_[] = {st[2], st[3]}, sv_[] = {st[4], st[5]},
                  so_[] = {st[6], st[7]};
  const long long nl[] = {H, total_q}, sl[] = {st[8], 1};
  r = fa::validate_problem(P, D, nq, sq_, sk_, sv_, so_, nk, 2, nl, sl, 2);
  if (r != FA_OK) return r;
  return fa::launch_dtype(P, D, causal, dtype, stream);
}

int fa_fwd_diag(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int S, int D, int causal, float scale, hipStream_t stream, int dtype,
                int threshold_log2, int variant, unsigned long long* rescale_events) {
  long long st[14];
  fa::dense_strides(st, H, S, D);
  fa::Problem P;
  bool empty;
  const int r = fa::make_fixed(&P, q, k, v, o, lse, B, H, S, S, D, causal, scale, dtype, st, &empty);
  if (r != FA_OK) return r;
  if (threshold_log2 != 0 && threshold_log2 != 8) return FA_ERR_ARG;
  if (variant < fa::kAuto || variant > fa::kPersistent) return FA_ERR_ARG;
  if (!rescale_events) return FA_ERR_NULL;
  if (((uintptr_t)rescale_events & 7) != 0) return FA_ERR_ALIGN;
  if (empty) return FA_OK;
  P.events = rescale_events;
  const bool bf = dtype == FA_BF16;
  if (threshold_log2 == 8)
    return bf ? fa::launch<__bf16, 8, true>(P, D, causal, stream, variant)
              : fa::launch<_Float16, 8, true>(P, D, causal, stream, variant);
  return bf ? fa::launch<__bf16, 0, true>(P, D, causal, stream, variant)
            : fa::launch<_Float16, 0, true>(P, D, causal, stream, variant);
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
    case FA_ERR_LAYOUT: return "a stride is negative, a row stride is below D, or output rows overlap";
    default: return "unknown status";
  }
}

int fa_fwd_kt(const void* q, const void* kt, const void* v, void* o, float* lse, int B, int H,
              int S, int D, int causal, float scale, hipStream_t stream, int dtype) {
  fa::Problem P;
  bool empty;
  const int r = fa::make_kt(&P, q, kt, v, o, lse, B, H, S, D, causal, scale, dtype, &empty);
  if (r != FA_OK || empty) return r;
  return dtype == FA_BF16 ? fa::launch_kt<__bf16>(P, D, causal, stream)
                          : fa::launch_kt<_Float16>(P, D, causal, stream);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int S, int D, int causal, float scale, float descale_q, float descale_k,
               float descale_v, hipStream_t stream) {
  fa::Problem P;
  bool empty;
  const int r = fa::make_fp8(&P, q, k, v, o, lse, B, H, S, D, causal, scale, descale_q,
                             descale_k, descale_v, &empty);
  if (r != FA_OK || empty) return r;
  return fa::launch_fp8(P, D, causal, stream);
}

int fa_version(void) { return 310; }

}  // extern "C"
