// One wave's share of the 16-bit attention-forward work-groups (gfx950): its
// 32 query rows held as MFMA operands, its O accumulators, and the per-tile
// operations on them (DMA of its share of a K/V tile, S = K Q^T, the online
// softmax with the lagging base, O += V^T P^T, the epilogue). The
// work-group bodies (fa_pingpong.h and the four-wave kernel in
// fa_kernels.h) are written over this interface.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_device.h"


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
  unsigned n_events;  // rescale events of the wave's rows so far (wave-uniform)

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
  // Hides the keys of the tile at kv0 this lane's row cannot see: keys past
  // Lk and, causal, past qrow + off. Element (kb, r) holds key
  // kv0 + 8*hh + 32*kb + 16*(r/8) + r%8 (acc_key32), a lane base plus a
  // compile-time offset, so one bound on the offset covers both conditions:
  // one compare and one select per score.
  __device__ __forceinline__ void mask(f32x16 (&s)[NKB], int kv0) const {
    const int base = kv0 + 8 * hh;
    int lim = Lk - base;
    if (CAUSAL) lim = min(lim, qrow + off + 1 - base);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int o = 32 * kb + acc_key32(r, 0);
        s[kb][r] = o < lim ? s[kb][r] : -INFINITY;
      }
  }
  // p = 2^(s*c - b) and P packed for the P.V MFMA; returns this lane's sum of
  // the unrounded p over the tile (its k-half of each row's keys)
  __device__ __forceinline__ float exp_tile(const f32x16 (&s)[NKB], u32x4 (&p)[NKC]) const {
    const float nb = (b == -INFINITY) ? 0.f : -b;  // fully hidden row: p = 0
    float ls[4];  // four sum chains, so no add waits on the one before
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float e[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          e[x] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * g + x], c, nb));
          if (kb == 0 && g == 0 && x < 4) ls[x] = 0.f;
          ls[x & 3] += e[x];
        }
        p[2 * kb + g] = (u32x4){Ops<T>::pack2(e[0], e[1]), Ops<T>::pack2(e[2], e[3]),
                                Ops<T>::pack2(e[4], e[5]), Ops<T>::pack2(e[6], e[7])};
      }
    return (ls[0] + ls[1]) + (ls[2] + ls[3]);
  }
  // p = 2^(s*c - b), row sum of the unrounded p, P packed for the P.V MFMA
  __device__ __forceinline__ void softmax_exp(const f32x16 (&s)[NKB], u32x4 (&p)[NKC]) {
    lsum += exp_tile(s, p);
  }
  // rare path: some row of the wave moved its base -> rescale O
  __device__ __forceinline__ void rescale(int j, float hist) {
    if (DIAG && j >= 1)
      n_events += (unsigned)__builtin_popcountll(
          __builtin_amdgcn_ballot_w64(hh == 0 && qrow < Lq && hist < 1.f));
    if (j >= 1 && __builtin_amdgcn_ballot_w64(hist < 1.f) != 0) {
#pragma unroll
      for (int jd = 0; jd < NDB; ++jd) o[jd] *= hist;
    }
  }
  // Softmax of tile j in place: mask, base update, rescale of O, P(j).
  // On a row's first tile the base comes from the tile max (from -inf; V41
  // steps 2-4). After that the exponentials come first, against the current
  // base and in place of the scores: every p of a lane is at most that lane's
  // share of the tile sum, so when no share exceeds 2^THR no scaled score
  // exceeds b + THR and the base stays with history 1 (V41 step 4), and the
  // tile's max is never formed. Otherwise (rare) the row max of the p gives
  // the candidate b + log2(max p); a row whose max p exceeds 2^THR moves its
  // base there and scales its p, its row sum and O by 2^(b_old - b_new).
  // A row's visible keys are a prefix from key 0, so a row whose base is
  // still -inf after its first tile sees no key: all its p are 0 (base 0).
  __device__ __forceinline__ void softmax_tile(f32x16 (&s)[NKB], u32x4 (&p)[NKC], int j) {
    softmax_tile_at(s, p, j * BN, j);
  }
  // The same for the tile at key kv0 that is the j-th tile these rows see
  // (the key-split kernel's groups take every fourth tile)
  __device__ __forceinline__ void softmax_tile_at(f32x16 (&s)[NKB], u32x4 (&p)[NKC], int kv0,
                                                  int j) {
    if (this->needs_mask(kv0)) mask(s, kv0);
    float hist = 1.f;
    if (j == 0) hist = this->softmax_max(s);
    const float nb = (b == -INFINITY) ? 0.f : -b;
    float ls[4];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[kb][r] = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, nb));
        if (kb == 0 && r < 4) ls[r] = 0.f;
        ls[r & 3] += s[kb][r];
      }
    float ts = (ls[0] + ls[1]) + (ls[2] + ls[3]);
    if (j >= 1 && __builtin_amdgcn_ballot_w64(!(ts <= (float)(1 << THR))) != 0) {
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = vmax(mx, s[kb][r]);
      mx = max_xor32(mx);
      const bool rebase = mx > (float)(1 << THR);
      if (__builtin_amdgcn_ballot_w64(rebase) != 0) {
        const float lm = rebase ? __builtin_amdgcn_logf(mx) : 0.f;  // log2 of the row's max p
        hist = rebase ? __builtin_amdgcn_exp2f(-lm) : 1.f;
        b += lm;
        lsum *= hist;
        ts *= hist;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] *= hist;
      }
    }
    rescale(j, hist);
    lsum += ts;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const f32x16& e = s[kb];
        const int r0 = 8 * g;
        p[2 * kb + g] = (u32x4){Ops<T>::pack2(e[r0 + 0], e[r0 + 1]), Ops<T>::pack2(e[r0 + 2], e[r0 + 3]),
                                Ops<T>::pack2(e[r0 + 4], e[r0 + 5]), Ops<T>::pack2(e[r0 + 6], e[r0 + 7])};
      }
  }

  // Normalise once, write O and lse. A row past Lq gets the byte offset
  // where the range ends, so the range check drops it, also where its row
  // times the row stride would wrap in 32 bits (a head's rows take less than
  // 2^31 bytes, so no offset formed here wraps). Both k-halves of a row hold
  // the same lse and both store it. A row that sees no key (possible when
  // Lk < Lq under the causal mask, or Lk = 0) gets O = 0 and lse = -inf.
  __device__ __forceinline__ void store_rows() {
    const float ltot = sum_xor32(lsum);
    const bool in = qrow < Lq;
    // lane part of the offset in the register; the part fixed at compile
    // time goes in the instruction's scalar offset (left to itself the
    // compiler keeps one register per store)
    const uint32_t oend = (uint32_t)Lq * rso, lend = (uint32_t)Lq * 4u;
    const uint32_t orow = (in ? (uint32_t)qrow * rso : oend) + (uint32_t)(16 * hh);
    const uint32_t lrow = in ? (uint32_t)qrow * 4u : lend;
    const auto ro = FA_RSRC(Oh, oend);
    const auto rl = FA_RSRC(Lh, lend);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    // Every value is packed before the first store, and no instruction
    // writes a store's data registers after it (the empty asm below keeps
    // them allocated to the end). Left to itself the compiler reused a
    // 16-byte store's data registers one or two instructions after the store,
    // which the wait states it inserts allow; under heavy LDS-DMA traffic from
    // other waves the store read its data later than that and wrote the new
    // contents (an fp32 where two bf16 were meant): elements 0-1 of some
    // O blocks in lanes 12-15 of each 16-lane group, in a few launches.
    static_assert(NDB == 2 || NDB == 4, "head dimension 64 or 128");
    u32x4 w[NDB][2];
#pragma unroll
    for (int jd = 0; jd < NDB; ++jd)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const f32x16& a = o[jd];
        const int r0 = 8 * g;
        w[jd][g] = (u32x4){Ops<T>::pack2(a[r0 + 0] * inv, a[r0 + 1] * inv),
                           Ops<T>::pack2(a[r0 + 2] * inv, a[r0 + 3] * inv),
                           Ops<T>::pack2(a[r0 + 4] * inv, a[r0 + 5] * inv),
                           Ops<T>::pack2(a[r0 + 6] * inv, a[r0 + 7] * inv)};
      }
    const float l2 = ltot > 0.f ? (b + __builtin_amdgcn_logf(ltot)) * kLn2 : -INFINITY;
    const uint32_t lbits = __builtin_bit_cast(uint32_t, l2);
    __builtin_amdgcn_raw_buffer_store_b32(lbits, rl, lrow, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int jd = 0; jd < NDB; ++jd)
#pragma unroll
      for (int g = 0; g < 2; ++g)  // element r0+e of lane (i, hh): d = 32jd + 16g + 8hh + e
        __builtin_amdgcn_raw_buffer_store_b128(w[jd][g], ro, orow,
                                               (int)(o_frag_off<D>(0, jd, g, 0, rso)), 0);
    if constexpr (NDB == 4)
      asm volatile("" ::"v"(w[0][0]), "v"(w[0][1]), "v"(w[1][0]), "v"(w[1][1]), "v"(w[2][0]),
                   "v"(w[2][1]), "v"(w[3][0]), "v"(w[3][1]), "v"(lbits));
    else
      asm volatile("" ::"v"(w[0][0]), "v"(w[0][1]), "v"(w[1][0]), "v"(w[1][1]), "v"(lbits));
  }
  // the rescale events counted so far, added to *events
  __device__ __forceinline__ void flush_events(unsigned long long* events) const {
    if (DIAG && n_events && lane == 0) atomicAdd(events, (unsigned long long)n_events);
  }
  __device__ __forceinline__ void epilogue(unsigned long long* events) {
    store_rows();
    flush_events(events);
  }
};

}  // namespace fa
