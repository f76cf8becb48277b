// The key-split kernel, for grids too small to fill the chip (D = 64).
//
// With few (query tile, head) items the time is the serial chain of the
// longest item: one wave per SIMD, each KV tile a dependent round of LDS
// reads, MFMAs and exponentials. Here a work-group holds kSplitGroups groups
// of two waves; every group covers the same 64 query rows and takes every
// kSplitGroups-th KV tile (group g: tiles g, g + 4, g + 8, ...), with the
// four-wave kernel's pipeline on its own two-stage K/V buffers. Each group
// keeps its own base, row sums and O for its keys (the online softmax of
// "FlashAttention" (Dao et al.), section 3.1, run over a subset of the
// key blocks); at the end groups 1..3 park theirs in LDS and group 0 adds
// them in, each scaled by 2^(its base - the largest base) (the same
// rescaling as between two key blocks of one pass), then normalises and
// writes the rows. The chain of the longest item is a quarter as long, and
// two waves share each SIMD.
#pragma once
#include "fa_device.h"
#include "fa_wave.h"

namespace fa {

// two waves (64 query rows) per group, 64-key tiles
template <int D> using CfgSplit = Cfg<D, 2, 64>;
constexpr int kSplitGroups = 4;

// The K/V buffers: one array per role (K buffer 0 and 1, V buffer 0 and 1),
// so that the compiler sees which buffer a DMA in flight writes, each in
// kSplitGroups slices, one per group. V arrays come first in name order (as
// in the other kernels). All groups run one copy of the code (with four
// copies, one per group, the kernel's code no longer fit the instruction
// cache).
#define FA_SPLIT_STAGES(TB, NG)                                \
  __shared__ __attribute__((aligned(1024))) char a_v0[(NG) * (TB)]; \
  __shared__ __attribute__((aligned(1024))) char a_v1[(NG) * (TB)]; \
  __shared__ __attribute__((aligned(1024))) char b_k0[(NG) * (TB)]; \
  __shared__ __attribute__((aligned(1024))) char b_k1[(NG) * (TB)];

// Where a group parks its partial result for the merge, in its own slices
// (free once its last iteration has ended): wave v's O in K buffer v, as
// [d-block][4 accumulator elements][lane] of 16-byte entries; base and row
// sum in V buffer 0 at 512 * v, as [lane][2] floats.
template <class W> struct SplitPark {
  static_assert(W::NDB * 16 * 64 * 4 <= W::Config::tileBytes, "O of a wave fits a buffer");
  static __device__ __forceinline__ uint32_t o_off(int jd, int q, int lane) {
    return (uint32_t)(((jd * 4 + q) * 64 + lane) * 16);
  }
  static __device__ __forceinline__ uint32_t s_off(int wv, int lane) {
    return (uint32_t)(512 * wv + 8 * lane);
  }
};

// Group g's pass over its tiles g, g+NG, ... (the four-wave kernel's
// three-stage register pipeline), then its part of the merge. ntiles: the
// work-group's KV tiles; nw: this wave's. Every group runs group 0's number
// of iterations (the most), so all waves pass the same barriers. The K/V
// buffer arrays hold the groups' slices of TB bytes.
template <class W, int NG>
__device__ __forceinline__ void split_group(const Problem& P, W& w, int g, int ntiles, int nw,
                                            lds_char* const bk0, lds_char* const bk1,
                                            lds_char* const bv0, lds_char* const bv1) {
  using C = typename W::Config;
  constexpr int NKB = W::NKB, NKC = W::NKC, NDB = W::NDB;
  constexpr int TB = C::tileBytes;
  const uint32_t slice = (uint32_t)g * TB;
  lds_char* const lk0 = bk0 + slice;
  lds_char* const lk1 = bk1 + slice;
  lds_char* const lv0 = bv0 + slice;
  lds_char* const lv1 = bv1 + slice;
  const int nt = ntiles > g ? (ntiles - g + NG - 1) / NG : 0;  // this group's tiles
  const int n0 = (ntiles + NG - 1) / NG;                       // group 0's
  const int nwg = nw > g ? (nw - g + NG - 1) / NG : 0;         // this wave's
  auto tile = [&](int i) { return NG * i + g; };

  f32x16 sA[NKB], sB[NKB];  // S of local tile i lives in sA for even i, sB for odd i
  u32x4 pA[NKC], pB[NKC];   // P likewise
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) pB[kc] = (u32x4){};  // P(-1) = 0

  // prologue: the group's first two K tiles; V buffer 1 zero (iteration 0
  // multiplies P(-1) = 0 by it, and 0 * NaN would poison O); S of tile 0
  if (nt > 0) w.dma_k(lk0, tile(0));
  if (nt > 1) w.dma_k(lk1, tile(1));
#pragma unroll
  for (int i = 0; i < TB / (16 * 64 * C::NW); ++i)
    *(__attribute__((address_space(3))) u32x4*)(lv1 + 16 * ((threadIdx.x & (64 * C::NW - 1)) +
                                                            i * 64 * C::NW)) = (u32x4){};
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (nwg > 0) w.qk(sA, lk0);
  __syncthreads();  // K buffer 0 is refilled in iteration 0

  // iteration i (PH = i % 2): DMA of V(i) of the group's tiles, then, for a
  // wave that still has local tile i, P(i-1).V(i-1) and softmax(i), the DMA
  // of K(i+2), and S(i+1); iteration nwg only drains P(nwg-1).V(nwg-1).
  // (Issuing K(i+2) after the softmax rather than at the top spreads the
  // work-group's 64 KiB of DMA per iteration over the iteration: 2-3%
  // shorter on the small causal grids this kernel serves.)
  auto iter = [&](auto ph, int i) {
    constexpr int PH = decltype(ph)::value;
    f32x16(&scur)[NKB] = pick<PH>(sB, sA);
    f32x16(&snext)[NKB] = pick<PH>(sA, sB);
    u32x4(&pcur)[NKC] = pick<PH>(pB, pA);
    u32x4(&pprev)[NKC] = pick<PH>(pA, pB);
    lds_char* k_next = PH ? lk0 : lk1;  // holds K of local tile i+1
    lds_char* k_dma = PH ? lk1 : lk0;   // receives K of local tile i+2
    lds_char* v_cur = PH ? lv1 : lv0;   // receives V of local tile i
    lds_char* v_oth = PH ? lv0 : lv1;   // holds V of local tile i-1
    if (i < nt) w.dma_v(v_cur, tile(i));
    __builtin_amdgcn_sched_barrier(0);
    if (i < nwg) {
      const int kv0 = tile(i) * W::BN;
      if (w.needs_mask(kv0)) w.mask(scur, kv0);
      w.pv(pprev, v_oth);
      const float hist = w.softmax_max(scur);
      w.softmax_exp(scur, pcur);
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) asm volatile("" : "+v"(pcur[kc]));
      asm volatile("" : "+v"(w.lsum));
      __builtin_amdgcn_sched_barrier(0);
      if (i + 2 < nt) w.dma_k(k_dma, tile(i + 2));
      __builtin_amdgcn_sched_barrier(0);
      w.qk(snext, k_next);
      w.rescale(i, hist);
    } else {
      if (i + 2 < nt) w.dma_k(k_dma, tile(i + 2));
      if (i == nwg) w.pv(pprev, v_oth);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  const int niter = n0 + 1;
  int i = 0;
  for (; i + 1 < niter; i += 2) {
    iter(IC<0>{}, i);
    iter(IC<1>{}, i + 1);
  }
  if (i < niter) iter(IC<0>{}, i);

  // merge: groups 1..NG-1 park their O, base and row sum in their own slices
  // (wave v's O in K buffer v, base and row sum in V buffer 0); group 0 adds
  // them in and writes the rows
  using Park = SplitPark<W>;
  const int lane = w.lane;
  if (g > 0) {
    lds_char* const ob = (w.wave == 0 ? bk0 : bk1) + slice;
#pragma unroll
    for (int jd = 0; jd < NDB; ++jd)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x16& a = w.o[jd];
        *(__attribute__((address_space(3))) f32x2*)(ob + Park::o_off(jd, q, lane)) =
            (f32x2){a[4 * q], a[4 * q + 1]};
        *(__attribute__((address_space(3))) f32x2*)(ob + Park::o_off(jd, q, lane) + 8) =
            (f32x2){a[4 * q + 2], a[4 * q + 3]};
      }
    *(__attribute__((address_space(3))) f32x2*)(lv0 + Park::s_off(w.wave, lane)) =
        (f32x2){w.b, w.lsum};
  }
  __syncthreads();
  if (g == 0) {
#pragma unroll
    for (int h = 1; h < NG; ++h) {
      const f32x2 bl =
          *(__attribute__((address_space(3))) f32x2*)(bv0 + h * TB + Park::s_off(w.wave, lane));
      const float bn = vmax(w.b, bl[0]);
      // 2^(b_old - b_new) for each part; a part that saw no key (base -inf)
      // adds nothing
      const float f0 = w.b == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(w.b - bn);
      const float f1 = bl[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(bl[0] - bn);
      lds_char* const ob = (w.wave == 0 ? bk0 : bk1) + h * TB;
#pragma unroll
      for (int jd = 0; jd < NDB; ++jd)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x2 x = *(__attribute__((address_space(3))) f32x2*)(ob + Park::o_off(jd, q, lane));
          const f32x2 y =
              *(__attribute__((address_space(3))) f32x2*)(ob + Park::o_off(jd, q, lane) + 8);
          w.o[jd][4 * q] = w.o[jd][4 * q] * f0 + x[0] * f1;
          w.o[jd][4 * q + 1] = w.o[jd][4 * q + 1] * f0 + x[1] * f1;
          w.o[jd][4 * q + 2] = w.o[jd][4 * q + 2] * f0 + y[0] * f1;
          w.o[jd][4 * q + 3] = w.o[jd][4 * q + 3] * f0 + y[1] * f1;
        }
      w.lsum = w.lsum * f0 + bl[1] * f1;
      w.b = bn;
    }
    w.epilogue(P.events);
  } else {
    w.flush_events(P.events);
  }
}

template <typename T, int D, bool CAUSAL, int THR, bool DIAG>
__global__ void __launch_bounds__(64 * 2 * kSplitGroups)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd_split(const Problem P) {
  using C = CfgSplit<D>;
  using W = Wave<T, C, CAUSAL, THR, DIAG>;
  static_assert(D == 64, "four groups of two 64-key buffer pairs fit the LDS at D = 64");
  FA_SPLIT_STAGES(C::tileBytes, kSplitGroups)
  W w;
  if (!w.init(P)) return;  // the same for every wave
  const int grp = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6) / C::NW);
  split_group<W, kSplitGroups>(P, w, grp, w.group_tiles(), w.wave_tiles(), (lds_char*)b_k0,
                               (lds_char*)b_k1, (lds_char*)a_v0, (lds_char*)a_v1);
}

}  // namespace fa
