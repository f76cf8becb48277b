// The key-split kernel, for grids too small to fill the chip (D = 64).
//
// With few (query tile, head) items the time is the serial chain of the
// longest item: one KV tile after another, each a dependent round of LDS
// reads, MFMAs and exponentials. Here a work-group holds kSplitGroups groups
// of two waves; every group covers the same 64 query rows and takes every
// kSplitGroups-th KV tile (group g: tiles g, g + 4, g + 8, ...) on its own
// two K and two V buffers. Each group keeps its own base, row sums and O
// for its keys (the online softmax of "FlashAttention" (Dao et al.), section
// 3.1, run over a subset of the key blocks); at the end the groups' parts
// are added pairwise, each scaled by 2^(its base - the larger base) (the
// same rescaling as between two key blocks of one pass), and group 0
// normalises and writes the rows. The chain of the longest item is a
// quarter as long, and two waves share each SIMD.
#pragma once
#include "fa_device.h"
#include "fa_wave.h"

namespace fa {

// two waves (64 query rows) per group, 64-key tiles
template <int D> using CfgSplit = Cfg<D, 2, 64>;
constexpr int kSplitGroups = 4;

// The K/V buffers: one array per role (K buffer 0 and 1, V buffer 0 and 1),
// so that the compiler sees which buffer a DMA in flight writes, each in
// kSplitGroups slices, one per group; then the merge's (base, row sum)
// slots. V arrays come first in name order (as in the other kernels). All
// groups run one copy of the code (with four copies, one per group, the
// kernel's code no longer fit the instruction cache).
#define FA_SPLIT_STAGES(TB, NG)                                \
  __shared__ __attribute__((aligned(1024))) char a_v0[(NG) * (TB)]; \
  __shared__ __attribute__((aligned(1024))) char a_v1[(NG) * (TB)]; \
  __shared__ __attribute__((aligned(1024))) char b_k0[(NG) * (TB)]; \
  __shared__ __attribute__((aligned(1024))) char b_k1[(NG) * (TB)]; \
  __shared__ __attribute__((aligned(16))) char c_par[(NG) * 1024];

// Where a group parks its partial result for the merge, in its own slices
// (free once the last iteration has ended): wave v's d-block jd of O in
// buffer (K0, K1, V0, V1)[2v + jd], as [4 accumulator elements][lane] of
// 16-byte entries; base and row sum in the group's kilobyte of c_par at
// 512 * v, as [lane][2] floats.
template <class W> struct SplitPark {
  static_assert(W::NDB == 2 && 4 * 64 * 16 <= W::Config::tileBytes,
                "two d-blocks of O per wave, one per buffer");
  static __device__ __forceinline__ uint32_t o_off(int q, int lane) {
    return (uint32_t)((q * 64 + lane) * 16);
  }
  static __device__ __forceinline__ uint32_t s_off(int g, int wv, int lane) {
    return (uint32_t)(1024 * g + 512 * wv + 8 * lane);
  }
};

// Group g's pass over its tiles g, g+NG, ..., then its part of the merge.
// ntiles: the work-group's KV tiles; nw: this wave's. Every group runs group
// 0's number of steps (the most), so all waves pass the same barriers. The
// K/V buffer arrays hold the groups' slices of TB bytes; par the (base, row
// sum) slots.
template <class W, int NG>
__device__ __forceinline__ void split_group(const Problem& P, W& w, int g, int ntiles, int nw,
                                            lds_char* const bk0, lds_char* const bk1,
                                            lds_char* const bv0, lds_char* const bv1,
                                            lds_char* const par) {
  using C = typename W::Config;
  constexpr int NKB = W::NKB, NKC = W::NKC, NDB = W::NDB;
  constexpr int TB = C::tileBytes;
  static_assert((NG & (NG - 1)) == 0, "the merge halves the groups");
  const uint32_t slice = (uint32_t)g * TB;
  lds_char* const lk0 = bk0 + slice;
  lds_char* const lk1 = bk1 + slice;
  lds_char* const lv0 = bv0 + slice;
  lds_char* const lv1 = bv1 + slice;
  const int nt = ntiles > g ? (ntiles - g + NG - 1) / NG : 0;  // this group's tiles
  const int n0 = (ntiles + NG - 1) / NG;                       // group 0's
  const int nwg = nw > g ? (nw - g + NG - 1) / NG : 0;         // this wave's
  auto tile = [&](int i) { return NG * i + g; };

  // Step i (PH = i % 2): local tile i sits in buffers PH; the DMA of tile
  // i+1 into the other buffers (read in step i-1, which every wave has left
  // at the barrier), then tile i start to end: S, the lazy softmax, P.V; a
  // full wait and the barrier. (A three-stage register pipeline, S(i+1) and
  // P(i-1).V(i-1) under softmax(i), took 232 registers and ran 10-12%
  // longer on these grids.)
  f32x16 s[NKB];
  u32x4 p[NKC];
  if (nt > 0) {
    w.dma_k(lk0, tile(0));
    w.dma_v(lv0, tile(0));
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  auto step = [&](auto ph, int i) {
    constexpr int PH = decltype(ph)::value;
    if (i + 1 < nt) {
      w.dma_k(PH ? lk0 : lk1, tile(i + 1));
      w.dma_v(PH ? lv0 : lv1, tile(i + 1));
    }
    __builtin_amdgcn_sched_barrier(0);
    if (i < nwg) {
      w.qk(s, PH ? lk1 : lk0);
      W::qk_schedule();
      w.softmax_tile_at(s, p, tile(i) * W::BN, i);
      w.pv(p, PH ? lv1 : lv0);
      W::pv_schedule();
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  int i = 0;
  for (; i + 1 < n0; i += 2) {
    step(IC<0>{}, i);
    step(IC<1>{}, i + 1);
  }
  if (i < n0) step(IC<0>{}, i);

  // merge, a tree: in the round for `half` (NG/2, ..., 1), groups half ..
  // 2*half-1 park their part and groups 0 .. half-1 add part g + half. A
  // round's parkers write only their own slices, which no group reads in
  // that round, so one barrier per round.
  using Park = SplitPark<W>;
  const int lane = w.lane;
#pragma unroll
  for (int half = NG / 2; half >= 1; half /= 2) {
    if (g >= half && g < 2 * half) {
#pragma unroll
      for (int jd = 0; jd < NDB; ++jd) {
        lds_char* const ob = (w.wave == 0 ? (jd == 0 ? bk0 : bk1) : (jd == 0 ? bv0 : bv1)) + slice;
        const f32x16& a = w.o[jd];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          *(__attribute__((address_space(3))) f32x2*)(ob + Park::o_off(q, lane)) =
              (f32x2){a[4 * q], a[4 * q + 1]};
          *(__attribute__((address_space(3))) f32x2*)(ob + Park::o_off(q, lane) + 8) =
              (f32x2){a[4 * q + 2], a[4 * q + 3]};
        }
      }
      *(__attribute__((address_space(3))) f32x2*)(par + Park::s_off(g, w.wave, lane)) =
          (f32x2){w.b, w.lsum};
    }
    __syncthreads();
    if (g < half) {
      const int h = g + half;
      const f32x2 bl =
          *(__attribute__((address_space(3))) f32x2*)(par + Park::s_off(h, w.wave, lane));
      const float bn = vmax(w.b, bl[0]);
      // 2^(b_old - b_new) for each part; a part that saw no key (base -inf)
      // adds nothing
      const float f0 = w.b == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(w.b - bn);
      const float f1 = bl[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(bl[0] - bn);
#pragma unroll
      for (int jd = 0; jd < NDB; ++jd) {
        lds_char* const ob =
            (w.wave == 0 ? (jd == 0 ? bk0 : bk1) : (jd == 0 ? bv0 : bv1)) + (uint32_t)h * TB;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x2 x = *(__attribute__((address_space(3))) f32x2*)(ob + Park::o_off(q, lane));
          const f32x2 y =
              *(__attribute__((address_space(3))) f32x2*)(ob + Park::o_off(q, lane) + 8);
          w.o[jd][4 * q] = w.o[jd][4 * q] * f0 + x[0] * f1;
          w.o[jd][4 * q + 1] = w.o[jd][4 * q + 1] * f0 + x[1] * f1;
          w.o[jd][4 * q + 2] = w.o[jd][4 * q + 2] * f0 + y[0] * f1;
          w.o[jd][4 * q + 3] = w.o[jd][4 * q + 3] * f0 + y[1] * f1;
        }
      }
      w.lsum = w.lsum * f0 + bl[1] * f1;
      w.b = bn;
    }
  }
  if (g == 0) {
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
                               (lds_char*)b_k1, (lds_char*)a_v0, (lds_char*)a_v1,
                               (lds_char*)c_par);
}

}  // namespace fa
