// The four-waves-per-SIMD kernel: head dimension 64 without the causal
// mask, on grids that fill the chip.
//
// At D = 64 a score costs a SIMD about 0.25 cycles of matrix core (one QK
// and one PV multiply-add per d) but about 0.32 cycles of vector issue (an
// FMA, an exponential, an add and half a pack), and one wave alone issues
// vector instructions at about two thirds of the rate two waves sharing the
// SIMD reach (the issue-rate probes, include/fa_probe.h). The ping-pong
// kernel keeps one exponentiating wave per SIMD at a time. Here eight waves
// of 32 query rows (256 rows per work-group) take 64-key tiles in at most
// 128 registers each, so two work-groups share a CU and four waves share
// each SIMD; the hardware interleaves their MFMAs and vector work. Each wave
// runs a tile start to end (S = K Q^T, the online softmax of
// "FlashAttention" (Dao et al.) section 3.1 with the lagging base of
// hjcheng0602.cn G6 "V41: Conditional Scale", O += V^T P^T); K/V live in two
// LDS stages, and the next tile's DMA is issued at the top of each step.
// With the causal mask the waves of a diagonal tile finish at different
// steps, and the ping-pong kernel is faster there; the kernel is correct for
// both masks (the diagnostic library runs it on both).
#pragma once
#include "fa_device.h"
#include "fa_wave.h"

namespace fa {

// eight waves (256 query rows), 64-key tiles
template <int D> using CfgOcc4 = Cfg<D, 8, 64>;

template <typename T, int D, bool CAUSAL, int THR, bool DIAG>
__global__ void __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu(4, 4)))
fa_fwd_occ4(const Problem P) {
  using C = CfgOcc4<D>;
  using W = Wave<T, C, CAUSAL, THR, DIAG>;
  static_assert(D == 64, "a wave's state fits 128 registers at D = 64 only");
  constexpr int NKB = W::NKB, NKC = W::NKC;
  constexpr int TB = C::tileBytes;
  // one array per stage (the compiler then sees which stage a DMA in flight
  // writes), V stages first in name order as in the other kernels
  __shared__ __attribute__((aligned(1024))) char a_vstage0[TB];
  __shared__ __attribute__((aligned(1024))) char a_vstage1[TB];
  __shared__ __attribute__((aligned(1024))) char b_kstage0[TB];
  __shared__ __attribute__((aligned(1024))) char b_kstage1[TB];
  lds_char* const lk0 = (lds_char*)b_kstage0;
  lds_char* const lk1 = (lds_char*)b_kstage1;
  lds_char* const lv0 = (lds_char*)a_vstage0;
  lds_char* const lv1 = (lds_char*)a_vstage1;

  W w;
  if (!w.init(P)) return;  // the same for every wave
  const int ntiles = w.group_tiles();
  const int nw = w.wave_tiles();
  f32x16 s[NKB];
  u32x4 p[NKC];

  w.dma_k(lk0, 0);
  w.dma_v(lv0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  wg_barrier();
  // step j (PH = j % 2): tile j in stage PH; the DMA of tile j+1 into the
  // other stage (read in step j-1, which every wave has left at the
  // barrier), then tile j's products and softmax, then a wait for that DMA
  // and the barrier. A wave past its last visible tile keeps issuing its
  // DMA share and meeting the barriers.
  auto step = [&](auto ph, int j) {
    constexpr int PH = decltype(ph)::value;
    lds_char* const kc = PH ? lk1 : lk0;
    lds_char* const vc = PH ? lv1 : lv0;
    if (j + 1 < ntiles) {
      w.dma_k(PH ? lk0 : lk1, j + 1);
      w.dma_v(PH ? lv0 : lv1, j + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (j < nw) {
      // The S MFMAs at raised wave priority: where a wave of the other
      // work-group is exponentiating, these MFMAs and their operand reads
      // issue first. With the three parts kept apart by scheduling barriers
      // this is 1.5-2% shorter on the non-causal D = 64 shapes; the priority
      // without the barrier before P.V, the barriers without the priority,
      // or the priority also for P.V gained nothing.
      __builtin_amdgcn_s_setprio(1);
      w.qk(s, kc);
      W::qk_schedule();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      w.softmax_tile(s, p, j);
      __builtin_amdgcn_sched_barrier(0);
      w.pv(p, vc);
      W::pv_schedule();
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    wg_barrier();
  };
  int j = 0;
  for (; j + 1 < ntiles; j += 2) {
    step(IC<0>{}, j);
    step(IC<1>{}, j + 1);
  }
  if (j < ntiles) step(IC<0>{}, j);
  w.epilogue(P.events);
}

}  // namespace fa
