// The eight-wave interleaved work-group of the 8-bit kernel
// (fa_fwd_fp8.hip), written over a wave type W with the interface pp_body in
// fa_pingpong.h uses, plus il_schedule: the scheduling pattern of the
// softmax-with-QK block.
//
// All eight waves (two per SIMD) run the same code. Per KV tile j a wave
//   * issues its share of DMA pair j (K(j+2) and V(j+1)), waits until its
//     share of pair j-1 (K(j+1) and V(j)) has landed, and meets the barrier;
//   * masks S(j) where needed, then in one scheduling block computes the
//     softmax of S(j) (max, base, exponentials, P(j)) between the MFMAs of
//     S(j+1) = K(j+1) Q^T, whose result only the next tile needs;
//   * rescales O if some row moved its base, then O += P(j) V(j).
// So each wave overlaps its own exponentials with its own MFMAs, and the two
// waves of a SIMD issue vector instructions side by side, where the
// ping-pong schedule lets only one wave per SIMD exponentiate at a time.
// S(j) and S(j+1) alternate between two register tiles; K and V tiles use
// three LDS stages (tile t in stage t mod 3).
//
// Stage safety: pair j overwrites K(j-1) and V(j-2), both last read in
// iteration j-2 (S(j-1) is computed in iteration j-2), and the wave issuing
// it has passed the barrier of iteration j-1, which every wave reaches only
// after its reads of iteration j-2 have completed (lgkmcnt(0) before each
// barrier). Pair j-1 is complete for every wave after the barrier of
// iteration j.
#pragma once
#include "fa_device.h"

namespace fa {

template <class W> __device__ __forceinline__ void il_body(const Problem& P) {
  using C = typename W::Config;
  constexpr int TB = C::tileBytes;
  constexpr int DPW = C::dmaPerWave;
  static_assert(kStages == 3, "the loop below is unrolled over three stages");
  // one array per stage, V stages first in name order (as in pp_body)
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
  if (!w.init(P)) return;
  const int ntiles = w.group_tiles();
  const int nw = w.wave_tiles();
  typename W::STile s0, s1;  // S(j) for even j, odd j
  typename W::PTile p;

  // prologue: K(0), K(1), V(0) (K stage 2 and V stage 1 are first written
  // by DMA pair 0, before any read of them)
  w.dma_k(lk0, 0);
  w.dma_k(lk1, 1, ntiles);
  w.dma_v(lv0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  wg_barrier();
  if (nw > 0) {
    w.qk(s0, lk0);
    W::qk_schedule();
  }

  // iteration j (R = j mod 3, PS = j mod 2): S(j) in s[PS]; K(j+1) in stage
  // R+1, V(j) in stage R
  auto iter = [&](auto r, auto ps, int j) {
    constexpr int R = decltype(r)::value;
    constexpr int PS = decltype(ps)::value;
    auto& scur = pick<PS>(s1, s0);
    auto& snext = pick<PS>(s0, s1);
    w.dma_k(pick3<(R + 2) % 3>(lk0, lk1, lk2), j + 2, ntiles);
    w.dma_v(pick3<(R + 1) % 3>(lv0, lv1, lv2), j + 1, ntiles);
    wait_vm_lgkm0<2 * DPW>();
    wg_barrier();
    if (j < nw) {
      const int kv0 = j * W::BN;
      if (w.needs_mask(kv0)) w.mask(scur, kv0);
      __builtin_amdgcn_sched_barrier(0);
      // (at the wave's last tile S(j+1) is computed and not used: that keeps
      // the block free of branches, so its MFMAs and vector work interleave)
      const float hist = w.softmax_max(scur);
      w.softmax_exp(scur, p);
      w.qk(snext, pick3<(R + 1) % 3>(lk0, lk1, lk2));
      W::il_schedule();
      __builtin_amdgcn_sched_barrier(0);
      w.rescale(j, hist);
      w.pv(p, pick3<R>(lv0, lv1, lv2));
      W::pv_schedule();
    }
  };
  for (int j = 0;; j += 6) {
    if (j >= ntiles) break;
    iter(IC<0>{}, IC<0>{}, j);
    if (j + 1 >= ntiles) break;
    iter(IC<1>{}, IC<1>{}, j + 1);
    if (j + 2 >= ntiles) break;
    iter(IC<2>{}, IC<0>{}, j + 2);
    if (j + 3 >= ntiles) break;
    iter(IC<0>{}, IC<1>{}, j + 3);
    if (j + 4 >= ntiles) break;
    iter(IC<1>{}, IC<0>{}, j + 4);
    if (j + 5 >= ntiles) break;
    iter(IC<2>{}, IC<1>{}, j + 5);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no DMA into LDS outlives the work-group
  w.epilogue(P.events);
}

}  // namespace fa
