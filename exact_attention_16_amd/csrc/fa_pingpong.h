// The eight-wave ping-pong work-group, written once for any wave type W.
//
// W supplies: Config (a Cfg: D, BN, tile bytes, DMA issues per wave), STile
// and PTile (a wave's S and P of one KV tile), init / group_tiles /
// wave_tiles, dma_k / dma_v, qk / pv (the MFMA phase's two products),
// qk_schedule / pv_schedule (their scheduling patterns), softmax_tile and
// epilogue. The 16-bit and the 8-bit kernels differ only there.
#pragma once
#include "fa_device.h"



namespace fa {

template <class W>
__device__ __forceinline__ void pp_item(const Problem& P, W& w, lds_char* const lk0,
                                        lds_char* const lk1, lds_char* const lk2,
                                        lds_char* const lv0, lds_char* const lv1,
                                        lds_char* const lv2);

// The stage arrays of the ping-pong work-group, declared by each body.
#define FA_PP_STAGES(TB)                                              \
  __shared__ __attribute__((aligned(1024))) char a_vstage0[TB];      \
  __shared__ __attribute__((aligned(1024))) char a_vstage1[TB];      \
  __shared__ __attribute__((aligned(1024))) char a_vstage2[TB];      \
  __shared__ __attribute__((aligned(1024))) char b_kstage0[TB];      \
  __shared__ __attribute__((aligned(1024))) char b_kstage1[TB];      \
  __shared__ __attribute__((aligned(1024))) char b_kstage2[TB];      \
  lds_char* const lk0 = (lds_char*)b_kstage0;                        \
  lds_char* const lk1 = (lds_char*)b_kstage1;                        \
  lds_char* const lk2 = (lds_char*)b_kstage2;                        \
  lds_char* const lv0 = (lds_char*)a_vstage0;                        \
  lds_char* const lv1 = (lds_char*)a_vstage1;                        \
  lds_char* const lv2 = (lds_char*)a_vstage2;

template <class W> __device__ __forceinline__ void pp_body(const Problem& P) {
  using C = typename W::Config;
  constexpr int TB = C::tileBytes;
  static_assert(kStages == 3, "the step below is unrolled over three stages");
  // One array per stage: with the stage fixed at compile time the compiler
  // sees that an LDS read never aliases the DMA in flight into another stage
  // and inserts no wait for it. The compiler lays the arrays out in name
  // order; the V stages are named to come first, so that their transposed
  // reads (two per P.V MFMA, the part of the MFMA phase with the most
  // instructions per MFMA) mostly fit the 16-bit offset field of the LDS
  // instruction and need no address arithmetic. This affects speed only.
  FA_PP_STAGES(TB)

  W w;
  if (!w.init(P)) return;
  pp_item(P, w, lk0, lk1, lk2, lv0, lv1, lv2);
}

// The persistent form: a fixed grid (a multiple of 8 work-groups, one per
// CU) in which each work-group runs work items one after another, without
// a new launch per item. Work-group b on XCD x = b mod 8 (index c = b / 8
// among the G/8 work-groups of its XCD) takes, at round k, the item of rank
// k*G/8 + c on its XCD for even k and k*G/8 + G/8 - 1 - c for odd k: ranks
// follow the launch order (block_to_tile, or varlen_tile for a compacted
// variable-length launch; heaviest first when causal), so
// the snake pairs heavy items with light ones. Its item ids rise with k,
// so the first id past the end ends the work-group.
template <class W> __device__ __forceinline__ void pp_persistent(const Problem& P) {
  using C = typename W::Config;
  constexpr int TB = C::tileBytes;
  FA_PP_STAGES(TB)

  const int total = P.items;
  for (int k = 0;; ++k) {
    const int id = persistent_item(blockIdx.x, gridDim.x, k, total);
    if (id < 0) break;
    // value-initialised: every member is defined at the top of the item, so
    // no register of the previous item is carried around the loop (left
    // undefined, they were, and the D = 128 body then spilled)
    W w{};
    if (!w.init(P, 0, id)) continue;  // the same for every wave
    pp_item(P, w, lk0, lk1, lk2, lv0, lv1, lv2);
    wg_barrier();  // the next item's prologue refills the stages
  }
}

// One work item (Q tile, head) of the ping-pong work-group, after w.init:
// prologue DMA, the slots of both wave groups, and the epilogue.
template <class W>
__device__ __forceinline__ void pp_item(const Problem& P, W& w, lds_char* const lk0,
                                        lds_char* const lk1, lds_char* const lk2,
                                        lds_char* const lv0, lds_char* const lv1,
                                        lds_char* const lv2) {
  using C = typename W::Config;
  constexpr int DPW = C::dmaPerWave;
  constexpr bool ONE = pp_one_barrier<W::D>;  // one barrier per step, else two
  const int grp = w.wave >> 2;  // 0: waves 0-3, 1: waves 4-7 (one of each per SIMD)
  const int ntiles = w.group_tiles();
  const int nw = w.wave_tiles();
  typename W::STile s;  // S(j), from its MFMA phase to its softmax phase
  typename W::PTile p;  // P(j), from its softmax phase to the next MFMA phase

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

  // prologue: K(0), K(1), V(0) in their stages (K stage 2 and V stages 1
  // and 2 are first written by DMA pairs 0 and 1, before any read of them)
  w.dma_k(lk0, 0);
  w.dma_k(lk1, 1, ntiles);
  w.dma_v(lv0, 0);
  // Slot 0 reads only Q and K(0): K(1) and V(0), the last 2*DPW loads, may
  // still be in flight. They are first read in slot 1, after the end-of-slot
  // wait for all but the latest DMA pair.
  wait_vm_lgkm0<2 * DPW>();
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
    // wave's exponentials whenever both are ready. Group B's softmax phase
    // and DMA issue keep that priority too: its step (MFMA phase, softmax,
    // DMA issue) is the longer chain, which group A waits for at the barrier
    // (ramp 455 against 467 us, long 445 against 446, the other shapes within
    // noise).
    auto step = [&](auto r, int j) {
      constexpr int R = decltype(r)::value;
      __builtin_amdgcn_s_setprio(1);
      if constexpr (G == 0) dma_pair(r, j);
      __builtin_amdgcn_sched_barrier(0);
      if (j >= 1 && j - 1 < nw) {
        w.pv(p, pick3<(R + 2) % 3>(lv0, lv1, lv2));
        W::pv_schedule();
      }
      if (j < nw) {
        w.qk(s, pick3<R>(lk0, lk1, lk2));
        W::qk_schedule();
      }
      if constexpr (ONE) {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (G == 1) end_slot();
      } else {
        end_slot();
      }
      __builtin_amdgcn_s_setprio(G == 1 ? 1 : 0);
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
  w.epilogue(P.events);
}

}  // namespace fa
