// The 16-bit attention-forward kernels for gfx950 and their launch
// templates, shared by the product library (fa_fwd.hip: the production
// instantiations) and the diagnostic library (fa_fwd_diag.hip: the same
// kernels instantiated with a rescale-event counter and a lag threshold of
// 0 or 8, plus the persistent form of the ping-pong kernel).
//
//  * fa_fwd_pp (eight waves, 256 query rows; work-group body in
//    fa_pingpong.h): two wave groups whose slots alternate between an MFMA
//    phase and a softmax phase, so each SIMD always holds one multiplying
//    and one exponentiating wave; K/V in three LDS stages, two tiles ahead.
//  * fa_fwd_k4 (four waves, 128 query rows), for grids too small to fill the
//    chip with 256-row tiles: each wave runs a tile start to end, the other
//    waves on its SIMD covering its latencies.
//  * fa_fwd_split (fa_split.h), for small grids at D = 64: four groups of
//    two waves split each query tile's KV tiles, merged in LDS.
//  * fa_fwd_occ4 (fa_occ4.h), D = 64 without the causal mask on grids that
//    fill the chip: eight waves, 64-key tiles, four waves per SIMD.
//  * fa_fwd_pp_kt: the ping-pong body on a K given transposed ([D, S]).
//  * fa_fwd_pp_persist: the ping-pong body in persistent form.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/fa_fwd.h"
#include "fa_device.h"
#include "fa_pingpong.h"
#include "fa_occ4.h"
#include "fa_split.h"
#include "fa_wave.h"

namespace fa {

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


// ------------------------------------------------------------ four-wave
// Each wave runs a tile start to end: S = K Q^T, the softmax (base update
// from the tile max, the rare rescale of O, exponentials), P.V; K and V in
// two LDS stages each, the next tile's DMA issued at the top of the step.
// The other waves on the SIMD cover one wave's latencies. (A register
// pipeline, the next tile's S and, at D = 64, the previous tile's P.V under
// the current softmax, took 200-230 registers and ran 5-12% longer on the
// small grids this kernel serves.)
template <typename T, int D, bool CAUSAL, int THR, bool DIAG>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd_k4(const Problem P) {
  using C = Cfg4<D>;
  using W = Wave<T, C, CAUSAL, THR, DIAG>;
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
  f32x16 s[NKB];
  u32x4 p[NKC];

  w.dma_k(lk0, 0);
  w.dma_v(lv0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  wg_barrier();
  // step j (PH = j % 2): tile j in stage PH; the DMA of tile j+1 into the
  // other stage (read in step j-1, which every wave has left at the
  // barrier); a wave past its last visible tile keeps issuing its DMA share
  // and meeting the barriers
  auto step = [&](auto ph, int j) {
    constexpr int PH = decltype(ph)::value;
    if (j + 1 < ntiles) {
      w.dma_k(PH ? lk0 : lk1, j + 1);
      w.dma_v(PH ? lv0 : lv1, j + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (j < nw) {
      w.qk(s, PH ? lk1 : lk0);
      W::qk_schedule();
      const int kv0 = j * W::BN;
      if (w.needs_mask(kv0)) w.mask(s, kv0);
      const float hist = w.softmax_max(s);
      w.rescale(j, hist);
      w.softmax_exp(s, p);
      w.pv(p, PH ? lv1 : lv0);
      W::pv_schedule();
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

// ------------------------------------------------------------------- host

// Kernel choice: at D = 64 without the causal mask, the four-waves-per-SIMD
// kernel where the ping-pong kernel would run; else the ping-pong kernel
// when its 256-row tiles give at least one work-group per compute unit;
// else the four-wave kernel when its
// 128-row tiles do, or at D = 128, or for sequences under kSplitMinKeys
// (four KV tiles: there the key-split kernel's merge costs more than the
// shorter chain saves); else the key-split kernel (64-row tiles, four
// groups splitting the keys).
constexpr long long kPingPongMinGroups = 256;
constexpr long long kFourWaveMinGroups = 256;
constexpr int kSplitMinKeys = 256;

// Kernel variants (the diagnostic entry point can force one; 3, 4 and 6 are
// retired kernel numbers)
enum Variant { kAuto = 0, kFourWave = 1, kPingPong = 2, kPersistent = 5, kSplit = 7, kOcc4 = 8 };

template <int D> static inline bool use_pingpong(int BH, int S, int variant) {
  if (variant == kFourWave || variant == kSplit || variant == kOcc4) return false;
  if (variant == kPingPong || variant == kPersistent) return true;
  return (long long)num_q_tiles(S, Cfg8<D>::BM) * BH >= kPingPongMinGroups;
}
// (checked first)
template <int D, bool CAUSAL> static inline bool use_occ4(int BH, int S, int variant) {
  if (D != 64) return false;
  if (variant == kOcc4) return true;
  return variant == kAuto && !CAUSAL && use_pingpong<D>(BH, S, kAuto);
}
// (with the ping-pong kernel ruled out)
template <int D> static inline bool use_split(int BH, int S, int variant) {
  if (D != 64 || variant == kFourWave) return false;
  if (variant == kSplit) return true;
  return S >= kSplitMinKeys && (long long)num_q_tiles(S, Cfg4<D>::BM) * BH < kFourWaveMinGroups;
}

// Work-groups of the persistent kernel: one per CU of the current device,
// rounded down to a multiple of the 8 XCDs.
static inline int persistent_groups() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus / 8 * 8;
}

// The work items of a launch with query tiles of BM rows (P.nqt, P.items,
// P.compact): every (Q tile, sequence, head), or for a variable-length batch
// of at most kCompactMaxSeqs sequences only the tiles within the sequences,
// up to the bound varlen_cap (fa_layout.h) when that is smaller.
template <int BM> static inline void set_items(Problem& P) {
  P.nqt = num_q_tiles(P.Sq, BM);
  const long long full = (long long)P.nqt * P.B * P.H;  // below 2^31 (validated)
  P.items = (int)full;
  P.compact = 0;
  if (P.cuq && P.B <= kCompactMaxSeqs) {
    const long long cap = varlen_cap(P.totq, P.B, P.nqt, BM) * P.H;
    if (cap < full) {
      P.items = (int)cap;
      P.compact = 1;
    }
  }
}

// One launch of the kernel `variant` selects for a filled, validated Problem.
template <typename T, int D, bool CAUSAL, int THR, bool DIAG>
static int launch_one(Problem P, hipStream_t stream, int variant) {
  const int BH = P.B * P.H;
  if (DIAG && variant == kPersistent) {
    if constexpr (DIAG) {
      set_items<Cfg8<D>::BM>(P);
      const int g = persistent_groups();
      if (g <= 0) return FA_ERR_HIP;
      hipLaunchKernelGGL((fa_fwd_pp_persist<T, D, CAUSAL, THR, DIAG>), dim3((unsigned)g),
                         dim3(Cfg8<D>::threads), 0, stream, P);
    }
  } else if (use_occ4<D, CAUSAL>(BH, P.Sq, variant)) {
    // the product library runs it without the causal mask only
    if constexpr (D == 64 && (!CAUSAL || DIAG)) {
      set_items<CfgOcc4<D>::BM>(P);
      hipLaunchKernelGGL((fa_fwd_occ4<T, D, CAUSAL, THR, DIAG>),
                         dim3((unsigned)P.items), dim3(CfgOcc4<D>::threads), 0,
                         stream, P);
    }
  } else if (use_pingpong<D>(BH, P.Sq, variant)) {
    set_items<Cfg8<D>::BM>(P);
    hipLaunchKernelGGL((fa_fwd_pp<T, D, CAUSAL, THR, DIAG>), dim3((unsigned)P.items),
                       dim3(Cfg8<D>::threads), 0, stream, P);
  } else if (use_split<D>(BH, P.Sq, variant)) {
    if constexpr (D == 64) {
      set_items<CfgSplit<D>::BM>(P);
      hipLaunchKernelGGL((fa_fwd_split<T, D, CAUSAL, THR, DIAG>), dim3((unsigned)P.items),
                         dim3(CfgSplit<D>::threads * kSplitGroups), 0, stream, P);
    }
  } else {
    set_items<Cfg4<D>::BM>(P);
    // Unused dynamic LDS sets how many work-groups share a CU: at D = 128
    // 17 KiB (81 KiB, one per CU), at D = 64 22 KiB (54 KiB, at most two).
    // Timed against no padding (two per CU at D = 128): B=1 H=48 S=1024
    // causal 29.4 against 32.5 us, H=63 32.8 against 31.3, the other shapes
    // this kernel serves within 1%. (Two per CU once returned wrong rows; the
    // cause was the store-data reuse that store_rows in fa_wave.h now avoids,
    // and with that fix neither form returns a wrong row.)
    const unsigned lds_pad = D == 128 ? 17u * 1024u : 22u * 1024u;
    hipLaunchKernelGGL((fa_fwd_k4<T, D, CAUSAL, THR, DIAG>), dim3((unsigned)P.items),
                       dim3(Cfg4<D>::threads), lds_pad, stream, P);
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

}  // namespace fa
