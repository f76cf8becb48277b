// Issue-rate probes of one gfx950 compute unit (include/fa_probe.h): each
// wave of one work-group runs a fixed instruction stream between two reads
// of the shader clock, and reports its cycles and where it ran. Built into
// its own library; the attention kernels do not use it.
//
// The vector streams are inline asm, so the instruction order is exactly
// the one stated (eight independent chains, so one chain's latency does not
// set the rate). The matrix streams use the compiler builtin, so the
// compiler inserts whatever wait states the hardware needs between
// dependent MFMAs. Nothing here reads or writes memory except the final
// per-wave record.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fa_fwd.h"
#include "../../include/fa_probe.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxWavesPerSimd = 4;
constexpr int kMaxIters = 1 << 20;

// A block is one asm statement of four rounds over eight independent chains
// (32 instructions), so the loop's own instructions are a small share.
#define FA_R8(I) I(0) I(1) I(2) I(3) I(4) I(5) I(6) I(7)
#define FA_R32(I) FA_R8(I) FA_R8(I) FA_R8(I) FA_R8(I)
#define FA_FMA_X(i) "v_fma_f32 %" #i ", %" #i ", %8, %9\n\t"
#define FA_EXP_E(i) "v_exp_f32 %" #i ", %" #i "\n\t"

// 32 v_fma_f32: x[i] = x[i] * m + c
__device__ __forceinline__ void fma32(float (&x)[8], float m, float c) {
  asm volatile(FA_R32(FA_FMA_X)
               : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]),
                 "+v"(x[6]), "+v"(x[7])
               : "v"(m), "v"(c));
}

// 32 v_exp_f32: e[i] = 2^e[i]
__device__ __forceinline__ void exp32(float (&e)[8]) {
  asm volatile(FA_R32(FA_EXP_E)
               : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]), "+v"(e[4]), "+v"(e[5]),
                 "+v"(e[6]), "+v"(e[7]));
}

// One mix block as a single asm statement (so no wait state is inserted
// inside it): four rounds of 8 v_exp_f32 on e[0..7], each followed by R
// v_fma_f32 on x[0..R-1]. No instruction reads a result of the one before
// it.
#define FA_EXP1(i) "v_exp_f32 %" #i ", %" #i "\n\t"
#define FA_FMA1(i) "v_fma_f32 %" #i ", %" #i ", %16, %17\n\t"
#define FA_F0 ""
#define FA_F1 FA_FMA1(8)
#define FA_F2 FA_F1 FA_FMA1(9)
#define FA_F3 FA_F2 FA_FMA1(10)
#define FA_F4 FA_F3 FA_FMA1(11)
#define FA_F5 FA_F4 FA_FMA1(12)
#define FA_F6 FA_F5 FA_FMA1(13)
#define FA_F7 FA_F6 FA_FMA1(14)
#define FA_F8 FA_F7 FA_FMA1(15)
#define FA_MIX8(F)                                                                             \
  FA_EXP1(0) F FA_EXP1(1) F FA_EXP1(2) F FA_EXP1(3) F FA_EXP1(4) F FA_EXP1(5) F FA_EXP1(6) F \
  FA_EXP1(7) F
#define FA_MIX(F) FA_MIX8(F) FA_MIX8(F) FA_MIX8(F) FA_MIX8(F)
#define FA_MIX_LOOP(F)                                                                   \
  for (int it = 0; it < iters; ++it)                                                     \
    asm volatile(FA_MIX(F)                                                               \
                 : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]), "+v"(e[4]), "+v"(e[5]), \
                   "+v"(e[6]), "+v"(e[7]), "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), \
                   "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7])                       \
                 : "v"(m), "v"(c))

__device__ __forceinline__ void mix_loop(int mix, int iters, float (&e)[8], float (&x)[8], float m,
                                         float c) {
  switch (mix) {
    case 0: FA_MIX_LOOP(FA_F0); break;
    case 1: FA_MIX_LOOP(FA_F1); break;
    case 2: FA_MIX_LOOP(FA_F2); break;
    case 3: FA_MIX_LOOP(FA_F3); break;
    case 4: FA_MIX_LOOP(FA_F4); break;
    case 5: FA_MIX_LOOP(FA_F5); break;
    case 6: FA_MIX_LOOP(FA_F6); break;
    case 7: FA_MIX_LOOP(FA_F7); break;
    default: FA_MIX_LOOP(FA_F8); break;
  }
}

__device__ __forceinline__ float run_stream(int kind, int iters, int mix, float seed) {
  float x[8], e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = seed + (float)i;
    e[i] = -seed - (float)i;  // 2^-... stays finite and small
  }
  const float m = 0.999f, c = 1e-3f * seed;
  float out = 0.f;
  if (kind == FA_PROBE_FMA) {
    for (int it = 0; it < iters; ++it) fma32(x, m, c);
  } else if (kind == FA_PROBE_EXP) {
    for (int it = 0; it < iters; ++it) exp32(e);
  } else if (kind == FA_PROBE_MFMA || kind == FA_PROBE_MFMA_DEP) {
    const u32x4 a = {__float_as_uint(seed), 1u, 2u, 3u};
    const u32x4 b = {__float_as_uint(c), 3u, 2u, 1u};
    f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
    const bf16x8 av = __builtin_bit_cast(bf16x8, a), bv = __builtin_bit_cast(bf16x8, b);
    if (kind == FA_PROBE_MFMA) {
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc1, 0, 0, 0);
          acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc2, 0, 0, 0);
          acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc3, 0, 0, 0);
        }
      }
    } else {
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc0, 0, 0, 0);
      }
    }
    out = acc0[0] + acc1[1] + acc2[2] + acc3[3];
  } else if (kind == FA_PROBE_MIX) {
    mix_loop(mix, iters, e, x, m, c);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) out += x[i] + e[i];
  return out;
}

__global__ void __launch_bounds__(64 * 4 * kMaxWavesPerSimd)
probe_kernel(int a, int iters_a, int b, int iters_b, int mix, unsigned long long* out) {
  const int w = (int)(threadIdx.x >> 6);
  const bool first = w < 4;
  const int kind = __builtin_amdgcn_readfirstlane(first ? a : b);
  const int iters = __builtin_amdgcn_readfirstlane(first ? iters_a : iters_b);
  unsigned hw;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
  const float seed = (float)(threadIdx.x & 63) * 1e-3f;
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const float r = run_stream(kind, iters, mix, seed);
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  if ((threadIdx.x & 63) == 0) {
    out[3 * w] = kind == FA_PROBE_NONE ? 0 : t1 - t0;
    out[3 * w + 1] = (hw >> 4) & 3u;
    out[3 * w + 2] = (hw >> 8) & 15u;
  }
  // keeps the streams' results live; a value the streams never produce
  if (r == 1234.5f && (threadIdx.x & 63) == 1) out[3 * w] = 0;
}

bool stream_ok(int kind) { return kind >= FA_PROBE_NONE && kind <= FA_PROBE_MFMA_DEP; }

}  // namespace

extern "C" int fa_probe_run(int a, int iters_a, int b, int iters_b, int waves_per_simd, int mix,
                            unsigned long long* out, hipStream_t stream) {
  if (waves_per_simd < 1 || waves_per_simd > kMaxWavesPerSimd) return FA_ERR_ARG;
  if (!stream_ok(a) || !stream_ok(b) || (a == FA_PROBE_NONE && b == FA_PROBE_NONE))
    return FA_ERR_ARG;
  if (a != FA_PROBE_NONE && (iters_a < 1 || iters_a > kMaxIters)) return FA_ERR_ARG;
  if (b != FA_PROBE_NONE && (iters_b < 1 || iters_b > kMaxIters)) return FA_ERR_ARG;
  if (mix < 0 || mix > 8) return FA_ERR_ARG;
  if (!out) return FA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(out) % 8 != 0) return FA_ERR_ALIGN;
  hipLaunchKernelGGL(probe_kernel, dim3(1), dim3(64 * 4 * waves_per_simd), 0, stream, a,
                     a == FA_PROBE_NONE ? 0 : iters_a, b, b == FA_PROBE_NONE ? 0 : iters_b, mix,
                     out);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}
