/*
 * fa_probe.h -- issue-rate probes of one gfx950 compute unit.
 *
 * Not part of the attention library: fa_probe_run lives in libfa_probe.so,
 * built beside libfa_fwd.so, and is run by exact_attention_16_amd.probe.
 * It measures the rates the kernels' schedules are designed around: how
 * often one SIMD issues plain vector instructions (v_fma_f32),
 * transcendentals (v_exp_f32) and matrix instructions
 * (v_mfma_f32_32x32x16_bf16), alone and side by side, as a function of how
 * many waves share the SIMD. The method is the one P3 (blog.hotdry.top,
 * "FlashAttention的Triton性能考古学", section "MIO 瓶颈与 Tensor Core 挑战")
 * applies to the softmax's special-function work: measure the unit's issue
 * rate before scheduling work around it.
 *
 * Status codes are those of fa_fwd.h.
 */
#ifndef FA_PROBE_H
#define FA_PROBE_H

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

/* instruction streams; each runs `iters` blocks of a fixed content */
enum {
  FA_PROBE_NONE = 0,     /* the wave exits at once                            */
  FA_PROBE_FMA = 1,      /* 32 v_fma_f32 over 8 independent chains            */
  FA_PROBE_EXP = 2,      /* 32 v_exp_f32 over 8 independent chains            */
  FA_PROBE_MFMA = 3,     /* 16 v_mfma_f32_32x32x16_bf16 over 4 independent
                            accumulators                                      */
  FA_PROBE_MIX = 4,      /* 32 v_exp_f32 over 8 chains, each followed by `mix`
                            v_fma_f32 of 8 other independent chains           */
  FA_PROBE_MFMA_DEP = 5  /* 16 v_mfma_f32_32x32x16_bf16 on one accumulator,
                            each taking the one before as its addend          */
};

/*
 * fa_probe_run -- one work-group of 4 * waves_per_simd waves on one compute
 * unit. Waves are numbered from 0; the hardware places waves 0-3 on four
 * different SIMDs and wave w on the SIMD of wave w mod 4 (the kernel records
 * where each wave ran, so the caller can check). Waves 0-3 (one per SIMD)
 * run stream a for iters_a blocks; the other waves run
 * stream b for iters_b blocks. All waves start after one work-group barrier.
 *   waves_per_simd  1 to 4
 *   a, b            FA_PROBE_*, not both FA_PROBE_NONE
 *   iters_a/b       1 to 1 << 20 blocks (ignored for FA_PROBE_NONE)
 *   mix             0 to 8 (FA_PROBE_MIX only)
 *   out             device array of 3 * 4 * waves_per_simd uint64, owned by
 *                   the caller; for wave w: out[3w] = its shader-clock cycles
 *                   (s_memtime) from the barrier to its last block (0 for
 *                   a wave with no stream), out[3w+1]
 *                   = its SIMD (HW_ID bits 5:4), out[3w+2] = its CU id (HW_ID
 *                   bits 11:8).
 *   stream          the HIP stream the launch is enqueued on.
 * Errors: FA_ERR_ARG for a value out of range, FA_ERR_NULL for a NULL out,
 * FA_ERR_ALIGN for an out not 8-byte aligned, FA_ERR_HIP for a failed launch.
 * Nothing is launched when an argument is rejected.
 */
int fa_probe_run(int a, int iters_a, int b, int iters_b, int waves_per_simd, int mix,
                 unsigned long long* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H */
