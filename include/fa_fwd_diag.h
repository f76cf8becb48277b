/*
 * fa_fwd_diag.h -- test hook of the MI355X (gfx950) attention forward.
 *
 * Not part of the product library: fa_fwd_diag lives in the separate
 * diagnostic library libfa_fwd_diag.so, built beside libfa_fwd.so, which
 * instantiates the same kernels once more with a rescale-event counter. It
 * exists so that tests can count how often the conditional rescale of the
 * online softmax fires (the running max allowed to lag by 8 in log2 units
 * before the accumulator is rescaled: hjcheng0602.cn, "Flash Attention CUDA
 * Kernel 优化 ... G6", section "V41: Conditional Scale"), compare it with
 * the eager rule (lag 0), and force a kernel choice.
 *
 * Status codes, layouts, ownership and error behaviour are those of fa_fwd
 * (fa_fwd.h).
 */
#ifndef FA_FWD_DIAG_H
#define FA_FWD_DIAG_H

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fa_fwd_diag -- fa_fwd (same arguments, same result) with:
 *   threshold_log2   how far (log2 units of the scaled logit) the running
 *                    max may lag before the accumulator is rescaled:
 *                    8 (the production setting) or 0 (rescale on every
 *                    increase, the eager rule).
 *   variant          which kernel runs: 0 = the one fa_fwd picks for this
 *                    shape, 1 = the four-wave kernel (128 query rows per
 *                    work-group), 2 = the eight-wave ping-pong kernel (256
 *                    rows), 5 = the ping-pong kernel in persistent form (one
 *                    work-group per CU of the current device, rounded down to
 *                    a multiple of 8, each running query tiles in turn), 7 =
 *                    the key-split kernel (D = 64 only: 64 query rows per
 *                    work-group, four groups of two waves each taking every
 *                    fourth KV tile, merged at the end), 8 = the
 *                    four-waves-per-SIMD kernel (D = 64 only: 256 query
 *                    rows, 64-key tiles, two work-groups per CU; fa_fwd
 *                    runs it without the causal mask, the test hook with
 *                    either). 3, 4 and 6 are retired kernel numbers
 *                    (FA_ERR_ARG). Every variant computes the same result to
 *                    rounding.
 *   rescale_events   device pointer to one unsigned 64-bit counter, owned by
 *                    the caller; the kernel atomically adds the number of
 *                    (query row, KV tile) pairs whose running max moved
 *                    after the row's first tile. Not cleared by the library.
 * Errors: those of fa_fwd; threshold_log2 not 0 or 8, or variant not 0, 1,
 * 2, 5, 7 or 8, or 7 or 8 with D = 128: FA_ERR_ARG; NULL rescale_events:
 * FA_ERR_NULL; rescale_events not 8-byte aligned: FA_ERR_ALIGN; the CU count
 * of the current device not readable (variant 5): FA_ERR_HIP.
 */
int fa_fwd_diag(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int S, int D, int causal, float scale,
                hipStream_t stream, int dtype, int threshold_log2, int variant,
                unsigned long long* rescale_events);

#ifdef __cplusplus
}
#endif

#endif /* FA_FWD_DIAG_H */
