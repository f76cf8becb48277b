/*
 * fa_fwd.h -- C ABI of the MI355X (gfx950) fused attention forward.
 *
 * The operation (one call = every (batch, head) of one batch of inputs):
 *
 *   for each b < B, h < H, query row i < S:
 *     x_ij   = scale * <q[b,h,i,:], k[b,h,j,:]>        for visible keys j
 *     o[b,h,i,:] = sum_j softmax_j(x_ij) * v[b,h,j,:]
 *     lse[b,h,i] = ln sum_j exp(x_ij)                   (natural log)
 *
 * where key j is visible to row i iff causal == 0 or j <= i (the lower
 * triangle; square, top-left aligned). This is exact attention
 * softmax(scale * Q K^T + mask) V as stated by xdnf.cn, "CUDA手写masked
 * multi-head attention性能优化实战", section 3.1, computed the
 * FlashAttention way: Q tile resident, K/V tiles streamed, online softmax
 * with running max m and sum l, one normalisation at the end (hotdry.top,
 * "FlashAttention的Triton性能考古学", sections "核心算法回顾" and
 * "FlashAttention v2：循环重构与寄存器积累"), with the running max allowed to
 * lag by 8 in log2 units before the accumulator is rescaled (hjcheng0602.cn, "Flash
 * Attention CUDA Kernel 优化 ... G6", section "V41: Conditional Scale").
 * The row logsumexp output is this library's own addition; the pages do
 * not define it.
 *
 * Layouts: q, k, v, o are contiguous row-major [B, H, S, D] arrays of the
 * same 16-bit type (o is written in that type, rounded once to nearest
 * even from fp32); lse is a contiguous [B, H, S] fp32 array.
 *
 * Ownership: all pointers are DEVICE pointers owned by the caller. The
 * library never allocates, frees, synchronises, or changes the current
 * device; q, k, v are only read; o and lse are fully overwritten. Work is
 * enqueued on `stream` (NULL = the legacy default stream) and the call
 * returns without waiting for it.
 *
 * Errors: every entry point returns an fa_status_t. Arguments are checked
 * on the host before any HIP call, so the checks work without a GPU; a
 * failed check launches nothing. Launch failures reported by the HIP runtime
 * return FA_ERR_HIP. Faults during kernel execution surface at the caller's
 * next synchronisation, as usual for HIP. The library never prints, throws
 * across the ABI, or aborts. It keeps no mutable global state (re-entrant).
 */
#ifndef FA_FWD_H
#define FA_FWD_H

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. */
typedef enum { FA_F16 = 0, FA_BF16 = 1 } fa_dtype_t;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,        /* a required pointer is NULL                    */
  FA_ERR_DIM = -2,         /* B, H or S negative, or sizes too large        */
  FA_ERR_UNSUPPORTED = -3, /* D not 64 or 128, or unknown dtype             */
  FA_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned              */
  FA_ERR_SCALE = -5,       /* scale not finite or not > 0                   */
  FA_ERR_ALIAS = -6,       /* o or lse overlaps another buffer              */
  FA_ERR_HIP = -7,         /* the HIP runtime rejected the launch           */
  FA_ERR_ARG = -8          /* causal not 0/1, or a bad diagnostic argument  */
} fa_status_t;

/*
 * fa_fwd -- attention forward for all B*H heads.
 *
 *   q, k, v  device, [B,H,S,D] of `dtype`, 16-byte aligned, read only
 *   o        device, [B,H,S,D] of `dtype`, 16-byte aligned, written
 *   lse      device, [B,H,S] float, 16-byte aligned, written
 *   B, H, S  >= 0; B*H*S == 0 is a no-op returning FA_OK (pointers unused).
 *            Any S >= 1 is accepted (a ragged last tile is masked).
 *            Limits: S*D*2 < 2^31 (one head's K/V/O addressed with 32-bit
 *            offsets), B*H*S*D <= 2^40, B*H*ceil(S/128) < 2^31.
 *   D        head dimension, 64 or 128
 *   causal   0 = every key visible; 1 = key j visible to row i iff j <= i
 *   scale    multiplier of q.k; finite and > 0 (typically 1/sqrt(D)).
 *            The kernel folds it into its base-2 exponent and compares raw
 *            dot products, which needs scale > 0.
 *   stream   HIP stream the kernel is enqueued on
 *   dtype    FA_F16 or FA_BF16
 *
 * o and lse must not overlap q, k, v or each other (FA_ERR_ALIAS).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int S, int D, int causal, float scale,
           hipStream_t stream, int dtype);

/* fa_fwd with dtype fixed: exactly the argument list
 * (q, k, v, o, lse, B, H, S, D, causal, scale, stream). */
int fa_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int S, int D, int causal, float scale,
               hipStream_t stream);
int fa_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int S, int D, int causal, float scale,
                hipStream_t stream);

/*
 * fa_fwd_diag -- diagnostic variant of fa_fwd for tests.
 *
 * Same arguments and result as fa_fwd, plus:
 *   threshold_log2   how far (log2 units of the scaled logit) the running
 *                    max may lag before the accumulator is rescaled:
 *                    8 (the production setting) or 0 (rescale on every
 *                    increase, the eager FlashAttention-2 rule).
 *   rescale_events   device pointer to one unsigned 64-bit counter, owned
 *                    by the caller; the kernel atomically adds the number
 *                    of (query row, KV tile) pairs whose running max moved
 *                    after the row's first tile. Not cleared by the library.
 *   variant          which kernel runs: 0 = the one fa_fwd picks for this
 *                    shape, 1 = the four-wave kernel (128 query rows per
 *                    work-group), 2 = the eight-wave ping-pong kernel (256
 *                    rows), 3 = the four-wave kernel with two 32-row blocks
 *                    per wave (256 rows, 32-key tiles). Every variant
 *                    computes the same result, to rounding; the choice only
 *                    affects speed.
 * It runs separate, instrumented instantiations of the same kernels.
 * Invalid threshold_log2 or variant: FA_ERR_ARG; NULL rescale_events:
 * FA_ERR_NULL; rescale_events not 8-byte aligned: FA_ERR_ALIGN.
 */
int fa_fwd_diag(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int S, int D, int causal, float scale,
                hipStream_t stream, int dtype, int threshold_log2, int variant,
                unsigned long long* rescale_events);

/*
 * fa_fwd_tile -- the tile shape fa_fwd uses for a call with (B, H, S) at
 * head dimension D: query rows per work-group, keys per KV tile, threads per
 * work-group, and the number of work-groups launched. fa_fwd runs the
 * eight-wave kernel (256 rows; 64 keys per tile at D=128, 128 at D=64) when
 * B*H*ceil(S/256) >= 256, else the four-wave kernel (128 rows, 64 keys).
 * Any output pointer may be NULL. Returns FA_ERR_UNSUPPORTED for D not in
 * {64, 128}.
 */
int fa_fwd_tile(int D, int B, int H, int S, int* block_m, int* block_n,
                int* threads, long long* work_groups);

/* Static description of a status code (never NULL). */
const char* fa_strerror(int status);

/* Library version as major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_FWD_H */
