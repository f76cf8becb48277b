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
  FA_ERR_ARG = -8,         /* causal not 0/1 (or a bad argument of the
                              diagnostic library's fa_fwd_diag)             */
  FA_ERR_LAYOUT = -9       /* a stride is negative, a row stride < D, or an
                              output's rows overlap each other             */
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
 *            offsets), H*S*D <= 2^40 and B*H*S*D <= 2^40,
 *            B*H*ceil(S/128) < 2^31; beyond them FA_ERR_DIM.
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
 * fa_fwd_strided -- fa_fwd over strided tensors, with separate query and key
 * lengths. The kernel signature of "CUDA手写masked multi-head attention性能
 * 优化实战" (section 4.2) takes per-tensor strides; this entry point accepts
 * any layout whose rows are D contiguous elements.
 *
 *   q, o     device, element (b, h, i, d) at base + b*sb + h*sh + i*ss + d,
 *            i < Sq
 *   k, v     device, element (b, h, j, d) likewise, j < Sk
 *   lse      device float, element (b, h, i) at lse + b*lb + h*lh + i
 *   strides  host array of 14 element strides, read during the call:
 *            q (sb, sh, ss), k (sb, sh, ss), v (sb, sh, ss), o (sb, sh, ss),
 *            lse (lb, lh). All >= 0. The 12 tensor strides are multiples
 *            of 8 (every row 16-byte aligned) and each row stride is >= D.
 *   Sq, Sk   >= 0. B*H*Sq == 0 is a no-op returning FA_OK.
 *   causal   1: key j visible to query i iff j <= i + (Sk - Sq), the mask
 *            aligned to the last query and the last key (with Sq == Sk,
 *            j <= i). A query that sees no key gets O = 0 and lse = -inf.
 *   other arguments as for fa_fwd.
 *
 * Limits: Sq*ss*2 and Sk*ss*2 < 2^31 for each tensor's row stride ss (one
 * (sequence, head) addressed with 32-bit offsets); every stride <= 2^40
 * elements, and each tensor's span at most 2^40 elements (FA_ERR_DIM;
 * checked before any arithmetic that could overflow). Errors: negative or
 * overlapping-output strides FA_ERR_LAYOUT; strides not multiples of 8
 * FA_ERR_ALIGN; o or lse sharing bytes with q, k, v or each other (by the
 * byte ranges the strides span) FA_ERR_ALIAS; the rest as for fa_fwd.
 * k and v may alias each other or q (all read only); a zero head stride on
 * k and v shares one key/value head across all query heads.
 */
int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Sq, int Sk, int D, int causal, float scale,
                   hipStream_t stream, int dtype, const long long* strides);

/*
 * fa_fwd_varlen -- attention forward over B sequences of different lengths
 * packed along one token axis: dynamic sequence lengths without padding
 * (the shape-dependent dispatch of "CUDA手写masked multi-head attention性能
 * 优化实战", section 6.3, done here with per-sequence offsets in one launch).
 *
 *   cu_seqlens_q, cu_seqlens_k   device int arrays of B+1 token offsets,
 *            non-decreasing: sequence b has query tokens cu_seqlens_q[b] ..
 *            cu_seqlens_q[b+1]-1 and key tokens cu_seqlens_k[b] ..
 *            cu_seqlens_k[b+1]-1. Read by the kernel; owned by the caller.
 *            Offsets out of order are not an error the call can return: no
 *            memory outside the tensors is touched either way, and with at
 *            most 256 sequences, cu_seqlens_q out of order computes nothing
 *            and sets every row of o and lse to NaN.
 *   max_seqlen_q, max_seqlen_k   upper bounds of the lengths. A sequence
 *            longer than max_seqlen_q, or with more keys than max_seqlen_k,
 *            is not computed: all its rows get NaN in o and lse (the other
 *            sequences are unaffected).
 *   Work-groups: one per query tile of each (sequence, head). With at most
 *            256 sequences the launch holds H * min(B * ceil(max_seqlen_q /
 *            BM), floor((total_q + B * (BM - 1)) / BM)) work-groups (BM the
 *            kernel's query rows per tile; the second term bounds the tiles
 *            the sequences can have, since their lengths are on the device),
 *            and each finds its (sequence, tile, head) from the offsets, so
 *            no work-group is spent on tiles past a sequence's end; with more
 *            sequences, H * B * ceil(max_seqlen_q / BM).
 *   total_q, total_k   token rows q/o/lse and k/v hold; the kernel clamps
 *            every offset to them, so a bad offset array cannot address
 *            memory outside the tensors.
 *   q, o     element (token t, head h, d) at base + t*ss + h*sh + d
 *   k, v     likewise, t < total_k
 *   lse      float, element (h, t) at lse + h*lh + t
 *   strides  host array of 9 element strides: q (sh, ss), k (sh, ss),
 *            v (sh, ss), o (sh, ss), lse (lh); for the common packed layout
 *            [total, H, D]: sh = D, ss = H*D, and lh = total_q.
 *   causal   as for fa_fwd_strided, per sequence (j <= i + Lk - Lq).
 *   other arguments, limits (with the maxima as Sq, Sk) and errors as for
 *   fa_fwd_strided; misaligned cu_seqlens pointers FA_ERR_ALIGN.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H,
                  int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                  int D, int causal, float scale, hipStream_t stream, int dtype,
                  const long long* strides);

/*
 * fa_fwd_tile -- the tile shape fa_fwd uses for a call with (B, H, S,
 * causal) at head dimension D: query rows per work-group, keys per KV tile,
 * threads per work-group, and the number of work-groups launched. fa_fwd
 * runs, at D = 64 without the causal mask, the four-waves-per-SIMD kernel
 * (256 rows, 64 keys, 512 threads, two work-groups per CU) when
 * B*H*ceil(S/256) >= 256; else the eight-wave ping-pong kernel (256 rows; 96
 * keys per tile at D=128, 128 at D=64) when B*H*ceil(S/256) >= 256; else the
 * four-wave kernel (128 rows, 64 keys) when B*H*ceil(S/128) >= 256, D = 128
 * or S < 256; else (D = 64) the key-split kernel (64 rows, 64 keys, 512
 * threads: four groups of two waves, each taking every fourth KV tile,
 * merged at the end). The same choice, with S the query length, applies to
 * fa_fwd_strided and fa_fwd_varlen.
 * Any output pointer may be NULL. Returns FA_ERR_UNSUPPORTED for D not in
 * {64, 128}, FA_ERR_ARG for causal not 0 or 1.
 */
int fa_fwd_tile(int D, int B, int H, int S, int causal, int* block_m, int* block_n,
                int* threads, long long* work_groups);

/*
 * fa_fwd_kt -- fa_fwd with K given transposed: "FlashAttention的Triton性能
 * 考古学" (hotdry.top, section "解决方案：预转置 K 矩阵") stores K^T so that
 * the Q K^T tiles read contiguous memory.
 *
 *   kt       device, [B,H,D,S] of `dtype` (for each (b, h), D rows of S
 *            keys: element (b, h, d, j) at kt + ((b*H + h)*D + d)*S + j),
 *            16-byte aligned, read only
 *   S        a multiple of 8 (each d row starts 16-byte aligned), else
 *            FA_ERR_ALIGN; B*H*S == 0 is a no-op
 *   q, v, o, lse and the other arguments as for fa_fwd (q, v, o [B,H,S,D]).
 *
 * The result equals fa_fwd's on the same values (up to the rounding order
 * of the row sums: the kernel uses 64-key tiles at D = 128 and 128-key
 * tiles at D = 64). Errors as for fa_fwd; o or lse overlapping kt:
 * FA_ERR_ALIAS.
 */
int fa_fwd_kt(const void* q, const void* kt, const void* v, void* o, float* lse,
              int B, int H, int S, int D, int causal, float scale,
              hipStream_t stream, int dtype);

/*
 * fa_fwd_fp8 -- fa_fwd on 8-bit float inputs with one descale per tensor:
 * the FP8 support that "FlashAttention的Triton性能考古学" (hotdry.top,
 * section "架构感知优化策略") lists for newer GPUs.
 *
 *   q, k, v  device, [B,H,S,D] E4M3 codes (OCP 8-bit float: 1 sign, 4
 *            exponent bits with bias 7, 3 mantissa bits; no infinities,
 *            S.1111.111 is NaN), one byte per element, 16-byte aligned
 *   o        device, [B,H,S,D] bf16, 16-byte aligned, written
 *   lse      device, [B,H,S] float, 16-byte aligned, written
 *   descale_q, descale_k, descale_v
 *            the value of a code x of q is decode(x) * descale_q, and
 *            likewise for k and v; finite and > 0. The output is attention
 *            of those values: o and lse as fa_fwd defines them with
 *            x_ij = scale * descale_q * descale_k * <q_i, k_j>.
 *   D        64 or 128 (FA_ERR_UNSUPPORTED otherwise)
 *   other arguments as for fa_fwd; any S >= 1; B*H*S == 0 is a no-op.
 *
 * Precision: the logits and the row sums are exact products accumulated in
 * fp32, as in fa_fwd; the probabilities are rounded to E4M3 (after scaling
 * by a power of two that keeps them in (0, 256]) before the P V product, so
 * O carries up to 2^-4 relative error per probability, the rounding of the
 * 8-bit matrix units; lse is not affected.
 *
 * Errors: a descale or scale not finite and > 0, or a product
 * scale * descale_q * descale_k * log2(e) outside the normal float range:
 * FA_ERR_SCALE; o or lse sharing bytes with q, k, v or each other:
 * FA_ERR_ALIAS; S*D*2 >= 2^31 or B*H*S*D > 2^40: FA_ERR_DIM; the rest as
 * for fa_fwd.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int S, int D, int causal, float scale,
               float descale_q, float descale_k, float descale_v, hipStream_t stream);

/* Static description of a status code (never NULL). */
const char* fa_strerror(int status);

/* Library version as major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_FWD_H */
