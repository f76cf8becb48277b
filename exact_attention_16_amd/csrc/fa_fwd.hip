// Fused attention forward for AMD Instinct MI355X (gfx950, CDNA4).
//
// Each wave owns 32 query rows of one (batch, head) for the whole kernel,
// with its Q rows held in registers as MFMA operands, and streams the K/V
// tiles of that head through LDS. Per KV tile j a wave computes
//   S(j) = K(j) Q^T          (v_mfma_f32_32x32x16, raw dot products in fp32)
//   softmax(S(j)) -> P(j)    (VALU: tile max, lagging base, exp2, row sum)
//   O^T += V(j)^T P(j)^T     (v_mfma_f32_32x32x16)
// and at the end normalises once and writes O and the row logsumexp.
//
// Data movement: K and V tiles go from HBM to LDS by buffer loads with the
// LDS bit (direct DMA, 16 bytes per lane; no staging registers, no VALU),
// whose range check zero-fills rows past the end of the sequence. K is read
// back as 16-byte S^T operand fragments (no transpose); V^T operand
// fragments come from the row-major V tile through ds_read_b64_tr_b16,
// which transposes in the LDS crossbar. Both tiles are XOR-swizzled per row
// so that the operand reads are free of bank conflicts.
//
// Softmax: base 2 with a lagging running base b per row (log2 units of the
// scaled logit). The tile max of the raw dot products is exchanged between
// the two lanes of a row with v_permlane32_swap; b moves only when the
// candidate exceeds b + THR, with history factor 2^(b_old - b_new); p =
// 2^(s*c - b) with c = scale*log2(e), so p <= 2^THR. Row sums accumulate the
// unrounded fp32 p; P is rounded once to the input type for the MFMA. The
// O rescale is skipped, wave-uniformly, unless a ballot finds a row with
// history < 1. Causal tiles wholly above the diagonal are never visited;
// only tiles crossing the diagonal or the ragged end compare indices.
//
// fa_fwd picks one of two kernels (fa_kernels.h), which overlap the matrix
// cores and the vector ALU differently:
//  * fa_fwd_pp (eight waves, 256 query rows; work-group body in
//    fa_pingpong.h): the waves form two groups whose slots alternate between
//    an MFMA phase (P(j-1).V(j-1) and K(j).Q^T) and a softmax phase, offset
//    by one slot, so each SIMD always holds one multiplying and one
//    exponentiating wave; K/V use three LDS stages, issued two tiles ahead.
//  * fa_fwd_k4 (four waves, 128 query rows), for grids too small to fill the
//    chip with 256-row tiles: each wave overlaps the next tile's K.Q^T (and,
//    at D=64, the previous tile's P.V) with its own current softmax; two LDS
//    stages.
// fa_fwd_kt runs the ping-pong body on a K given transposed ([D, S] per
// head), read like a V tile. The 8-bit kernel is in fa_fwd_fp8.hip. This
// file holds the host side of the product library: argument checks
// (fa_validate.h), the kernel choice and the C entry points.
//
// Method sources: exact attention softmax(QK^T/sqrt(d)+mask)V with a
// lower-triangle causal mask (xdnf.cn, "CUDA手写masked multi-head attention
// 性能优化实战", 3.1); tiling with running max/sum, v2 loop order, deferred
// normalisation and the (Q tile, head) grid (hotdry.top, "FlashAttention的
// Triton性能考古学", sections "核心算法回顾" and "FlashAttention v2：循环重构与
// 寄存器积累"); the conditional rescale with a lag of 8 and p in (0, 256], the
// warp-vote skip of the rescale, the rescale done by the softmax workers
// themselves, and issuing the next tile's Q.K^T ahead of the current P.V
// (hjcheng0602.cn, "Flash Attention CUDA Kernel 优化 ... G6", V39, V41, V44).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/fa_fwd.h"
#include "fa_kernels.h"
#include "fa_validate.h"

namespace fa {

template <typename T> static int launch_kt(Problem P, int D, int causal, hipStream_t st) {
  static_assert(CfgKT<64>::BM == CfgKT<128>::BM, "one query tile size for both head dims");
  P.nqt = num_q_tiles(P.Sq, CfgKT<128>::BM);
  P.items = P.nqt * P.B * P.H;
  const dim3 grid((unsigned)P.items), block(512);
  if (D == 64) {
    if (causal) hipLaunchKernelGGL((fa_fwd_pp_kt<T, 64, true>), grid, block, 0, st, P);
    else hipLaunchKernelGGL((fa_fwd_pp_kt<T, 64, false>), grid, block, 0, st, P);
  } else {
    if (causal) hipLaunchKernelGGL((fa_fwd_pp_kt<T, 128, true>), grid, block, 0, st, P);
    else hipLaunchKernelGGL((fa_fwd_pp_kt<T, 128, false>), grid, block, 0, st, P);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// production instantiations: threshold 8, no event counter, kernel by shape
static int launch_dtype(const Problem& P, int D, int causal, int dtype, hipStream_t st) {
  return dtype == FA_BF16 ? launch<__bf16, 8, false>(P, D, causal, st, kAuto)
                          : launch<_Float16, 8, false>(P, D, causal, st, kAuto);
}

// 8-bit inputs (fa_fwd_fp8.hip)
int launch_fp8(Problem P, int D, int causal, hipStream_t stream);

}  // namespace fa

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int S,
           int D, int causal, float scale, hipStream_t stream, int dtype) {
  fa::Problem P;
  bool empty;
  const int r = fa::make_dense(&P, q, k, v, o, lse, B, H, S, D, causal, scale, dtype, &empty);
  if (r != FA_OK || empty) return r;
  return fa::launch_dtype(P, D, causal, dtype, stream);
}

int fa_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int S, int D, int causal, float scale, hipStream_t stream) {
  return fa_fwd(q, k, v, o, lse, B, H, S, D, causal, scale, stream, FA_F16);
}

int fa_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int S, int D, int causal, float scale, hipStream_t stream) {
  return fa_fwd(q, k, v, o, lse, B, H, S, D, causal, scale, stream, FA_BF16);
}

int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int H, int Sq, int Sk, int D, int causal, float scale, hipStream_t stream,
                   int dtype, const long long* strides) {
  fa::Problem P;
  bool empty;
  const int r =
      fa::make_fixed(&P, q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale, dtype, strides, &empty);
  if (r != FA_OK || empty) return r;
  return fa::launch_dtype(P, D, causal, dtype, stream);
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H,
                  int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int D,
                  int causal, float scale, hipStream_t stream, int dtype,
                  const long long* strides) {
  fa::Problem P;
  bool empty;
  const int r = fa::make_varlen(&P, q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, H,
                                max_seqlen_q, max_seqlen_k, total_q, total_k, D, causal, scale,
                                dtype, strides, &empty);
  if (r != FA_OK || empty) return r;
  return fa::launch_dtype(P, D, causal, dtype, stream);
}

int fa_fwd_tile(int D, int B, int H, int S, int causal, int* block_m, int* block_n, int* threads,
                long long* work_groups) {
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  const int BH = (B < 0 || H < 0) ? 0 : B * H;
  const int SS = S < 0 ? 0 : S;
  const bool occ = D == 64 && (causal ? fa::use_occ4<64, true>(BH, SS, fa::kAuto)
                                      : fa::use_occ4<64, false>(BH, SS, fa::kAuto));
  const bool pp = !occ && (D == 64 ? fa::use_pingpong<64>(BH, SS, fa::kAuto)
                                   : fa::use_pingpong<128>(BH, SS, fa::kAuto));
  const bool split = !occ && !pp && D == 64 && fa::use_split<64>(BH, SS, fa::kAuto);
  const int bm = (occ || pp) ? 256 : (split ? 64 : 128);
  if (block_m) *block_m = bm;
  if (block_n) *block_n = pp ? (D == 64 ? fa::Cfg8<64>::BN : fa::Cfg8<128>::BN) : 64;
  if (threads) *threads = (occ || pp || split) ? 512 : 256;
  if (work_groups) *work_groups = (long long)BH * fa::num_q_tiles(SS, bm);
  return FA_OK;
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_DIM: return "B, H or S is negative or the sizes or strides exceed the supported limits";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension (D must be 64 or 128) or dtype";
    case FA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case FA_ERR_SCALE: return "scale must be finite and > 0";
    case FA_ERR_ALIAS: return "o or lse overlaps another buffer";
    case FA_ERR_HIP: return "the HIP runtime rejected the kernel launch";
    case FA_ERR_ARG: return "causal must be 0 or 1 (or a diagnostic argument is invalid)";
    case FA_ERR_LAYOUT: return "a stride is negative, a row stride is below D, or output rows overlap";
    default: return "unknown status";
  }
}

int fa_fwd_kt(const void* q, const void* kt, const void* v, void* o, float* lse, int B, int H,
              int S, int D, int causal, float scale, hipStream_t stream, int dtype) {
  fa::Problem P;
  bool empty;
  const int r = fa::make_kt(&P, q, kt, v, o, lse, B, H, S, D, causal, scale, dtype, &empty);
  if (r != FA_OK || empty) return r;
  return dtype == FA_BF16 ? fa::launch_kt<__bf16>(P, D, causal, stream)
                          : fa::launch_kt<_Float16>(P, D, causal, stream);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int S, int D, int causal, float scale, float descale_q, float descale_k,
               float descale_v, hipStream_t stream) {
  fa::Problem P;
  bool empty;
  const int r = fa::make_fp8(&P, q, k, v, o, lse, B, H, S, D, causal, scale, descale_q,
                             descale_k, descale_v, &empty);
  if (r != FA_OK || empty) return r;
  return fa::launch_fp8(P, D, causal, stream);
}

int fa_version(void) { return 500; }

}  // extern "C"
