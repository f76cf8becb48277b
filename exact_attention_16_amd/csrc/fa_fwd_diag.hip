// Diagnostic library of the attention forward (libfa_fwd_diag.so): the
// production kernels of fa_kernels.h instantiated once more with a
// rescale-event counter and with the lag threshold of the online softmax at
// 8 (the production setting) or 0 (rescale on every increase of the running
// max), and the persistent form of the ping-pong kernel. Tests load it
// beside the product library to count how often the conditional rescale
// fires (hjcheng0602.cn, "Flash Attention CUDA Kernel 优化 ... G6", section
// "V41: Conditional Scale") and to force a kernel choice. The argument checks
// are the product library's (fa_validate.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fa_fwd.h"
#include "../../include/fa_fwd_diag.h"
#include "fa_kernels.h"
#include "fa_validate.h"

extern "C" {

int fa_fwd_diag(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int S, int D, int causal, float scale, hipStream_t stream, int dtype,
                int threshold_log2, int variant, unsigned long long* rescale_events) {
  fa::Problem P;
  bool empty;
  const int r = fa::make_dense(&P, q, k, v, o, lse, B, H, S, D, causal, scale, dtype, &empty);
  if (r != FA_OK) return r;
  if (threshold_log2 != 0 && threshold_log2 != 8) return FA_ERR_ARG;
  if (variant != fa::kAuto && variant != fa::kFourWave && variant != fa::kPingPong &&
      variant != fa::kPersistent && !((variant == fa::kSplit || variant == fa::kOcc4) && D == 64))
    return FA_ERR_ARG;
  if (!rescale_events) return FA_ERR_NULL;
  if (((uintptr_t)rescale_events & 7) != 0) return FA_ERR_ALIGN;
  if (empty) return FA_OK;
  P.events = rescale_events;
  const bool bf = dtype == FA_BF16;
  if (threshold_log2 == 8)
    return bf ? fa::launch<__bf16, 8, true>(P, D, causal, stream, variant)
              : fa::launch<_Float16, 8, true>(P, D, causal, stream, variant);
  return bf ? fa::launch<__bf16, 0, true>(P, D, causal, stream, variant)
            : fa::launch<_Float16, 0, true>(P, D, causal, stream, variant);
}

}  // extern "C"
