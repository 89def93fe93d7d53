// attn_mfma.hip -- the plain decode kernels of the matrix-core family for
// grouped-query heads (the kernel body and its layout are described in
// attn_mfma.h).
#include "attn_mfma.h"
#include "pkv_internal.h"

namespace pkv {

bool mfma_supported(int q_dtype, int kv_dtype, int d, int bs, int group) {
  return (q_dtype == F16::kId || q_dtype == BF16::kId) &&
         (kv_dtype == q_dtype || kv_dtype == FP8::kId || kv_dtype == BF8::kId) && (d == 128 || d == 256) &&
         bs == 16 && group >= 2 && group <= 16;
}

hipError_t launch_attention_mfma(const AttnParams& p, int q_dtype, int kv_dtype, int d, hipStream_t stream) {
  return launch_mfma_family<false>(p, q_dtype, kv_dtype, d, stream);
}

}  // namespace pkv
