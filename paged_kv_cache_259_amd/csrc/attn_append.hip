// attn_append.hip -- the decode-with-append kernels of both attention families:
// the same bodies as attn_vector.hip and attn_mfma.hip, where the wave that will
// read a sequence's last block first writes that sequence's new K/V row into its
// slot (append_new_row in pkv_device.h).  Separate kernels, so the plain decode
// carries no append code and a kernel trace tells the two launches apart.
#include "attn_mfma.h"
#include "attn_vector.h"
#include "pkv_internal.h"

namespace pkv {

hipError_t launch_attention_vector_append(const AttnParams& p, int q_dtype, int kv_dtype, int d, int bs,
                                          hipStream_t stream) {
  return launch_vector_family<true>(p, q_dtype, kv_dtype, d, bs, stream);
}

hipError_t launch_attention_mfma_append(const AttnParams& p, int q_dtype, int kv_dtype, int d, hipStream_t stream) {
  return launch_mfma_family<true>(p, q_dtype, kv_dtype, d, stream);
}

}  // namespace pkv
