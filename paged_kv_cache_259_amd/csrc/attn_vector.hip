// attn_vector.hip -- the plain decode kernels of the vector family (no
// matrix cores; the kernel body and its layout are described in attn_vector.h).
#include "attn_vector.h"
#include "pkv_internal.h"

namespace pkv {

bool vector_supported(int q_dtype, int kv_dtype, int d, int bs) {
  if (d != 64 && d != 128 && d != 256) return false;
  if (bs != 8 && bs != 16 && bs != 32) return false;
  int kv_bytes;
  if (q_dtype == 0 && kv_dtype == 0) kv_bytes = 4;
  else if ((q_dtype == 1 || q_dtype == 2) && kv_dtype == q_dtype) kv_bytes = 2;
  else if ((q_dtype == 1 || q_dtype == 2) && (kv_dtype == 3 || kv_dtype == 4)) kv_bytes = 1;
  else return false;
  const int lpr = d * kv_bytes / 16;
  const int rpw = 64 / lpr;
  return lpr >= 1 && lpr <= 64 && bs % rpw == 0 && bs / rpw <= 16;
}

hipError_t launch_attention_vector(const AttnParams& p, int q_dtype, int kv_dtype, int d, int bs, hipStream_t stream) {
  return launch_vector_family<false>(p, q_dtype, kv_dtype, d, bs, stream);
}

}  // namespace pkv
