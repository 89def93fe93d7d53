// pkv_internal.h -- launchers shared between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pkv.h"
#include "pkv_device.h"

namespace pkv {

// Host-side helpers of the C-ABI layer.
inline int dtype_bytes(int dt) {
  switch (dt) {
    case PKV_F32: return 4;
    case PKV_F16: case PKV_BF16: return 2;
    case PKV_FP8_E4M3: case PKV_FP8_E5M2: return 1;
  }
  return 0;
}
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool good_scale(float s) { return isfinite(s) && s > 0.f; }
inline int launch_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH; }

bool vector_supported(int q_dtype, int kv_dtype, int head_dim, int block_size);
bool mfma_supported(int q_dtype, int kv_dtype, int head_dim, int block_size, int group);

hipError_t launch_attention_vector(const AttnParams& p, int q_dtype, int kv_dtype, int head_dim, int block_size,
                                   hipStream_t stream);
hipError_t launch_attention_mfma(const AttnParams& p, int q_dtype, int kv_dtype, int head_dim, hipStream_t stream);
// the same launches for decode with append (p.new_k set): separate kernels
hipError_t launch_attention_vector_append(const AttnParams& p, int q_dtype, int kv_dtype, int head_dim,
                                          int block_size, hipStream_t stream);
hipError_t launch_attention_mfma_append(const AttnParams& p, int q_dtype, int kv_dtype, int head_dim,
                                        hipStream_t stream);
// decode over groups of sequences sharing leading blocks (attn_shared.hip)
bool shared_supported(int q_dtype, int kv_dtype, int head_dim, int block_size);
hipError_t launch_attention_shared(const AttnParams& p, int q_dtype, int kv_dtype, int head_dim, bool append,
                                   hipStream_t stream);
hipError_t launch_attention_reduce(const ReduceParams& p, int out_dtype, int head_dim, hipStream_t stream);

bool prefill_supported(int q_dtype, int kv_dtype, int head_dim, int block_size);
int prefill_tile_rows();
hipError_t launch_prefill(const PrefillParams& p, int dtype, int head_dim, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                    const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                    int head_dim, int block_size, int num_blocks, int src_dtype, int kv_dtype,
                                    float k_scale, float v_scale, const float* k_scales, const float* v_scales,
                                    hipStream_t stream);
hipError_t launch_copy_blocks(const void* src_k, const void* src_v, int src_blocks, void* dst_k, void* dst_v,
                              int dst_blocks, const int64_t* pairs, int num_pairs, int64_t block_bytes,
                              hipStream_t stream);

}  // namespace pkv
