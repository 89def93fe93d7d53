// pkv_internal.h -- launchers shared between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"

namespace pkv {

bool vector_supported(int q_dtype, int kv_dtype, int head_dim, int block_size);
bool mfma_supported(int q_dtype, int kv_dtype, int head_dim, int block_size, int group);

hipError_t launch_attention_vector(const AttnParams& p, int q_dtype, int kv_dtype, int head_dim, int block_size,
                                   hipStream_t stream);
hipError_t launch_attention_mfma(const AttnParams& p, int q_dtype, int head_dim, hipStream_t stream);
hipError_t launch_attention_reduce(const ReduceParams& p, int out_dtype, int head_dim, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                    const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                    int head_dim, int block_size, int num_blocks, int src_dtype, int kv_dtype,
                                    float k_scale, float v_scale, hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int num_pairs,
                              int64_t block_bytes, int num_blocks, hipStream_t stream);

}  // namespace pkv
