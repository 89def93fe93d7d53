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
hipError_t launch_prefill(const PrefillParams& p, int dtype, int kv_dtype, int head_dim, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                    const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                    int head_dim, int block_size, int num_blocks, int src_dtype, int kv_dtype,
                                    float k_scale, float v_scale, const float* k_scales, const float* v_scales,
                                    hipStream_t stream);
// 16-byte chunks of each tensor one copy_blocks workgroup moves (256 threads x 4)
#ifndef PKV_COPY_CHUNKS_PER_WG
#define PKV_COPY_CHUNKS_PER_WG 1024
#endif
constexpr int kCopyChunksPerWg = PKV_COPY_CHUNKS_PER_WG;
hipError_t launch_copy_blocks(const void* src_k, const void* src_v, int src_blocks, void* dst_k, void* dst_v,
                              int dst_blocks, const int64_t* pairs, int num_pairs, int64_t block_bytes,
                              bool device_only, hipStream_t stream);

// Debug checks of the device-resident values (checks.hip, pkv_set_debug_checks).
// An entry point whose host checks passed builds one DeviceChecks on its
// stream, adds the checks that fit its arguments, and calls finish(): PKV_OK,
// PKV_ERR_PRECONDITION (launch nothing more) or PKV_ERR_LAUNCH.  The object
// holds the library-wide check lock until it is destroyed.
bool debug_checks_on();

class DeviceChecks {
 public:
  explicit DeviceChecks(hipStream_t stream);
  ~DeviceChecks();
  DeviceChecks(const DeviceChecks&) = delete;
  DeviceChecks& operator=(const DeviceChecks&) = delete;
  void tables(const int32_t* tables, int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
              int block_size, int num_blocks, int max_context_len);
  void permutation(const int32_t* order, int n);
  void slots(const int64_t* slots, int n, long long num_slots);
  void append_slots(const int64_t* slots, const int32_t* tables, int max_blocks_per_seq, const int32_t* context_lens,
                    int num_seqs, int block_size, long long num_slots);
  void pairs(const int64_t* mapping, int n, int src_blocks, int dst_blocks, bool same_pool);
  void groups(const int32_t* offsets, const int32_t* members, const int32_t* shared, int num_groups,
              int max_group_size, const int32_t* tables, int max_blocks_per_seq, const int32_t* context_lens,
              int num_seqs, int block_size, int ctx_cap);
  void query_starts(const int32_t* query_start_loc, int num_seqs, int num_tokens, int max_query_len);
  void scales(const float* k_scales, const float* v_scales, int num_kv_heads);
  int finish();

 private:
  struct Impl;
  Impl* impl_;
  void note(hipError_t e);
};

}  // namespace pkv
