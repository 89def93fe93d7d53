// cache_ops.hip -- the data-movement kernels of the paged cache and their C entry points
// (pkv_reshape_and_cache, pkv_copy_blocks, pkv_swap_blocks; include/pkv.h).
//
// reshape_and_cache: scatter each new token's key/value rows into the slot the
//   host chose ("PagedAttention", Ultralytics glossary, section "Cách phân trang
//   hoạt động": token pos is stored in block table[pos / bs] at offset
//   pos % bs; a flat slot is block * bs + offset).  One thread per 16 source
//   bytes: a bit copy when the cache has the source's type, else the E4M3
//   encode of value / scale (the FP8 cache of section "Các kỹ thuật liên quan").
// copy_blocks: whole-block copies for copy-on-write ("KV cache paginado e
//   batching contínuo para LLMs", section "Como funciona": a sequence writing
//   into a shared block first gets a fresh block holding a copy).  A block of
//   every kv head is one contiguous run of num_kv_heads * bs * head_dim
//   elements, so a pair is two flat 16-byte-vector copies (K and V).
// swap_blocks: the same copy between a device pool and a pinned host pool
//   (same page and section: preempted requests' blocks are swapped out to CPU
//   memory and back in).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

struct ReshapeParams {
  const void* key;
  const void* value;
  void* k_cache;
  void* v_cache;
  const int64_t* slot_mapping;
  int64_t num_slots;          // num_blocks * block_size
  int num_tokens;
  int num_kv_heads;
  int head_dim;
  int block_size;
  float k_scale;
  float v_scale;
  const float* k_scales;      // per kv head, or NULL
  const float* v_scales;
};

// Bit copy: 16 bytes of source -> 16 bytes of cache.
template <class T>
__global__ __launch_bounds__(256) void reshape_copy_kernel(ReshapeParams p) {
  constexpr int V = 16 / T::bytes;                       // elements per chunk
  const int chunks_per_row = p.head_dim / V;
  const int chunks_per_token = p.num_kv_heads * chunks_per_row;
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t token = gid / chunks_per_token;
  if (token >= (size_t)p.num_tokens) return;
  const int r = (int)(gid - token * chunks_per_token);
  const int h = r / chunks_per_row;
  const int c = r - h * chunks_per_row;
  const int64_t slot = p.slot_mapping[token];
  if (slot < 0 || slot >= p.num_slots) return;           // padding / out of pool: skipped
  const int64_t blk = slot / p.block_size;
  const int64_t off = slot - blk * p.block_size;
  const size_t src = (token * p.num_kv_heads + h) * (size_t)p.head_dim + (size_t)c * V;
  const size_t dst = (((size_t)blk * p.num_kv_heads + h) * p.block_size + off) * (size_t)p.head_dim + (size_t)c * V;
  const uint4 kv = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(p.key) + src * T::bytes);
  const uint4 vv = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(p.value) + src * T::bytes);
  *reinterpret_cast<uint4*>(reinterpret_cast<char*>(p.k_cache) + dst * T::bytes) = kv;
  *reinterpret_cast<uint4*>(reinterpret_cast<char*>(p.v_cache) + dst * T::bytes) = vv;
}

// Encode: 16 bytes of source (4 fp32 or 8 16-bit values) -> 4 or 8 codes of
// 8-bit format F (E4M3 or E5M2), with the pool's or the kv head's scale.
template <class S, class F>
__global__ __launch_bounds__(256) void reshape_fp8_kernel(ReshapeParams p) {
  constexpr int V = 16 / S::bytes;
  const int chunks_per_row = p.head_dim / V;
  const int chunks_per_token = p.num_kv_heads * chunks_per_row;
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t token = gid / chunks_per_token;
  if (token >= (size_t)p.num_tokens) return;
  const int r = (int)(gid - token * chunks_per_token);
  const int h = r / chunks_per_row;
  const int c = r - h * chunks_per_row;
  const int64_t slot = p.slot_mapping[token];
  if (slot < 0 || slot >= p.num_slots) return;
  const int64_t blk = slot / p.block_size;
  const int64_t off = slot - blk * p.block_size;
  const size_t src = (token * p.num_kv_heads + h) * (size_t)p.head_dim + (size_t)c * V;
  const size_t dst = (((size_t)blk * p.num_kv_heads + h) * p.block_size + off) * (size_t)p.head_dim + (size_t)c * V;
  const uint4 kr = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(p.key) + src * S::bytes);
  const uint4 vr = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(p.value) + src * S::bytes);
  const float ks = p.k_scales ? p.k_scales[h] : p.k_scale;
  const float vs = p.v_scales ? p.v_scales[h] : p.v_scale;
  float kf[V], vf[V];
  Unpack<S>::run(kr, kf);
  Unpack<S>::run(vr, vf);
  uint32_t kc[V / 4], vc[V / 4];
#pragma unroll
  for (int j = 0; j < V / 4; ++j) {
    uint32_t a = 0, b = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      a |= fp8_encode_scaled<F>(kf[4 * j + t], ks) << (8 * t);
      b |= fp8_encode_scaled<F>(vf[4 * j + t], vs) << (8 * t);
    }
    kc[j] = a;
    vc[j] = b;
  }
  char* kd = reinterpret_cast<char*>(p.k_cache) + dst;
  char* vd = reinterpret_cast<char*>(p.v_cache) + dst;
  if constexpr (V == 8) {
    *reinterpret_cast<uint2*>(kd) = make_uint2(kc[0], kc[1]);
    *reinterpret_cast<uint2*>(vd) = make_uint2(vc[0], vc[1]);
  } else {
    *reinterpret_cast<uint32_t*>(kd) = kc[0];
    *reinterpret_cast<uint32_t*>(vd) = vc[0];
  }
}

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                    const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                    int head_dim, int block_size, int num_blocks, int src_dtype, int kv_dtype,
                                    float k_scale, float v_scale, const float* k_scales, const float* v_scales,
                                    hipStream_t stream) {
  ReshapeParams p{key, value, k_cache, v_cache, slot_mapping, (int64_t)num_blocks * block_size,
                  num_tokens, num_kv_heads, head_dim, block_size, k_scale, v_scale, k_scales, v_scales};
  const int src_bytes = src_dtype == 0 ? 4 : 2;
  const size_t chunks = (size_t)num_tokens * num_kv_heads * (head_dim * src_bytes / 16);
  const dim3 grid((unsigned)((chunks + 255) / 256));
  if (kv_dtype == src_dtype) {
    if (src_bytes == 4) hipLaunchKernelGGL(reshape_copy_kernel<F32>, grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL(reshape_copy_kernel<F16>, grid, dim3(256), 0, stream, p);  // 16-bit: raw bits
  } else if (kv_dtype == FP8::kId) {
    if (src_dtype == 0) hipLaunchKernelGGL((reshape_fp8_kernel<F32, FP8>), grid, dim3(256), 0, stream, p);
    else if (src_dtype == 1) hipLaunchKernelGGL((reshape_fp8_kernel<F16, FP8>), grid, dim3(256), 0, stream, p);
    else if (src_dtype == 2) hipLaunchKernelGGL((reshape_fp8_kernel<BF16, FP8>), grid, dim3(256), 0, stream, p);
    else return hipErrorInvalidValue;
  } else if (kv_dtype == BF8::kId) {
    if (src_dtype == 0) hipLaunchKernelGGL((reshape_fp8_kernel<F32, BF8>), grid, dim3(256), 0, stream, p);
    else if (src_dtype == 1) hipLaunchKernelGGL((reshape_fp8_kernel<F16, BF8>), grid, dim3(256), 0, stream, p);
    else if (src_dtype == 2) hipLaunchKernelGGL((reshape_fp8_kernel<BF16, BF8>), grid, dim3(256), 0, stream, p);
    else return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

struct CopyParams {
  const char* src_k;
  const char* src_v;
  char* dst_k;
  char* dst_v;
  const int64_t* pairs;
  int64_t block_bytes;
  int src_blocks;
  int dst_blocks;
  int wgs_per_block;
};

// Whole blocks, K and V.  Serves copy_blocks (one pool) and swap_blocks (a
// device pool and a pinned host pool, either way round).  A workgroup copies
// 256 * U 16-byte chunks of one pair's block in each tensor: thread t takes
// chunks t + 256 u (u < U) and issues all 2U loads before the first store, so
// each thread keeps 2U loads in flight.  NT: both ends are device memory, and
// the copy reads each source byte once and writes each destination byte once,
// so loads and stores carry the non-temporal cache policy; copies to or from
// the host pool keep the default.
template <int U, bool NT>
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyParams p) {
  const int pair = blockIdx.x / p.wgs_per_block;
  const int64_t c0 = (int64_t)(blockIdx.x - pair * p.wgs_per_block) * (256 * U) + threadIdx.x;
  const int64_t chunks = p.block_bytes / 16;
  const int64_t src = p.pairs[2 * pair];
  const int64_t dst = p.pairs[2 * pair + 1];
  if (src < 0 || src >= p.src_blocks || dst < 0 || dst >= p.dst_blocks) return;
  const u32x4_t* sk = reinterpret_cast<const u32x4_t*>(p.src_k + src * p.block_bytes);
  const u32x4_t* sv = reinterpret_cast<const u32x4_t*>(p.src_v + src * p.block_bytes);
  u32x4_t* dk = reinterpret_cast<u32x4_t*>(p.dst_k + dst * p.block_bytes);
  u32x4_t* dv = reinterpret_cast<u32x4_t*>(p.dst_v + dst * p.block_bytes);
  u32x4_t k[U], v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = c0 + 256 * u;
    if (c < chunks) {
      if constexpr (NT) {
        k[u] = __builtin_nontemporal_load(sk + c);
        v[u] = __builtin_nontemporal_load(sv + c);
      } else {
        k[u] = sk[c];
        v[u] = sv[c];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = c0 + 256 * u;
    if (c < chunks) {
      if constexpr (NT) {
        __builtin_nontemporal_store(k[u], dk + c);
        __builtin_nontemporal_store(v[u], dv + c);
      } else {
        dk[c] = k[u];
        dv[c] = v[u];
      }
    }
  }
}

hipError_t launch_copy_blocks(const void* src_k, const void* src_v, int src_blocks, void* dst_k, void* dst_v,
                              int dst_blocks, const int64_t* pairs, int num_pairs, int64_t block_bytes,
                              bool device_only, hipStream_t stream) {
  constexpr int U = kCopyChunksPerWg / 256;
  const int64_t chunks = block_bytes / 16;
  const int wgs = (int)((chunks + kCopyChunksPerWg - 1) / kCopyChunksPerWg);
  CopyParams p{reinterpret_cast<const char*>(src_k), reinterpret_cast<const char*>(src_v),
               reinterpret_cast<char*>(dst_k), reinterpret_cast<char*>(dst_v), pairs, block_bytes,
               src_blocks, dst_blocks, wgs};
  const dim3 grid((unsigned)((int64_t)num_pairs * wgs));
  if (device_only) hipLaunchKernelGGL((copy_blocks_kernel<U, true>), grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL((copy_blocks_kernel<U, false>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv

using namespace pkv;

namespace {

// The address a kernel uses for p: p itself for device memory, the runtime's
// device-side address for pinned host memory, NULL for anything else (pageable
// host memory, unknown pointers).  Clears the error the query leaves behind.
static void* device_address(void* p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (attr.type == hipMemoryTypeDevice) return p;
  if (attr.type == hipMemoryTypeHost) {
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, p, 0) != hipSuccess || d == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    return d;
  }
  return nullptr;
}

}  // namespace

extern "C" {

int pkv_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                          const int64_t* slot_mapping, int num_tokens, int num_kv_heads, int head_dim,
                          int block_size, int num_blocks, int src_dtype, int kv_dtype, float k_scale, float v_scale,
                          const float* k_scales, const float* v_scales, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PKV_ERR_BAD_SIZE;
  if (src_dtype != PKV_F32 && src_dtype != PKV_F16 && src_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  const bool fp8 = kv_dtype == PKV_FP8_E4M3 || kv_dtype == PKV_FP8_E5M2;
  if (kv_dtype != src_dtype && !fp8) return PKV_ERR_UNSUPPORTED;
  if (head_dim % 16 != 0 || head_dim > 1024) return PKV_ERR_UNSUPPORTED;
  if (fp8 && !((k_scales || good_scale(k_scale)) && (v_scales || good_scale(v_scale)))) return PKV_ERR_SCALE;
  if ((double)num_tokens * num_kv_heads * head_dim / 4.0 > 2147483647.0 * 256.0) return PKV_ERR_BAD_SIZE;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PKV_ERR_NULL_POINTER;
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_UNSUPPORTED;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (debug_checks_on()) {
    DeviceChecks c(s);
    c.slots(slot_mapping, num_tokens, (long long)num_blocks * block_size);
    if (fp8) c.scales(k_scales, v_scales, num_kv_heads);
    const int cst = c.finish();
    if (cst != PKV_OK) return cst;
  }
  (void)hipGetLastError();
  return launch_status(launch_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, num_tokens,
                                                     num_kv_heads, head_dim, block_size, num_blocks, src_dtype,
                                                     kv_dtype, k_scale, v_scale, fp8 ? k_scales : nullptr,
                                                     fp8 ? v_scales : nullptr, s));
}

int pkv_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping, int num_pairs, int num_kv_heads,
                    int head_dim, int block_size, int num_blocks, int kv_dtype, void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PKV_ERR_BAD_SIZE;
  const int eb = dtype_bytes(kv_dtype);
  if (eb == 0) return PKV_ERR_UNSUPPORTED;
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * eb;
  if (block_bytes % 16 != 0) return PKV_ERR_UNSUPPORTED;
  const int64_t wgs = (block_bytes / 16 + kCopyChunksPerWg - 1) / kCopyChunksPerWg;
  if ((double)num_pairs * wgs > 2147483647.0) return PKV_ERR_BAD_SIZE;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !block_mapping) return PKV_ERR_NULL_POINTER;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_UNSUPPORTED;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (debug_checks_on()) {
    DeviceChecks c(s);
    c.pairs(block_mapping, num_pairs, num_blocks, num_blocks, true);
    const int cst = c.finish();
    if (cst != PKV_OK) return cst;
  }
  (void)hipGetLastError();
  return launch_status(launch_copy_blocks(k_cache, v_cache, num_blocks, k_cache, v_cache, num_blocks,
                                               block_mapping, num_pairs, block_bytes, true, s));
}

int pkv_swap_blocks(const void* src_k, const void* src_v, int src_num_blocks, void* dst_k, void* dst_v,
                    int dst_num_blocks, const int64_t* block_mapping, int num_pairs, int num_kv_heads,
                    int head_dim, int block_size, int kv_dtype, void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || src_num_blocks <= 0 ||
      dst_num_blocks <= 0)
    return PKV_ERR_BAD_SIZE;
  const int eb = dtype_bytes(kv_dtype);
  if (eb == 0) return PKV_ERR_UNSUPPORTED;
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * eb;
  if (block_bytes % 16 != 0) return PKV_ERR_UNSUPPORTED;
  const int64_t wgs = (block_bytes / 16 + kCopyChunksPerWg - 1) / kCopyChunksPerWg;
  if ((double)num_pairs * wgs > 2147483647.0) return PKV_ERR_BAD_SIZE;
  if (num_pairs == 0) return PKV_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !block_mapping) return PKV_ERR_NULL_POINTER;
  const char* sk = static_cast<const char*>(src_k);
  const char* sv = static_cast<const char*>(src_v);
  const char* dk = static_cast<const char*>(dst_k);
  const char* dv = static_cast<const char*>(dst_v);
  const int64_t sbytes = src_num_blocks * block_bytes, dbytes = dst_num_blocks * block_bytes;
  auto overlap = [](const char* a, int64_t na, const char* b, int64_t nb) { return a < b + nb && b < a + na; };
  if (overlap(sk, sbytes, dk, dbytes) || overlap(sk, sbytes, dv, dbytes) || overlap(sv, sbytes, dk, dbytes) ||
      overlap(sv, sbytes, dv, dbytes))
    return PKV_ERR_BAD_SIZE;
  void* a[5] = {const_cast<void*>(src_k), const_cast<void*>(src_v), dst_k, dst_v,
                const_cast<int64_t*>(block_mapping)};
  for (void*& x : a) {
    x = device_address(x);
    if (!x) return PKV_ERR_MEMORY_KIND;
  }
  for (int i = 0; i < 4; ++i)
    if (!aligned16(a[i])) return PKV_ERR_UNSUPPORTED;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (debug_checks_on()) {
    DeviceChecks c(s);
    c.pairs(static_cast<const int64_t*>(a[4]), num_pairs, src_num_blocks, dst_num_blocks, false);
    const int cst = c.finish();
    if (cst != PKV_OK) return cst;
  }
  (void)hipGetLastError();
  return launch_status(launch_copy_blocks(a[0], a[1], src_num_blocks, a[2], a[3], dst_num_blocks,
                                               static_cast<const int64_t*>(a[4]), num_pairs, block_bytes, false, s));
}

}  // extern "C"
