// hbm_probe.hip -- the read-rate probes declared in include/pkv_probe.h: what a
// read-only kernel gets from HBM on the machine at hand, measured beside the
// decode step by the benchmark.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;   // 16-byte loads per thread per round of the stream read

__device__ __forceinline__ uint32_t fold(const uint4& v) { return v.x ^ v.y ^ v.z ^ v.w; }

// NT: the loads carry the non-temporal cache policy, as the decode kernels' K/V
// loads do (read once, the lines stream through the caches; on this GPU plain
// loads read scattered tiles 9-11 % and a stream 7 % slower).  Plain loads
// displace what the caches hold, which a cache flush needs.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ uint4 load16(const uint4* p) {
  if constexpr (NT) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *p;
  }
}

// Each wave reads whole 8 KiB chunks (eight 1 KiB loads of consecutive bytes,
// all in flight together); wave w takes chunks w, w + W, w + 2W, ... of the
// buffer (W waves in the grid), so at any time the grid reads one contiguous
// stretch.  The bytes past the last whole chunk are read one 16-byte load per
// lane.
template <bool NT>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ buf, uint64_t n16,
                                                               uint32_t salt, uint32_t* __restrict__ sink) {
  constexpr uint64_t kChunk16 = 64 * kInFlight;            // 16-byte units per chunk
  const int lane = threadIdx.x & 63;
  const uint64_t waves = (uint64_t)gridDim.x * (kThreads / 64);
  const uint64_t wave = (uint64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const uint64_t chunks = n16 / kChunk16;
  uint32_t acc = 0;
  for (uint64_t c = wave; c < chunks; c += waves) {
    const uint4* p = buf + c * kChunk16 + lane;
    uint4 v[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) v[k] = load16<NT>(p + k * 64);
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) acc ^= fold(v[k]);
  }
  for (uint64_t i = chunks * kChunk16 + wave * 64 + lane; i < n16; i += waves * 64) acc ^= fold(load16<NT>(buf + i));
  if (acc == salt) sink[0] = acc;
}

// Tile of read number lin = wave * per_wave + i: (lin * P + salt) mod num_tiles
// with P a prime that divides no tile count a buffer can have (it exceeds any
// tile count below 2^32), so the map is a bijection of [0, num_tiles): a launch
// that reads at most num_tiles tiles reads every tile at most once, and no read
// can be served by the caches from an earlier read of the same launch.
constexpr uint64_t kTilePrime = 4294967291ull;   // the largest prime below 2^32
__device__ __forceinline__ uint64_t tile_index(uint32_t wave, int i, int per_wave, uint32_t salt, uint64_t num_tiles) {
  const uint64_t lin = (uint64_t)wave * (uint64_t)per_wave + (uint64_t)i;
  return (lin % num_tiles * (kTilePrime % num_tiles) + salt) % num_tiles;
}

template <int TILE, bool NT>
__global__ __launch_bounds__(kThreads) void tile_read_kernel(const uint4* __restrict__ buf, uint64_t num_tiles,
                                                             int per_wave, uint32_t salt,
                                                             uint32_t* __restrict__ sink) {
  constexpr int LOADS = TILE / (64 * 16);   // 16-byte loads per lane per tile
  const int lane = threadIdx.x & 63;
  const uint32_t wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  uint32_t acc = 0;
  uint4 a[LOADS], b[LOADS];
  auto issue = [&](int i, uint4* t) {
    const uint4* p = buf + tile_index(wave, i, per_wave, salt, num_tiles) * (TILE / 16) + lane;
#pragma unroll
    for (int k = 0; k < LOADS; ++k) t[k] = load16<NT>(p + k * 64);
  };
  auto use = [&](const uint4* t) {
#pragma unroll
    for (int k = 0; k < LOADS; ++k) acc ^= fold(t[k]);
  };
  if (per_wave <= 0) return;
  issue(0, a);
  for (int i = 0; i < per_wave; i += 2) {
    if (i + 1 < per_wave) issue(i + 1, b);
    use(a);
    if (i + 1 < per_wave) {
      if (i + 2 < per_wave) issue(i + 2, a);
      use(b);
    }
  }
  if (acc == salt) sink[0] = acc;
}

template <int TILE>
hipError_t launch_tiles(const uint4* buf, uint64_t num_tiles, int wgs, int per_wave, uint32_t salt, uint32_t* sink,
                        bool nt, hipStream_t s) {
  if (nt)
    hipLaunchKernelGGL((tile_read_kernel<TILE, true>), dim3(wgs), dim3(kThreads), 0, s, buf, num_tiles, per_wave, salt,
                       sink);
  else
    hipLaunchKernelGGL((tile_read_kernel<TILE, false>), dim3(wgs), dim3(kThreads), 0, s, buf, num_tiles, per_wave,
                       salt, sink);
  return hipGetLastError();
}

}  // namespace

extern "C" {

int pkv_probe_stream_read(const void* buf, size_t bytes, int num_workgroups, unsigned salt, unsigned* sink,
                          int nontemporal, void* stream) {
  if (!buf || !sink) return -1;
  if (bytes == 0 || bytes % 16 != 0 || num_workgroups <= 0 || (reinterpret_cast<uintptr_t>(buf) & 15u)) return -2;
  (void)hipGetLastError();
  const uint4* b = reinterpret_cast<const uint4*>(buf);
  uint32_t* k = reinterpret_cast<uint32_t*>(sink);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3(num_workgroups), dim3(kThreads), 0, s, b, (uint64_t)(bytes / 16),
                       (uint32_t)salt, k);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3(num_workgroups), dim3(kThreads), 0, s, b,
                       (uint64_t)(bytes / 16), (uint32_t)salt, k);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int pkv_probe_tile_read(const void* buf, size_t bytes, int tile_bytes, int num_workgroups, int tiles_per_wave,
                        unsigned salt, unsigned* sink, int nontemporal, void* stream) {
  if (!buf || !sink) return -1;
  if (num_workgroups <= 0 || tiles_per_wave <= 0 || (reinterpret_cast<uintptr_t>(buf) & 15u)) return -2;
  if (tile_bytes != 1024 && tile_bytes != 2048 && tile_bytes != 4096 && tile_bytes != 8192) return -2;
  const uint64_t num_tiles = bytes / (size_t)tile_bytes;   // whole tiles only: every load stays inside buf
  if (num_tiles == 0) return -2;
  const uint4* b = reinterpret_cast<const uint4*>(buf);
  uint32_t* k = reinterpret_cast<uint32_t*>(sink);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool nt = nontemporal != 0;
  (void)hipGetLastError();
  hipError_t e;
  switch (tile_bytes) {
    case 1024: e = launch_tiles<1024>(b, num_tiles, num_workgroups, tiles_per_wave, salt, k, nt, s); break;
    case 2048: e = launch_tiles<2048>(b, num_tiles, num_workgroups, tiles_per_wave, salt, k, nt, s); break;
    case 4096: e = launch_tiles<4096>(b, num_tiles, num_workgroups, tiles_per_wave, salt, k, nt, s); break;
    default: e = launch_tiles<8192>(b, num_tiles, num_workgroups, tiles_per_wave, salt, k, nt, s); break;
  }
  return e == hipSuccess ? 0 : -7;
}

}  // extern "C"
