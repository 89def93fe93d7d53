// pkv_device.h -- device-side helpers shared by the paged-KV kernels (gfx950 / CDNA4).
//
// Wave64 only.  Cross-lane work uses DPP inside 16-lane rows, ds_swizzle across
// the two rows of a 32-lane half and ds_bpermute (__shfl_xor) across halves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// ---------------------------------------------------------------------------
// Element types.  `bytes` is the storage size; kId matches the PKV_* codes.
// ---------------------------------------------------------------------------
struct F32 { static constexpr int bytes = 4; static constexpr int kId = 0; };
struct F16 { static constexpr int bytes = 2; static constexpr int kId = 1; };
struct BF16 { static constexpr int bytes = 2; static constexpr int kId = 2; };
struct FP8 { static constexpr int bytes = 1; static constexpr int kId = 3; };    // OCP E4M3 "FN"
struct BF8 { static constexpr int bytes = 1; static constexpr int kId = 4; };    // OCP E5M2

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float u32_as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f32_as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

// Two packed 16-bit values (low half first) -> fp32.
__device__ __forceinline__ void f16x2_to_f32(uint32_t u, float& lo, float& hi) {
  half2_t h = __builtin_bit_cast(half2_t, u);
  lo = (float)h.x;
  hi = (float)h.y;
}
__device__ __forceinline__ void bf16x2_to_f32(uint32_t u, float& lo, float& hi) {
  lo = u32_as_f32(u << 16);
  hi = u32_as_f32(u & 0xffff0000u);
}

// K/V tile loads of the decode kernels, through a buffer resource per tile.
// When a launch reads each cached byte once (distinct contexts), NT gives the
// loads the non-temporal cache policy: the lines stream through the caches
// instead of displacing others.  On this GPU the read-only probes read
// scattered tiles 9-11 % and a stream 7 % faster with it, and the one-pass
// decodes ran 5-7 % faster.  Blocks that several sequences of one launch share
// are read again by the later sequences, and those re-reads hit L2 or the
// Infinity Cache only with the default policy (NT false).  A tile that need not
// be read (an entry outside the pool, or the repeat of a wave's last block
// that keeps its loads unconditional) gets a resource of 0 bytes: a buffer load
// past the resource's end returns zeros and reads no memory.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
// A raw buffer resource over the `bytes`-byte range at `base` (wave-uniform:
// it lives in scalar registers); loads address it with 32-bit byte offsets.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
template <class V, bool NT> __device__ __forceinline__ V load_tile(__amdgpu_buffer_rsrc_t r, uint32_t off);
template <> __device__ __forceinline__ uint4 load_tile<uint4, true>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);     // cache policy: nt
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <> __device__ __forceinline__ uint4 load_tile<uint4, false>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <> __device__ __forceinline__ uint2 load_tile<uint2, true>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 2);
  return make_uint2(v.x, v.y);
}
template <> __device__ __forceinline__ uint2 load_tile<uint2, false>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v.x, v.y);
}

// 16 bytes of storage -> 16/bytes fp32 values.
template <class T> struct Unpack;
template <> struct Unpack<F32> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void run(const uint4& r, float* f) {
    f[0] = u32_as_f32(r.x); f[1] = u32_as_f32(r.y); f[2] = u32_as_f32(r.z); f[3] = u32_as_f32(r.w);
  }
};
template <> struct Unpack<F16> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void run(const uint4& r, float* f) {
    f16x2_to_f32(r.x, f[0], f[1]); f16x2_to_f32(r.y, f[2], f[3]);
    f16x2_to_f32(r.z, f[4], f[5]); f16x2_to_f32(r.w, f[6], f[7]);
  }
};
template <> struct Unpack<BF16> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void run(const uint4& r, float* f) {
    bf16x2_to_f32(r.x, f[0], f[1]); bf16x2_to_f32(r.y, f[2], f[3]);
    bf16x2_to_f32(r.z, f[4], f[5]); bf16x2_to_f32(r.w, f[6], f[7]);
  }
};
// E4M3 decode uses the gfx950 convert, which implements the OCP E4M3 "FN"
// decoding (all 256 codes were checked against the format's definition).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t u, float* f) {
  auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)u, false);
  auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)u, true);
  f[0] = lo[0]; f[1] = lo[1]; f[2] = hi[0]; f[3] = hi[1];
}
template <> struct Unpack<FP8> {
  static constexpr int N = 16;
  __device__ __forceinline__ static void run(const uint4& r, float* f) {
    fp8x4_to_f32(r.x, f); fp8x4_to_f32(r.y, f + 4); fp8x4_to_f32(r.z, f + 8); fp8x4_to_f32(r.w, f + 12);
  }
};
// E5M2 decode: an E5M2 code is the top byte of the fp16 with the same value
// (same sign and exponent fields, 2 of fp16's 10 mantissa bits), so the code
// shifted into the high byte of a half is exact, infinities and NaN included.
__device__ __forceinline__ void bf8x4_to_f32(uint32_t u, float* f) {
  f16x2_to_f32(((u & 0xffu) << 8) | ((u & 0xff00u) << 16), f[0], f[1]);
  f16x2_to_f32(((u >> 8) & 0xff00u) | (u & 0xff000000u), f[2], f[3]);
}
template <> struct Unpack<BF8> {
  static constexpr int N = 16;
  __device__ __forceinline__ static void run(const uint4& r, float* f) {
    bf8x4_to_f32(r.x, f); bf8x4_to_f32(r.y, f + 4); bf8x4_to_f32(r.z, f + 8); bf8x4_to_f32(r.w, f + 12);
  }
};

// 8-bit K/V (E4M3 = FP8, E5M2 = BF8) as MFMA operands.  Both formats convert
// exactly to f16 and bf16, so the products and sums are those of the 16-bit
// path over the dequantised values; the scales are applied to the logits (k)
// and to the output (v).
// Two 8-bit codes (the low or high half of a word) -> two elements of the
// 16-bit MFMA type T, through gfx950's scaled converts at scale 1 (exact:
// checked on every code of both formats, both halves, NaN and infinity
// classes included).
template <class T, class KT> __device__ __forceinline__ uint32_t kv8x2_to_16(uint32_t u, bool hi);
template <> __device__ __forceinline__ uint32_t kv8x2_to_16<BF16, FP8>(uint32_t u, bool hi) {
  return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u, 1.0f, true)
                                         : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u, 1.0f, false));
}
template <> __device__ __forceinline__ uint32_t kv8x2_to_16<BF16, BF8>(uint32_t u, bool hi) {
  return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(u, 1.0f, true)
                                         : __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(u, 1.0f, false));
}
template <> __device__ __forceinline__ uint32_t kv8x2_to_16<F16, FP8>(uint32_t u, bool hi) {
  return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(u, 1.0f, true)
                                         : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(u, 1.0f, false));
}
template <> __device__ __forceinline__ uint32_t kv8x2_to_16<F16, BF8>(uint32_t u, bool hi) {
  return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(u, 1.0f, true)
                                         : __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(u, 1.0f, false));
}

// Eight 8-bit codes (two words) -> eight elements of the 16-bit MFMA type T.
template <class T, class KT>
__device__ __forceinline__ uint4 kv8x8_to_16(uint32_t a, uint32_t b) {
  return make_uint4(kv8x2_to_16<T, KT>(a, false), kv8x2_to_16<T, KT>(a, true), kv8x2_to_16<T, KT>(b, false),
                    kv8x2_to_16<T, KT>(b, true));
}

// One scalar element of storage type T at p[i] -> fp32.
template <class T> __device__ __forceinline__ float load_elem(const void* p, size_t i);
template <> __device__ __forceinline__ float load_elem<F32>(const void* p, size_t i) {
  return reinterpret_cast<const float*>(p)[i];
}
template <> __device__ __forceinline__ float load_elem<F16>(const void* p, size_t i) {
  return (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(p)[i]);
}
template <> __device__ __forceinline__ float load_elem<BF16>(const void* p, size_t i) {
  return u32_as_f32((uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16);
}

// fp32 -> storage, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = f32_as_u32(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
template <class T> __device__ __forceinline__ void store_elem(void* p, size_t i, float v);
template <> __device__ __forceinline__ void store_elem<F32>(void* p, size_t i, float v) {
  reinterpret_cast<float*>(p)[i] = v;
}
template <> __device__ __forceinline__ void store_elem<F16>(void* p, size_t i, float v) {
  reinterpret_cast<uint16_t*>(p)[i] = __builtin_bit_cast(uint16_t, (_Float16)v);
}
template <> __device__ __forceinline__ void store_elem<BF16>(void* p, size_t i, float v) {
  reinterpret_cast<uint16_t*>(p)[i] = f32_to_bf16_rne(v);
}

// ---------------------------------------------------------------------------
// E4M3 encode (OCP "FN"): nearest code with ties to even mantissa, saturating
// to +-448 (also for +-inf), NaN -> 0x7F | sign.  `v` is the already-scaled
// fp32 value.  Pure integer/float bit work, independent of the hardware
// convert (which does not saturate).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t u = f32_as_u32(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t ua = u & 0x7fffffffu;
  if (ua > 0x7f800000u) return 0x7fu | sign;          // NaN
  if (ua >= 0x43e00000u) return 0x7eu | sign;         // |v| >= 448 (and inf): saturate
  if (ua < 0x3c800000u) {                              // |v| < 2^-6: subnormal step 2^-9
    const float k = __builtin_rintf(u32_as_f32(ua) * 512.0f);  // exact scaling, RNE
    return sign | (uint32_t)k;                         // k == 8 is the smallest normal
  }
  // normal: keep 3 mantissa bits of the fp32 pattern, round to nearest even
  const uint32_t r = ua + 0x7ffffu + ((ua >> 20) & 1u);
  const uint32_t e = (r >> 23) - 127u + 7u;            // E4M3 biased exponent (1..15)
  const uint32_t m = (r >> 20) & 7u;
  return sign | (e << 3) | m;
}

// Code of x / scale: the division is IEEE fp32 (correctly rounded; the library
// is built without fast-math); a NaN input keeps its own sign bit.
__device__ __forceinline__ uint32_t e4m3_encode_scaled(float x, float scale) {
  const uint32_t u = f32_as_u32(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fu | ((u >> 24) & 0x80u);
  return e4m3_encode(x / scale);
}

// E5M2 encode (OCP): nearest code with ties to even mantissa, saturating to
// +-57344 (also for +-inf: the cache stores finite values), NaN -> 0x7F | sign.
__device__ __forceinline__ uint32_t e5m2_encode(float v) {
  const uint32_t u = f32_as_u32(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t ua = u & 0x7fffffffu;
  if (ua > 0x7f800000u) return 0x7fu | sign;          // NaN
  if (ua >= 0x47600000u) return 0x7bu | sign;         // |v| >= 57344 (and inf): saturate
  if (ua < 0x38800000u) {                              // |v| < 2^-14: subnormal step 2^-16
    const float k = __builtin_rintf(u32_as_f32(ua) * 65536.0f);  // exact scaling, RNE
    return sign | (uint32_t)k;                         // k == 4 is the smallest normal
  }
  // normal: keep 2 mantissa bits of the fp32 pattern, round to nearest even
  const uint32_t r = ua + 0xfffffu + ((ua >> 21) & 1u);
  const uint32_t e = (r >> 23) - 127u + 15u;           // E5M2 biased exponent (1..30)
  const uint32_t m = (r >> 21) & 3u;
  return sign | (e << 2) | m;
}

// Code of x / scale in 8-bit format F (FP8 = E4M3, BF8 = E5M2).
template <class F> __device__ __forceinline__ uint32_t fp8_encode_scaled(float x, float scale);
template <> __device__ __forceinline__ uint32_t fp8_encode_scaled<FP8>(float x, float scale) {
  return e4m3_encode_scaled(x, scale);
}
template <> __device__ __forceinline__ uint32_t fp8_encode_scaled<BF8>(float x, float scale) {
  const uint32_t u = f32_as_u32(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fu | ((u >> 24) & 0x80u);
  return e5m2_encode(x / scale);
}

// ---------------------------------------------------------------------------
// Cross-lane reductions.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float swz_xor16(float x) {  // lane ^ 16 within each 32-lane half
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401f));
}
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// Reductions over the lane pairs (l, l ^ 32) and (l, l ^ 16) with gfx950's row
// swaps, which move values between VGPRs without the LDS crossbar:
// v_permlane32_swap_b32 exchanges the upper 32 lanes of its first operand with
// the lower 32 of its second, v_permlane16_swap_b32 the odd 16-lane rows of the
// first with the even rows of the second.  Given two copies of x, the two
// results hold x of lanes l and l ^ 32 (l ^ 16) between them, so a commutative
// op of the pair is the reduction (checked on hardware with lane ids).  The
// instruction is written in asm because this toolchain's optimiser drops the
// builtin's second result; the s_nops give it its VALU hazard wait states.
__device__ __forceinline__ void row_swap32(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void row_swap16(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
// max (sum) over the four lanes l, l ^ 16, l ^ 32, l ^ 48 of each column of 16.
// The max is one asm block with its v_max_f32: an fmaxf of the asm outputs
// would first quiet possible signalling NaNs (two more instructions per max);
// the values here are never NaN (finite logits or -inf).
__device__ __forceinline__ float max_over_rows(float x) {
  float y;
  asm("v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\t"
      "v_max_f32 %0, %0, %1\n\t"
      "v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1\n\t"
      "v_max_f32 %0, %0, %1"
      : "+v"(x), "=&v"(y));
  return x;
}
__device__ __forceinline__ float sum_over_rows(float x) {
  float y = x;
  row_swap32(x, y);
  x += y;
  y = x;
  row_swap16(x, y);
  return x + y;
}

// Sum over each aligned group of N consecutive lanes (N = 1..64, power of two);
// every lane of the group ends with the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_f32<0xb1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (N >= 4) x += dpp_f32<0x4e>(x);    // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (N >= 8) x += dpp_f32<0x141>(x);   // row_half_mirror: other quad of the 8
  if constexpr (N >= 16) x += dpp_f32<0x140>(x);  // row_mirror: other half of the 16
  if constexpr (N >= 32) x += swz_xor16(x);
  if constexpr (N >= 64) x += xor32(x);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 1; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Workgroup-id remap.  The dispatcher hands workgroup i to XCD i % 8 (each XCD
// has its own L2).  Logical ids are regrouped in chunks of C consecutive ids:
// a chunk runs on one XCD, back to back, and consecutive chunks go to
// consecutive XCDs.  Consecutive sequences of one (head, partition) -- e.g. the
// samples of one prompt that share its cached blocks -- then meet in one L2,
// while every XCD still receives an even mix of partitions.  A bijection on
// [0, n); ids past the last whole round of 8*C keep their order.
// ---------------------------------------------------------------------------
// Workgroup -> logical work id.  The hardware deals consecutive workgroup ids
// round-robin to the 8 XCDs (each with its own L2).  chunk == 0 keeps that
// order; chunk C > 0 gives each XCD runs of C consecutive logical ids instead
// (the tail that does not fill 8 * C ids keeps the hardware order).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t i, uint32_t n, uint32_t chunk) {
  constexpr uint32_t X = 8;
  if (chunk == 0) return i;
  const uint32_t full = n / (X * chunk) * (X * chunk);
  if (i >= full) return i;
  const uint32_t x = i % X, k = i / X;
  return ((k / chunk) * X + x) * chunk + (k % chunk);
}

// One-pass launches with U head units per sequence, U a multiple of 8: the
// logical id of workgroup i, such that the XCD of i (i % 8) takes head units
// [x U/8, (x+1) U/8) of every sequence.  Neighbouring (block, head) tiles of a
// block -- one contiguous run in the pool -- are then read by one XCD, and a
// given head always runs on the same XCD, so forks of a prompt launched
// together meet their shared blocks in that XCD's L2.  A bijection on each
// sequence's U ids.
__device__ __forceinline__ uint32_t head_runs(uint32_t i, uint32_t units) {
  const uint32_t r = i / units, w = i - r * units;
  return r * units + (w & 7u) * (units >> 3) + (w >> 3);
}

// Logical work id -> (sequence, head unit, partition).  Partitions are the
// slowest dimension.  With PKV_HEAD_FASTEST the head units of one sequence are
// consecutive, so concurrent workgroups read the neighbouring per-head tiles of
// the same physical blocks (one block of every kv head is one contiguous run).
#ifndef PKV_HEAD_FASTEST
#define PKV_HEAD_FASTEST 1
#endif
#ifndef PKV_PARTITIONS_REVERSED
#define PKV_PARTITIONS_REVERSED 1
#endif
__device__ __forceinline__ void decode_work_id(uint32_t L, int num_seqs, int num_units, int& seq, int& unit,
                                               int& part) {
  if constexpr (PKV_HEAD_FASTEST) {
    unit = (int)(L % (uint32_t)num_units);
    const uint32_t rest = L / (uint32_t)num_units;
    seq = (int)(rest % (uint32_t)num_seqs);
    part = (int)(rest / (uint32_t)num_seqs);
  } else {
    seq = (int)(L % (uint32_t)num_seqs);
    const uint32_t rest = L / (uint32_t)num_seqs;
    unit = (int)(rest % (uint32_t)num_units);
    part = (int)(rest / (uint32_t)num_units);
  }
}

// ---------------------------------------------------------------------------
// Kernel parameter blocks (passed by value as kernel arguments).
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Balanced slices of the context.  For one head unit, the work items are the
// (sequence, block) pairs of every sequence laid end to end: sequence s owns
// items [prefix[s], prefix[s+1]) with prefix[s+1] - prefix[s] = ceil(ctx_s/bs).
// Slice k of NS covers items [k*T/NS, (k+1)*T/NS), T = prefix[S], so every
// workgroup gets the same amount of KV to read whatever the length mix.
// ---------------------------------------------------------------------------
constexpr int kMaxSliceSeqs = 1024;   // prefix kept in LDS; more sequences use fixed partitions

__device__ __forceinline__ int64_t slice_begin(int k, int64_t T, int ns) { return (int64_t)k * T / ns; }

// Slice holding item x (0 <= x < T).
__device__ __forceinline__ int slice_of(int64_t x, int64_t T, int ns) {
  int k = (int)(x * ns / T);
  while (k + 1 < ns && slice_begin(k + 1, T, ns) <= x) ++k;
  while (k > 0 && slice_begin(k, T, ns) > x) --k;
  return k;
}

// Exclusive block prefix of the (clamped) context lengths into LDS:
// s_prefix[s] for s = 0..S (s_prefix[S] = T).  Every thread of the workgroup
// calls it; NT threads, S <= kMaxSliceSeqs.  Ends with a barrier.
template <int NT>
__device__ void block_prefix(const int32_t* context_lens, int S, int ctx_cap, int bs, int* s_prefix, int* s_wsum,
                             bool at_least_one = false) {
  constexpr int PER = (kMaxSliceSeqs + NT - 1) / NT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int v[PER];
  int local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = tid * PER + i;
    int c = idx < S ? context_lens[idx] : 0;
    c = c < 0 ? 0 : (c > ctx_cap ? ctx_cap : c);
    v[i] = (c + bs - 1) / bs;
    if (at_least_one && idx < S && v[i] == 0) v[i] = 1;   // an empty context still owns one (zero-output) item
    local += v[i];
  }
  int x = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_wsum[w] = x;
  __syncthreads();
  int run = x - local;
  for (int i = 0; i < w; ++i) run += s_wsum[i];
  if (tid == 0) s_prefix[0] = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = tid * PER + i;
    run += v[i];
    if (idx < S) s_prefix[idx + 1] = run;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Longest-first order for one-pass launches, computed inside every workgroup.
// Sequences are keyed by their block count in half-octave buckets (key 0 for
// an empty context, then 2 keys per power of two), counted with wave ballots;
// rank r is the r-th sequence in decreasing key order, ties in index order.
// Dispatching workgroups in this order is greedy longest-processing-time list
// scheduling up to a factor sqrt(2) in the sort key; which workgroup takes a
// sequence never changes its result.  All threads call it; S <= kMaxSliceSeqs.
// ---------------------------------------------------------------------------
constexpr int kOrderKeys = 32;

__device__ __forceinline__ int order_key(int nblk) {
  if (nblk <= 0) return 0;
  const int msb = 31 - __builtin_clz((unsigned)nblk);
  const int half = msb > 0 ? (nblk >> (msb - 1)) & 1 : 0;
  const int k = 1 + 2 * msb + half;
  return k < kOrderKeys ? k : kOrderKeys - 1;
}

template <int NT>
__device__ __forceinline__ int seq_of_rank(const int32_t* context_lens, int S, int ctx_cap, int bs, int r, int* s_cnt, int* s_pick) {
  constexpr int NWV = NT / 64;
  constexpr int CHUNKS = (kMaxSliceSeqs + NT - 1) / NT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int key[CHUNKS];
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
    const int t = c * NT + tid;
    int ctx = t < S ? context_lens[t] : 0;
    ctx = ctx < 0 ? 0 : (ctx > ctx_cap ? ctx_cap : ctx);
    key[c] = t < S ? order_key((ctx + bs - 1) / bs) : -1;
  }
  // s_cnt[(c * NWV + w) * kOrderKeys + k]: sequences with key k in wave w of chunk c
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
    if (c * NT >= S) break;                                  // uniform
    int mine = 0;
#pragma unroll
    for (int k = 0; k < kOrderKeys; ++k) {
      const int n = __builtin_popcountll(__ballot(key[c] == k));
      if (lane == k) mine = n;
    }
    if (lane < kOrderKeys) s_cnt[(c * NWV + w) * kOrderKeys + lane] = mine;
  }
  __syncthreads();
  // the bucket holding rank r (keys in decreasing order), and r's position in
  // it: lane k sums bucket k, a suffix scan over lanes gives each bucket's first
  // rank, a ballot finds the bucket containing r
  const int groups = ((S + NT - 1) / NT) * NWV;
  int tot = 0;
  if (lane < kOrderKeys)
    for (int g = 0; g < groups; ++g) tot += s_cnt[g * kOrderKeys + lane];
  int suffix = tot;                                          // sum of buckets lane .. kOrderKeys-1
#pragma unroll
  for (int off = 1; off < kOrderKeys; off <<= 1) {
    const int y = __shfl_down(suffix, off, 64);
    if (lane + off < kOrderKeys) suffix += y;
  }
  const int first_rank = suffix - tot;                       // ranks of longer buckets come first
  const bool hit = lane < kOrderKeys && tot > 0 && r >= first_rank && r < first_rank + tot;
  const int K = __builtin_ffsll((long long)__ballot(hit)) - 1;
  int before = r - __shfl(first_rank, K, 64);                // members of bucket K before the target
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
    if (c * NT >= S) break;
    int prior = 0;                                           // bucket-K members in earlier waves of this chunk
    for (int g = 0; g < w; ++g) prior += s_cnt[(c * NWV + g) * kOrderKeys + K];
    const uint64_t m = __ballot(key[c] == K);
    const int below = __builtin_popcountll(m & ((1ull << lane) - 1ull));
    if (key[c] == K && prior + below == before) *s_pick = c * NT + tid;
    int chunk_total = 0;
    for (int g = 0; g < NWV; ++g) chunk_total += s_cnt[(c * NWV + g) * kOrderKeys + K];
    before -= chunk_total;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*s_pick);           // the same in every lane: keep it scalar
}

struct AttnParams {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_m;   // [S][H][NP]      running max of each partition (log2 domain)
  float* ws_l;   // [S][H][NP]      exp-sum of each partition
  float* ws_o;   // [S][H][NP][D]   unnormalised output of each partition (v_scale applied)
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int group;               // num_heads / num_kv_heads
  int max_blocks_per_seq;
  int num_blocks;
  int partition_blocks;    // blocks per partition
  int num_partitions;      // NP; 1 => the attention kernel writes `out` directly
  int ctx_cap;             // contexts are clamped to this many tokens
  int num_slices;          // > 0: balanced slices (partition fields unused)
  int longest_first;       // one pass: workgroup r takes the r-th longest sequence
  const int32_t* seq_order;  // one pass: the caller's longest-first order (else derived in-workgroup)
  int* ws_prefix;          // [S+1] block prefix, written by workgroup 0 in slice mode
  // decode with append: sequence s's new token (row s of new_k / new_v, q's
  // dtype) goes to slot slot_mapping[s] before the attention reads it; NULL
  // new_k for a plain decode.  enc_*_scale: the pool-wide 8-bit encode scales.
  const void* new_k;
  const void* new_v;
  const int64_t* slot_mapping;
  float enc_k_scale;
  float enc_v_scale;
  const float* k_scales;   // [num_kv_heads] per-head 8-bit scales, or NULL (then k_scale is in qk_scale)
  const float* v_scales;   // [num_kv_heads] or NULL (then v_scale applies)
  float qk_scale;          // scale * log2(e) * k_scale
  float v_scale;
  int compact_partitions;   // fixed partitions: work ids walk the (sequence, partition) units that exist,
                            // sequence by sequence, per head unit (else the partition-major grid)
  uint32_t total_wgs;
  uint32_t xcd_chunk;       // see xcd_remap
  uint32_t head_run_units;  // > 0: one pass, workgroup -> work id through head_runs (xcd_chunk unused)
  int kv_cached;            // K/V loads with the default cache policy (else non-temporal; see load_tile)
  // shared-block decode only (attn_shared.hip): group g's members are
  // grp_mem[grp_off[g] .. grp_off[g+1]) (at most grp_max of them); the first
  // grp_shared[g] blocks of their tables are the same physical blocks.
  const int32_t* grp_off;
  const int32_t* grp_mem;
  const int32_t* grp_shared;
  int grp_max;
};

// Decode with append: the wave that will load sequence seq's last block (wave
// `owner` of the workgroup) writes that sequence's new K/V row for kv head g
// into its slot (bit copy, or the 8-bit encode with the pool's or the head's
// scale) and waits for the stores before going on, so its own later loads see
// the row; the other waves do not wait, and no other workgroup reads the row in
// this launch.  Several query-head workgroups sharing a kv head each write the
// same bytes.  Called by every thread of the workgroup (the wave index is
// uniform).
template <class ST, class KT, int D, int BS, int NT>
__device__ void append_new_row(const AttnParams& p, int seq, int g, int owner) {
  if ((int)(threadIdx.x >> 6) != owner) return;
  constexpr int NT_ = 64;                                   // the owner wave's lanes do the writes
  (void)NT;
  const int64_t slot = p.slot_mapping[seq];
  if (slot >= 0 && slot < (int64_t)p.num_blocks * BS) {
    const int64_t blk = slot / BS, off = slot - blk * BS;
    const size_t src = ((size_t)seq * p.num_kv_heads + g) * D;
    const size_t dst = (((size_t)blk * p.num_kv_heads + g) * BS + off) * D;
    char* kd = reinterpret_cast<char*>(const_cast<void*>(p.k_cache));
    char* vd = reinterpret_cast<char*>(const_cast<void*>(p.v_cache));
    if constexpr (KT::kId == ST::kId) {                     // bit copy in 16-byte chunks
      constexpr int V = 16 / ST::bytes;
      for (int c = threadIdx.x & 63; c < D / V; c += NT_) {
        const char* ks = reinterpret_cast<const char*>(p.new_k) + (src + c * V) * ST::bytes;
        const char* vs = reinterpret_cast<const char*>(p.new_v) + (src + c * V) * ST::bytes;
        *reinterpret_cast<uint4*>(kd + (dst + c * V) * KT::bytes) = *reinterpret_cast<const uint4*>(ks);
        *reinterpret_cast<uint4*>(vd + (dst + c * V) * KT::bytes) = *reinterpret_cast<const uint4*>(vs);
      }
    } else {                                                // 8-bit cache: each lane encodes D/64 elements
      constexpr int EPL = D / 64;
      static_assert(EPL == 1 || EPL == 2 || EPL == 4, "head_dim 64, 128 or 256");
      const float ks = p.k_scales ? p.k_scales[g] : p.enc_k_scale;
      const float vs = p.v_scales ? p.v_scales[g] : p.enc_v_scale;
      const int c = threadIdx.x & 63;
      uint32_t kc = 0, vc = 0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        kc |= fp8_encode_scaled<KT>(load_elem<ST>(p.new_k, src + c * EPL + e), ks) << (8 * e);
        vc |= fp8_encode_scaled<KT>(load_elem<ST>(p.new_v, src + c * EPL + e), vs) << (8 * e);
      }
      if constexpr (EPL == 4) {
        *reinterpret_cast<uint32_t*>(kd + dst + c * EPL) = kc;
        *reinterpret_cast<uint32_t*>(vd + dst + c * EPL) = vc;
      } else if constexpr (EPL == 2) {
        *reinterpret_cast<uint16_t*>(kd + dst + c * EPL) = (uint16_t)kc;
        *reinterpret_cast<uint16_t*>(vd + dst + c * EPL) = (uint16_t)vc;
      } else {
        *reinterpret_cast<uint8_t*>(kd + dst + c) = (uint8_t)kc;
        *reinterpret_cast<uint8_t*>(vd + dst + c) = (uint8_t)vc;
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");   // stores done before this wave's later loads
}

// Per-head 8-bit scales of kv head g folded into the workgroup's copy of the
// parameters (the pool-wide scales are already in qk_scale / v_scale otherwise).
__device__ __forceinline__ void apply_head_scales(AttnParams& p, int g) {
  if (p.k_scales) p.qk_scale *= p.k_scales[g];
  if (p.v_scales) p.v_scale *= p.v_scales[g];
}

struct ReduceParams {
  void* out;
  const int32_t* context_lens;
  const float* ws_m;
  const float* ws_l;
  const float* ws_o;
  const int* ws_prefix;    // slice mode
  int num_seqs;
  int num_heads;
  int num_partitions;      // partition mode
  int partition_tokens;
  int num_slices;          // slice mode when > 0
  int ctx_cap;
};

// Chunked prefill over the paged cache (see prefill_mfma.hip).
struct PrefillParams {
  void* out;                       // [num_tokens][num_heads][D]
  const void* q;                   // [num_tokens][num_heads][D]
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start_loc;  // [num_seqs + 1]
  int num_seqs;
  int num_tokens;                  // rows of q / out
  int num_heads;
  int num_kv_heads;
  int group;
  int max_blocks_per_seq;
  int num_blocks;
  int max_query_len;
  int q_tiles;                     // query tiles per sequence in the grid
  int ctx_cap;
  int longest_first;               // sequences dispatched in decreasing context length
  float qk_scale;                  // scale * log2(e)
  float k_scale, v_scale;          // 8-bit cache: the pools' scales, or
  const float* k_scales;           // per kv head ([num_kv_heads]) when given
  const float* v_scales;
  uint32_t total_wgs;
  uint32_t xcd_chunk;
};

}  // namespace pkv
