// attn_vector.hip -- paged decode attention, one workgroup per (sequence, query
// head, context partition), no matrix cores.  Used for multi-head attention
// (one query head per kv head, where QK and PV are matrix-vector products) and
// for every dtype combination the MFMA family does not cover.
//
// What it computes ("PagedAttention", Ultralytics glossary, section "Cách phân
// trang hoạt động": the kernel gathers keys and values block by block through
// the request's block table; section "Các kỹ thuật liên quan": the score row is
// never written out, FlashAttention-style):
//   for the partition's blocks j: b = table[j]; K,V tile = pool[b][kv_head]
//   s_t = scale * <q, K_t>;  online softmax (running max m, running sum l);
//   acc += e^(s_t - m) V_t
//
// Data layout in registers.  A (block, kv head) tile is BS rows of D elements,
// contiguous.  One 16-byte load per lane per row group: lane `col` (0..LPR-1)
// of row group `row` holds elements [col*VEC, col*VEC+VEC) of token
// i*RPW + row, so one wave-wide load instruction reads RPW whole rows = 1 KiB of
// consecutive bytes.  The dot product of a token is reduced over its LPR lanes
// with DPP (row_mirror / half_mirror / quad_perm); each row group keeps its own
// running (m, l, acc) so the hot loop needs no cross-row traffic.  Row groups,
// then waves (through LDS), are merged once at the end.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

template <class QT, class KT, int VEC>
struct QFrag {
  // fp32 query slice, pre-multiplied by nothing (the scale is applied to the
  // reduced dot product so 16-bit queries keep their exact values).
  float f[VEC];
  __device__ __forceinline__ void load(const void* q, size_t off) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) f[e] = load_elem<QT>(q, off + e);
  }
  __device__ __forceinline__ float dot(const uint4& k) const {
    float kv[VEC];
    Unpack<KT>::run(k, kv);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) s = __builtin_fmaf(f[e], kv[e], s);
    return s;
  }
};

// 16-bit q against a 16-bit cache of the same type: packed dot2 with fp32 accumulation.
template <>
struct QFrag<F16, F16, 8> {
  uint32_t h[4];
  __device__ __forceinline__ void load(const void* q, size_t off) {
    const uint4 r = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(q) + off);
    h[0] = r.x; h[1] = r.y; h[2] = r.z; h[3] = r.w;
  }
  __device__ __forceinline__ float dot(const uint4& k) const {
    float s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, h[0]), __builtin_bit_cast(half2_t, k.x), 0.f, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, h[1]), __builtin_bit_cast(half2_t, k.y), s, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, h[2]), __builtin_bit_cast(half2_t, k.z), s, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, h[3]), __builtin_bit_cast(half2_t, k.w), s, false);
    return s;
  }
};
template <>
struct QFrag<BF16, BF16, 8> {
  uint32_t h[4];
  __device__ __forceinline__ void load(const void* q, size_t off) {
    const uint4 r = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(q) + off);
    h[0] = r.x; h[1] = r.y; h[2] = r.z; h[3] = r.w;
  }
  __device__ __forceinline__ float dot(const uint4& k) const {
    float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, h[0]), __builtin_bit_cast(bf162_t, k.x), 0.f, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, h[1]), __builtin_bit_cast(bf162_t, k.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, h[2]), __builtin_bit_cast(bf162_t, k.z), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, h[3]), __builtin_bit_cast(bf162_t, k.w), s, false);
    return s;
  }
};

template <class QT, class KT, int D, int BS, int NW, int UNROLL>
__global__ __launch_bounds__(NW * 64) void attn_vector_kernel(AttnParams p) {
  constexpr int ELT = KT::bytes;
  constexpr int VEC = 16 / ELT;        // elements per 16-byte load
  constexpr int LPR = D * ELT / 16;    // lanes per token row
  constexpr int RPW = 64 / LPR;        // token rows per wave-wide load
  constexpr int NI = BS / RPW;         // loads per lane per tile
  constexpr size_t ROW_BYTES = (size_t)D * ELT;
  constexpr size_t TILE_BYTES = ROW_BYTES * BS;
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "row must split into whole lanes");
  static_assert(NI >= 1 && BS % RPW == 0, "block must hold whole row groups");

  const uint32_t L = xcd_remap(blockIdx.x, p.total_wgs);
  int seq, head, part;
  decode_work_id(L, p.num_seqs, p.num_heads, seq, head, part);
  const int kvh = head / p.group;

  int ctx = p.context_lens[seq];
  ctx = ctx < 0 ? 0 : (ctx > p.ctx_cap ? p.ctx_cap : ctx);
  const int nblk = (ctx + BS - 1) / BS;
  const int b_begin = part * p.partition_blocks;
  const bool direct = p.num_partitions == 1;
  if (!direct && b_begin >= nblk) return;               // empty partition: the reduce skips it
  int b_end = b_begin + p.partition_blocks;
  b_end = b_end < nblk ? b_end : nblk;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane / LPR;
  const int col = lane % LPR;

  const size_t q_off = ((size_t)seq * p.num_heads + head) * D + (size_t)col * VEC;
  QFrag<QT, KT, VEC> qf;
  qf.load(p.q, q_off);

  const int32_t* table = p.block_tables + (size_t)seq * p.max_blocks_per_seq;
  const char* kbase = reinterpret_cast<const char*>(p.k_cache) + (size_t)kvh * TILE_BYTES + row * ROW_BYTES + col * 16;
  const char* vbase = reinterpret_cast<const char*>(p.v_cache) + (size_t)kvh * TILE_BYTES + row * ROW_BYTES + col * 16;
  const size_t block_stride = TILE_BYTES * (size_t)p.num_kv_heads;

  float m = -__builtin_inff();
  float l = 0.f;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

  const int last_partial = (ctx % BS) ? nblk - 1 : -1;

  for (int jb0 = b_begin + w; jb0 < b_end; jb0 += NW * UNROLL) {
    uint4 kr[UNROLL][NI], vr[UNROLL][NI];
    bool ok[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int jb = jb0 + u * NW;
      int blk = jb < b_end ? table[jb] : -1;
      ok[u] = blk >= 0 && blk < p.num_blocks;
      blk = ok[u] ? blk : 0;
      const char* kp = kbase + (size_t)blk * block_stride;
      const char* vp = vbase + (size_t)blk * block_stride;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if (ok[u]) {
          kr[u][i] = *reinterpret_cast<const uint4*>(kp + i * RPW * ROW_BYTES);
          vr[u][i] = *reinterpret_cast<const uint4*>(vp + i * RPW * ROW_BYTES);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int jb = jb0 + u * NW;
      if (!ok[u]) continue;                               // wave-uniform
      const bool masked = jb == last_partial;             // wave-uniform
      float s[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) s[i] = group_sum<LPR>(qf.dot(kr[u][i])) * p.qk_scale;
      if (masked) {
        const int valid = ctx - jb * BS;                  // 1 .. BS-1 tokens of this block are real
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const bool v = i * RPW + row < valid;
          s[i] = v ? s[i] : -__builtin_inff();
          if (!v) vr[u][i] = make_uint4(0u, 0u, 0u, 0u);  // tail slots may hold NaN: drop, never multiply
        }
      }
      float mb = s[0];
#pragma unroll
      for (int i = 1; i < NI; ++i) mb = fmaxf(mb, s[i]);
      const float mn = fmaxf(m, mb);
      const bool live = mn != -__builtin_inff();          // false only for a row with no token yet
      const float alpha = live ? exp2_fast(m - mn) : 1.f;
      float pr[NI];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        pr[i] = live ? exp2_fast(s[i] - mn) : 0.f;
        psum += pr[i];
      }
      l = l * alpha + psum;
      m = mn;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] *= alpha;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float vf[VEC];
        Unpack<KT>::run(vr[u][i], vf);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = __builtin_fmaf(pr[i], vf[e], acc[e]);
      }
    }
  }

  // merge the RPW row groups of this wave (lanes with the same col)
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const float l2 = __shfl_xor(l, off, 64);
    const float mn = fmaxf(m, m2);
    const float a = (m == -__builtin_inff()) ? 0.f : exp2_fast(m - mn);
    const float b = (m2 == -__builtin_inff()) ? 0.f : exp2_fast(m2 - mn);
    l = l * a + l2 * b;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = acc[e] * a + __shfl_xor(acc[e], off, 64) * b;
    m = mn;
  }

  // merge the NW waves through LDS
  __shared__ float sm_m[NW], sm_l[NW];
  __shared__ float sm_acc[NW][D];
  if (row == 0) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) sm_acc[w][col * VEC + e] = acc[e];
    if (col == 0) { sm_m[w] = m; sm_l[w] = l; }
  }
  __syncthreads();
  float M = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < NW; ++i) M = fmaxf(M, sm_m[i]);
  float wgt[NW];
  float Lsum = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    wgt[i] = (sm_m[i] == -__builtin_inff()) ? 0.f : exp2_fast(sm_m[i] - M);
    Lsum += wgt[i] * sm_l[i];
  }
  const size_t sh = (size_t)seq * p.num_heads + head;
  if (direct) {
    const float inv = Lsum > 0.f ? p.v_scale / Lsum : 0.f;
    for (int d = tid; d < D; d += NW * 64) {
      float o = 0.f;
#pragma unroll
      for (int i = 0; i < NW; ++i) o += wgt[i] * sm_acc[i][d];
      store_elem<QT>(p.out, sh * D + d, o * inv);
    }
  } else {
    const size_t sp = sh * p.num_partitions + part;
    for (int d = tid; d < D; d += NW * 64) {
      float o = 0.f;
#pragma unroll
      for (int i = 0; i < NW; ++i) o += wgt[i] * sm_acc[i][d];
      p.ws_o[sp * D + d] = o * p.v_scale;
    }
    if (tid == 0) { p.ws_m[sp] = M; p.ws_l[sp] = Lsum; }
  }
}

// ---------------------------------------------------------------------------
// launcher: (q dtype, kv dtype, head_dim, block_size) -> instantiation
// ---------------------------------------------------------------------------
#ifndef PKV_VEC_NW
#define PKV_VEC_NW 4
#endif
#ifndef PKV_VEC_UNROLL
#define PKV_VEC_UNROLL 2
#endif
template <class QT, class KT, int D, int BS>
static hipError_t launch_vec(const AttnParams& p, hipStream_t stream) {
  constexpr int NW = PKV_VEC_NW;
  constexpr int NI = BS / (64 / (D * KT::bytes / 16));
  constexpr int UNROLL = NI <= 4 ? PKV_VEC_UNROLL : 1;   // keep small tiles in flight per wave
  hipLaunchKernelGGL((attn_vector_kernel<QT, KT, D, BS, NW, UNROLL>), dim3(p.total_wgs), dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <class QT, class KT, int D>
static hipError_t launch_vec_bs(const AttnParams& p, int bs, hipStream_t stream) {
  constexpr int LPR = D * KT::bytes / 16;
  constexpr int RPW = 64 / LPR;
  switch (bs) {
    case 8: if constexpr (8 % RPW == 0 && 8 / RPW <= 16) return launch_vec<QT, KT, D, 8>(p, stream); break;
    case 16: if constexpr (16 % RPW == 0 && 16 / RPW <= 16) return launch_vec<QT, KT, D, 16>(p, stream); break;
    case 32: if constexpr (32 % RPW == 0 && 32 / RPW <= 16) return launch_vec<QT, KT, D, 32>(p, stream); break;
  }
  return hipErrorInvalidValue;
}

template <class QT, class KT>
static hipError_t launch_vec_d(const AttnParams& p, int d, int bs, hipStream_t stream) {
  switch (d) {
    case 64: return launch_vec_bs<QT, KT, 64>(p, bs, stream);
    case 128: return launch_vec_bs<QT, KT, 128>(p, bs, stream);
    case 256: return launch_vec_bs<QT, KT, 256>(p, bs, stream);
  }
  return hipErrorInvalidValue;
}

bool vector_supported(int q_dtype, int kv_dtype, int d, int bs) {
  if (d != 64 && d != 128 && d != 256) return false;
  if (bs != 8 && bs != 16 && bs != 32) return false;
  int kv_bytes;
  if (q_dtype == 0 && kv_dtype == 0) kv_bytes = 4;
  else if ((q_dtype == 1 || q_dtype == 2) && kv_dtype == q_dtype) kv_bytes = 2;
  else if ((q_dtype == 1 || q_dtype == 2) && kv_dtype == 3) kv_bytes = 1;
  else return false;
  const int lpr = d * kv_bytes / 16;
  const int rpw = 64 / lpr;
  return lpr >= 1 && lpr <= 64 && bs % rpw == 0 && bs / rpw <= 16;
}

hipError_t launch_attention_vector(const AttnParams& p, int q_dtype, int kv_dtype, int d, int bs, hipStream_t stream) {
  if (q_dtype == 0 && kv_dtype == 0) return launch_vec_d<F32, F32>(p, d, bs, stream);
  if (q_dtype == 1 && kv_dtype == 1) return launch_vec_d<F16, F16>(p, d, bs, stream);
  if (q_dtype == 2 && kv_dtype == 2) return launch_vec_d<BF16, BF16>(p, d, bs, stream);
  if (q_dtype == 1 && kv_dtype == 3) return launch_vec_d<F16, FP8>(p, d, bs, stream);
  if (q_dtype == 2 && kv_dtype == 3) return launch_vec_d<BF16, FP8>(p, d, bs, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
