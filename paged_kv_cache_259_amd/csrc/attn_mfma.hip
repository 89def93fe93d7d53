// attn_mfma.hip -- paged decode attention for grouped-query heads on the
// CDNA4 matrix cores.  One workgroup per (sequence, kv head, context
// partition); the G query heads that share the kv head ("PagedAttention",
// Ultralytics glossary, section "Các kỹ thuật liên quan": grouped-query
// attention shares K/V heads between query heads) are the 16 columns of the
// MFMA tiles (padded with zero queries when G < 16), so each K/V tile is read
// from HBM once for the whole group.
//
// Per 16-token block (tile = 16 rows x D, contiguous):
//   QK:  S[token][head] = sum_k K[token][k] Q[head][k]
//        v_mfma_f32_16x16x32 (bf16/f16), A = K tile rows, B = Q^T, D/32 steps.
//        Lane l feeds token l%16, dims 32c + 8(l/16) .. +8 (one 16-byte load).
//        Result: lane l holds S[token 4(l/16)+r][head l%16], r = 0..3.
//   online softmax per head (column): block max over the 16 tokens = max over
//        the lane's 4 values, then over lanes l^16 and l^32.
//   PV:  O^T[dcol][head] += sum_k V[tok_k][8*dcol+e] P[head][tok_k]
//        v_mfma_f32_16x16x4 f32, A = V^T, B = P^T, one MFMA per (token group
//        tg, element e): lane l feeds V[4(l/16)+tg][8(l%16)+e] (from a plain
//        row-major 16-byte load of token 4(l/16)+tg) and P[head l%16][token
//        4(l/16)+tg] -- which is exactly register r = tg of its QK result, so
//        no shuffle or transpose is needed between the two products, and P
//        stays fp32.
//        O_e: lane l holds O[head l%16][dim 8(4(l/16)+r)+e], r = 0..3.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

template <class T> struct MfmaOp;
template <> struct MfmaOp<BF16> {
  typedef bf16x8_t vec;
  __device__ __forceinline__ static f32x4_t qk(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(vec, a), __builtin_bit_cast(vec, b), c, 0, 0, 0);
  }
};
template <> struct MfmaOp<F16> {
  typedef f16x8_t vec;
  __device__ __forceinline__ static f32x4_t qk(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(vec, a), __builtin_bit_cast(vec, b), c, 0, 0, 0);
  }
};

template <class T, int D, int NW, int UNROLL>
__global__ __launch_bounds__(NW * 64) void attn_mfma_kernel(AttnParams p) {
  constexpr int BS = 16;
  constexpr int NC = D / 32;                 // QK steps of 32 dims
  constexpr int NH = D / 128;                // 128-element halves of a V row (16 lanes x 8)
  constexpr size_t ROW_BYTES = (size_t)D * 2;
  constexpr size_t TILE_BYTES = ROW_BYTES * BS;
  static_assert(D % 128 == 0, "MFMA family needs head_dim 128 or 256");

  const uint32_t L = xcd_remap(blockIdx.x, p.total_wgs);
  int seq, kvh, part;
  decode_work_id(L, p.num_seqs, p.num_kv_heads, seq, kvh, part);
  const int G = p.group;

  int ctx = p.context_lens[seq];
  ctx = ctx < 0 ? 0 : (ctx > p.ctx_cap ? p.ctx_cap : ctx);
  const int nblk = (ctx + BS - 1) / BS;
  const int b_begin = part * p.partition_blocks;
  const bool direct = p.num_partitions == 1;
  if (!direct && b_begin >= nblk) return;
  int b_end = b_begin + p.partition_blocks;
  b_end = b_end < nblk ? b_end : nblk;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15;   // QK: token row of A / head column of B and of the result
  const int g4 = lane >> 4;    // 0..3

  // B operand of QK: Q[head c16][32c + 8 g4 .. +8]; zero for padding heads.
  uint4 qop[NC];
  {
    const bool real = c16 < G;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                           ((size_t)seq * p.num_heads + (size_t)kvh * G + (real ? c16 : 0)) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qop[c] = real ? *reinterpret_cast<const uint4*>(qrow + c * 32 + g4 * 8) : make_uint4(0u, 0u, 0u, 0u);
  }

  const int32_t* table = p.block_tables + (size_t)seq * p.max_blocks_per_seq;
  const char* kbase = reinterpret_cast<const char*>(p.k_cache) + (size_t)kvh * TILE_BYTES + c16 * ROW_BYTES + g4 * 16;
  const char* vbase = reinterpret_cast<const char*>(p.v_cache) + (size_t)kvh * TILE_BYTES + (g4 * 4) * ROW_BYTES + c16 * 16;
  const size_t block_stride = TILE_BYTES * (size_t)p.num_kv_heads;

  float m = -__builtin_inff();   // running max of head c16 (same in all four row groups)
  float lsum = 0.f;              // this lane's share of the running exp-sum of head c16
  f32x4_t O[NH][8];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) O[hh][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int last_partial = (ctx % BS) ? nblk - 1 : -1;

  for (int jb0 = b_begin + w; jb0 < b_end; jb0 += NW * UNROLL) {
    uint4 kr[UNROLL][NC];
    uint4 vr[UNROLL][4][NH];
    bool ok[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int jb = jb0 + u * NW;
      int blk = jb < b_end ? table[jb] : -1;
      ok[u] = blk >= 0 && blk < p.num_blocks;
      blk = ok[u] ? blk : 0;
      const char* kp = kbase + (size_t)blk * block_stride;
      const char* vp = vbase + (size_t)blk * block_stride;
      if (ok[u]) {
#pragma unroll
        for (int c = 0; c < NC; ++c) kr[u][c] = *reinterpret_cast<const uint4*>(kp + c * 64);
#pragma unroll
        for (int tg = 0; tg < 4; ++tg)
#pragma unroll
          for (int hh = 0; hh < NH; ++hh) vr[u][tg][hh] = *reinterpret_cast<const uint4*>(vp + tg * ROW_BYTES + hh * 256);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int jb = jb0 + u * NW;
      if (!ok[u]) continue;                         // wave-uniform
      f32x4_t S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) S = MfmaOp<T>::qk(kr[u][c], qop[c], S);
      float s[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) s[r] = S[r] * p.qk_scale;
      if (jb == last_partial) {                     // wave-uniform
        const int valid = ctx - jb * BS;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool v = g4 * 4 + r < valid;
          s[r] = v ? s[r] : -__builtin_inff();
          if (!v) {
#pragma unroll
            for (int hh = 0; hh < NH; ++hh) vr[u][r][hh] = make_uint4(0u, 0u, 0u, 0u);
          }
        }
      }
      float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      mx = fmaxf(mx, swz_xor16(mx));
      mx = fmaxf(mx, xor32(mx));
      const float mn = fmaxf(m, mx);                // finite: every block has a real token
      const float alpha = exp2_fast(m - mn);
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[r] = exp2_fast(s[r] - mn);
      lsum = lsum * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
      m = mn;
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) O[hh][e] *= alpha;
#pragma unroll
      for (int tg = 0; tg < 4; ++tg) {
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          float vf[8];
          Unpack<T>::run(vr[u][tg][hh], vf);
#pragma unroll
          for (int e = 0; e < 8; ++e) O[hh][e] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[e], pr[tg], O[hh][e], 0, 0, 0);
        }
      }
    }
  }

  lsum += swz_xor16(lsum);
  lsum += xor32(lsum);

  // merge the NW waves through LDS (only the G real heads)
  constexpr int RS = D + 1;                        // padded row stride against bank conflicts
  __shared__ float sm_m[NW][16], sm_l[NW][16];
  __shared__ float sm_o[NW][16 * RS];
  if (c16 < G) {
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm_o[w][c16 * RS + hh * 128 + (g4 * 4 + r) * 8 + e] = O[hh][e][r];
    if (g4 == 0) { sm_m[w][c16] = m; sm_l[w][c16] = lsum; }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += NW * 64) {
    const int h = idx / D;
    const int d = idx - h * D;
    float M = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < NW; ++i) M = fmaxf(M, sm_m[i][h]);
    float o = 0.f, Lsum = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const float wt = (sm_m[i][h] == -__builtin_inff()) ? 0.f : exp2_fast(sm_m[i][h] - M);
      Lsum += wt * sm_l[i][h];
      o += wt * sm_o[i][h * RS + d];
    }
    const size_t sh = (size_t)seq * p.num_heads + (size_t)kvh * G + h;
    if (direct) {
      store_elem<T>(p.out, sh * D + d, Lsum > 0.f ? o * (p.v_scale / Lsum) : 0.f);
    } else {
      const size_t sp = sh * p.num_partitions + part;
      p.ws_o[sp * D + d] = o * p.v_scale;
      if (d == 0) { p.ws_m[sp] = M; p.ws_l[sp] = Lsum; }
    }
  }
}

#ifndef PKV_MFMA_NW
#define PKV_MFMA_NW 4
#endif
#ifndef PKV_MFMA_UNROLL
#define PKV_MFMA_UNROLL 1
#endif
template <class T, int D>
static hipError_t launch_mfma(const AttnParams& p, hipStream_t stream) {
  constexpr int NW = PKV_MFMA_NW;
  constexpr int UNROLL = PKV_MFMA_UNROLL;
  hipLaunchKernelGGL((attn_mfma_kernel<T, D, NW, UNROLL>), dim3(p.total_wgs), dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

bool mfma_supported(int q_dtype, int kv_dtype, int d, int bs, int group) {
  return (q_dtype == 1 || q_dtype == 2) && kv_dtype == q_dtype && (d == 128 || d == 256) && bs == 16 &&
         group >= 2 && group <= 16;
}

hipError_t launch_attention_mfma(const AttnParams& p, int q_dtype, int d, hipStream_t stream) {
  if (q_dtype == 2) {
    if (d == 128) return launch_mfma<BF16, 128>(p, stream);
    if (d == 256) return launch_mfma<BF16, 256>(p, stream);
  } else if (q_dtype == 1) {
    if (d == 128) return launch_mfma<F16, 128>(p, stream);
    if (d == 256) return launch_mfma<F16, 256>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
