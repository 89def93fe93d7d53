// attn_reduce.hip -- merge of the per-partition summaries of a split context.
//
// Each (sequence, head, partition p) left (m_p, l_p, o_p): running max (log2
// domain), exp-sum and unnormalised output.  The merge is the identity of the
// online softmax ("PagedAttention", Ultralytics glossary, section "Các kỹ thuật
// liên quan": FlashAttention-style tiling never forms the score row):
//   M = max_p m_p;  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p
// Many partitions: D/32 256-thread workgroups per (sequence, head), each for
// 32 dims of the output row; threads read the partition maxima and sums in
// parallel, and 32 stripes of 8 threads walk the partitions with float4 loads
// of o_p (the first 8 of each stripe issued with the maxima and sums), then
// combine through LDS.  Few partitions: one wave per (sequence,
// head), see attn_reduce_small_kernel.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

template <class OT, int D>
__global__ __launch_bounds__(256) void attn_reduce_kernel(ReduceParams p) {
  constexpr int NT = 256;
  constexpr int DW = 32;                 // output dims of this workgroup
  constexpr int DS = D / DW;             // workgroups per (sequence, head)
  constexpr int CH = DW / 4;             // float4 chunks of the dims
  constexpr int STRIPES = NT / CH;       // partitions walked side by side
  static_assert(D % DW == 0, "head_dim a multiple of 32");
  const int sh = blockIdx.x / DS;        // sequence * num_heads + head
  const int d0 = (blockIdx.x - sh * DS) * DW;
  const int seq = sh / p.num_heads;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;

  int ctx = p.context_lens[seq];
  ctx = ctx < 0 ? 0 : (ctx > p.ctx_cap ? p.ctx_cap : ctx);
  const int np = (ctx + p.partition_tokens - 1) / p.partition_tokens;
  if (np <= 1) return;                                 // written by the attention kernel (whole workgroup)
  const size_t base = (size_t)sh * p.num_partitions;

  __shared__ float red[4];
  __shared__ float sm[STRIPES][DW];

  // Every load a thread needs first is issued before any reduction: the max and
  // sum of partition tid, and the rows (these dims) of its stripe's first PRE
  // partitions st, st + STRIPES, ...  The merge then waits on one memory
  // latency instead of three (maxima, sums, rows).
  constexpr int PRE = 8;
  const int c = tid % CH;
  const int st = tid / CH;
  float4 ov[PRE];
  float om[PRE];
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    const int i = st + k * STRIPES;
    ov[k] = i < np ? *reinterpret_cast<const float4*>(p.ws_o + (base + i) * D + d0 + c * 4)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
    om[k] = i < np ? p.ws_m[base + i] : -__builtin_inff();
  }
  const float m_own = tid < np ? p.ws_m[base + tid] : -__builtin_inff();
  const float l_own = tid < np ? p.ws_l[base + tid] : 0.f;

  float mx = m_own;
  for (int i = tid + NT; i < np; i += NT) mx = fmaxf(mx, p.ws_m[base + i]);
  mx = wave_max(mx);
  if (lane == 0) red[w] = mx;
  __syncthreads();
  float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  M = (M == -__builtin_inff()) ? 0.f : M;   // no live partition: every weight below is 0
  __syncthreads();

  float ls = exp2_fast(m_own - M) * l_own;
  for (int i = tid + NT; i < np; i += NT) ls += exp2_fast(p.ws_m[base + i] - M) * p.ws_l[base + i];
  ls = wave_sum(ls);
  if (lane == 0) red[w] = ls;
  __syncthreads();
  const float Lsum = (red[0] + red[1]) + (red[2] + red[3]);

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    const float wt = exp2_fast(om[k] - M);                // 0 past np
    acc.x += wt * ov[k].x; acc.y += wt * ov[k].y; acc.z += wt * ov[k].z; acc.w += wt * ov[k].w;
  }
#pragma unroll 4
  for (int i = st + PRE * STRIPES; i < np; i += STRIPES) {
    const float wt = exp2_fast(p.ws_m[base + i] - M);
    const float4 o = *reinterpret_cast<const float4*>(p.ws_o + (base + i) * D + d0 + c * 4);
    acc.x += wt * o.x; acc.y += wt * o.y; acc.z += wt * o.z; acc.w += wt * o.w;
  }
  sm[st][c * 4 + 0] = acc.x;
  sm[st][c * 4 + 1] = acc.y;
  sm[st][c * 4 + 2] = acc.z;
  sm[st][c * 4 + 3] = acc.w;
  __syncthreads();
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  for (int d = tid; d < DW; d += NT) {
    float o = 0.f;
#pragma unroll
    for (int s = 0; s < STRIPES; ++s) o += sm[s][d];
    store_elem<OT>(p.out, (size_t)sh * D + d0 + d, o * inv);
  }
}

// Few partitions (<= 64): one wave per (sequence, head), four per workgroup.
// Lane p holds partition p's max and sum; lane l accumulates dims
// [l*DV, l*DV+DV) over the partitions, reading each weight with a uniform
// readlane.  No barriers, no LDS.
template <class OT, int D>
__global__ __launch_bounds__(256) void attn_reduce_small_kernel(ReduceParams p) {
  constexpr int DV = D / 64;
  const int lane = threadIdx.x & 63;
  const int sh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (sh >= p.num_seqs * p.num_heads) return;          // whole wave exits together
  const int seq = sh / p.num_heads;
  int ctx = p.context_lens[seq];
  ctx = ctx < 0 ? 0 : (ctx > p.ctx_cap ? p.ctx_cap : ctx);
  const int np = (ctx + p.partition_tokens - 1) / p.partition_tokens;
  if (np <= 1) return;                                 // written by the attention kernel
  const size_t base = (size_t)sh * p.num_partitions;
  const float mp = lane < np ? p.ws_m[base + lane] : -__builtin_inff();
  const float lp = lane < np ? p.ws_l[base + lane] : 0.f;
  float M = wave_max(mp);
  M = (M == -__builtin_inff()) ? 0.f : M;
  const float wp = exp2_fast(mp - M);                  // 0 for lanes past np
  const float L = wave_sum(wp * lp);
  float acc[DV];
#pragma unroll
  for (int j = 0; j < DV; ++j) acc[j] = 0.f;
  const float* o = p.ws_o + base * D + lane * DV;
  for (int i0 = 0; i0 < np; i0 += 4) {                // four partitions' loads in flight at once
    float v[4][DV];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < DV; ++j) v[u][j] = i0 + u < np ? o[(size_t)(i0 + u) * D + j] : 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wp), i0 + u));
#pragma unroll
      for (int j = 0; j < DV; ++j) acc[j] += wi * v[u][j];
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int j = 0; j < DV; ++j) store_elem<OT>(p.out, (size_t)sh * D + lane * DV + j, acc[j] * inv);
}

// Balanced-slice mode: one wave per (sequence, head).  A sequence whose blocks
// all fall in one slice was written by the attention kernel; an empty one gets
// a zero row here; one that crosses slice boundaries k0..k1 has one summary
// row per slice (row ((k*2 + which) * H + head), which = 1 only for the slice
// where the sequence starts mid-slice) and is merged here.
template <class OT, int D>
__global__ __launch_bounds__(256) void attn_slice_finish_kernel(ReduceParams p) {
  constexpr int DV = D / 64;
  const int lane = threadIdx.x & 63;
  const int sh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (sh >= p.num_seqs * p.num_heads) return;           // whole wave exits together
  const int seq = sh / p.num_heads;
  const int h = sh - seq * p.num_heads;
  const int start = p.ws_prefix[seq], end = p.ws_prefix[seq + 1];
  if (start == end) {
#pragma unroll
    for (int j = 0; j < DV; ++j) store_elem<OT>(p.out, (size_t)sh * D + lane * DV + j, 0.f);
    return;
  }
  const int64_t T = p.ws_prefix[p.num_seqs];
  const int NS = p.num_slices;
  const int k0 = slice_of(start, T, NS), k1 = slice_of(end - 1, T, NS);
  if (k0 == k1) return;
  const int n = k1 - k0 + 1;
  const bool starts_inside = start > slice_begin(k0, T, NS);
  auto row_of = [&](int i) -> int64_t {
    return ((int64_t)(k0 + i) * 2 + ((i == 0 && starts_inside) ? 1 : 0)) * p.num_heads + h;
  };
  // a slice with no items (more slices than items) wrote no row: skip it
  auto live = [&](int i) -> bool { return slice_begin(k0 + i, T, NS) < slice_begin(k0 + i + 1, T, NS); };
  float M = -__builtin_inff();
  for (int i0 = 0; i0 < n; i0 += 64)
    if (i0 + lane < n && live(i0 + lane)) M = fmaxf(M, p.ws_m[row_of(i0 + lane)]);
  M = wave_max(M);
  M = (M == -__builtin_inff()) ? 0.f : M;
  float L = 0.f;
  float acc[DV];
#pragma unroll
  for (int j = 0; j < DV; ++j) acc[j] = 0.f;
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int cnt = n - i0 < 64 ? n - i0 : 64;
    const bool mine = lane < cnt && live(i0 + lane);
    const float wi = mine ? exp2_fast(p.ws_m[row_of(i0 + lane)] - M) : 0.f;
    L += mine ? wi * p.ws_l[row_of(i0 + lane)] : 0.f;
    const uint64_t live_mask = __ballot(mine);
    for (int j0 = 0; j0 < cnt; j0 += 4) {               // four rows' loads in flight at once
      float v[4][DV];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < DV; ++j)
          v[u][j] = (j0 + u < cnt && ((live_mask >> (j0 + u)) & 1))
                        ? p.ws_o[(size_t)row_of(i0 + j0 + u) * D + lane * DV + j] : 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wi), j0 + u));
#pragma unroll
        for (int j = 0; j < DV; ++j) acc[j] += wu * v[u][j];
      }
    }
  }
  L = wave_sum(L);
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int j = 0; j < DV; ++j) store_elem<OT>(p.out, (size_t)sh * D + lane * DV + j, acc[j] * inv);
}

template <class OT>
static hipError_t launch_reduce_d(const ReduceParams& p, int d, hipStream_t stream) {
  if (p.num_slices > 0) {
    const dim3 grid((unsigned)((p.num_seqs * p.num_heads + 3) / 4));
    switch (d) {
      case 64: hipLaunchKernelGGL((attn_slice_finish_kernel<OT, 64>), grid, dim3(256), 0, stream, p); break;
      case 128: hipLaunchKernelGGL((attn_slice_finish_kernel<OT, 128>), grid, dim3(256), 0, stream, p); break;
      case 256: hipLaunchKernelGGL((attn_slice_finish_kernel<OT, 256>), grid, dim3(256), 0, stream, p); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const int units = p.num_seqs * p.num_heads;
  if (p.num_partitions <= 64) {
    const dim3 grid((unsigned)((units + 3) / 4));
    switch (d) {
      case 64: hipLaunchKernelGGL((attn_reduce_small_kernel<OT, 64>), grid, dim3(256), 0, stream, p); break;
      case 128: hipLaunchKernelGGL((attn_reduce_small_kernel<OT, 128>), grid, dim3(256), 0, stream, p); break;
      case 256: hipLaunchKernelGGL((attn_reduce_small_kernel<OT, 256>), grid, dim3(256), 0, stream, p); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(units * (d / 32)));         // D/32 workgroups per (sequence, head)
  switch (d) {
    case 64: hipLaunchKernelGGL((attn_reduce_kernel<OT, 64>), grid, dim3(256), 0, stream, p); break;
    case 128: hipLaunchKernelGGL((attn_reduce_kernel<OT, 128>), grid, dim3(256), 0, stream, p); break;
    case 256: hipLaunchKernelGGL((attn_reduce_kernel<OT, 256>), grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention_reduce(const ReduceParams& p, int out_dtype, int d, hipStream_t stream) {
  if (out_dtype == 0) return launch_reduce_d<F32>(p, d, stream);
  if (out_dtype == 1) return launch_reduce_d<F16>(p, d, stream);
  if (out_dtype == 2) return launch_reduce_d<BF16>(p, d, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
