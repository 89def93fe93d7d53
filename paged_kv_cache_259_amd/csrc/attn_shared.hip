// attn_shared.hip -- decode for groups of sequences whose block tables start
// with the same physical blocks: the samples forked from one prompt
// ([KVpag] "KV cache paginado e batching contínuo para LLMs", section "Como
// funciona": forks share blocks through reference counts; "PagedAttention"
// glossary, section "Chia sẻ block giữa các chuỗi": parallel samples and beams
// share the prompt's blocks).
//
// The result is the same attention as pkv_paged_attention_decode (up to
// rounding order); what changes is how often a shared block is read.  One
// workgroup per (group, kv head) runs the matrix-core body of attn_mfma.h with
// the group's queries as the MFMA columns: column c is query head
// kvh*G + c%G of member c/G.  It walks
//   1. the shared blocks once, every member's columns taking part, then
//   2. each member's own blocks (the rest of its table), only that member's
//      columns taking part (the others keep their softmax state untouched),
// and writes every member's normalised output rows.  So a block shared by n
// samples comes from memory once instead of n times, with no partial results
// written out and no second launch.  With append, the wave that will read a
// member's last block first writes its new K/V row (as attn_append.hip).
#include "attn_mfma.h"
#include "pkv_internal.h"

namespace pkv {

template <class T, class KT, int D, int NW, bool APPEND>
__device__ __forceinline__ void attn_shared_body(AttnParams p) {
  using A = MfmaAttention<T, KT, D, NW, true, true>;   // non-temporal loads: the group reads each block once
  constexpr int BS = A::BS;
  __shared__ typename A::Smem sm;
  __shared__ int s_seq[16];                                 // member of each group of G columns, -1 if none
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15;
  const int g4 = lane >> 4;
  const uint32_t L = p.head_run_units ? head_runs(blockIdx.x, p.head_run_units)
                                       : xcd_remap(blockIdx.x, p.total_wgs, p.xcd_chunk);
  const int kvh = (int)(L % (uint32_t)p.num_kv_heads);
  const int grp = (int)(L / (uint32_t)p.num_kv_heads);
  apply_head_scales(p, kvh);
  const int G = p.group;
  const int S = p.num_seqs;
  int o0 = p.grp_off[grp], o1 = p.grp_off[grp + 1];
  o0 = o0 < 0 ? 0 : (o0 > S ? S : o0);
  const int o1max = o0 + p.grp_max < S ? o0 + p.grp_max : S;
  o1 = o1 < o0 ? o0 : (o1 > o1max ? o1max : o1);
  const int nm = __builtin_amdgcn_readfirstlane(o1 - o0);
  // lane i < nm: member i's sequence (-1 when out of range) and clamped context
  int mseq = -1, mctx = 0;
  if (lane < nm) {
    const int s = p.grp_mem[o0 + lane];
    if (s >= 0 && s < S) {
      const int c = p.context_lens[s];
      mseq = s;
      mctx = c < 0 ? 0 : (c > p.ctx_cap ? p.ctx_cap : c);
    }
  }
  if (tid < 16) s_seq[tid] = tid < nm ? mseq : -1;
  // Shared blocks: the caller's count, kept below every member's newest token
  // (so a member's last block, which it may be writing, is always its own).
  int lim = mseq >= 0 ? (mctx > 0 ? (mctx - 1) / BS : 0) : 0x7fffffff;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_xor(lim, off, 64);
    lim = o < lim ? o : lim;
  }
  int nsh = p.grp_shared[grp];
  nsh = nsh < 0 ? 0 : (nsh > lim ? lim : nsh);
  nsh = __builtin_amdgcn_readfirstlane(nsh);
  const uint64_t valid = __builtin_amdgcn_ballot_w64(mseq >= 0);
  if (valid == 0) return;                                   // uniform: nothing to do
  const int lead = __builtin_ffsll((long long)valid) - 1;   // its table names the shared blocks

  const int mi = c16 / G;                                   // this lane's column belongs to member mi
  const int cseq = __shfl(mseq, mi, 64);
  const bool real = c16 < nm * G && cseq >= 0;
  typename A::State st;
  st.init();
  uint4 qop[A::NC];
  A::load_q(p, real, ((size_t)(real ? cseq : 0) * p.num_heads + (size_t)kvh * G + (c16 - mi * G)) * D, g4, qop);
  if (nsh > 0) {
    const int s = __builtin_amdgcn_readlane(mseq, lead);
    const int ctx = __builtin_amdgcn_readlane(mctx, lead);
    A::template walk<true>(p, p.block_tables + (size_t)s * p.max_blocks_per_seq, kvh, ctx, 0, nsh, w, c16, g4,
                           sm.vt[w], st, qop, real);
  }
  for (int i = 0; i < nm; ++i) {
    const int s = __builtin_amdgcn_readlane(mseq, i);
    if (s < 0) continue;                                    // uniform
    const int ctx = __builtin_amdgcn_readlane(mctx, i);
    const int nblk = (ctx + BS - 1) / BS;
    if (APPEND && nblk > 0)                                 // the member's last block is read by wave (nblk-1-nsh)%NW
      append_new_row<T, KT, D, BS, NW * 64>(p, s, kvh, (nblk - 1 - nsh) % NW);
    A::template walk<true>(p, p.block_tables + (size_t)s * p.max_blocks_per_seq, kvh, ctx, nsh, nblk, w, c16, g4,
                           sm.vt[w], st, qop, real && mi == i);
  }
  A::merge(st, sm, nm * G, tid, w, c16, g4, [&](int h, int d, float M, float Lsum, float o) {
    (void)M;
    const int s = s_seq[h / G];
    if (s >= 0) {
      const size_t row = (size_t)s * p.num_heads + (size_t)kvh * G + (h - (h / G) * G);
      store_elem<T>(p.out, row * D + d, Lsum > 0.f ? o * (p.v_scale / Lsum) : 0.f);
    }
  });
}

#ifndef PKV_SHARED_WAVES_PER_EU
#define PKV_SHARED_WAVES_PER_EU PKV_MFMA_WAVES_PER_EU_PIPE
#endif
#define PKV_SHARED_WAVES(D) ((D) == 128 ? PKV_SHARED_WAVES_PER_EU : 1)
template <class T, class KT, int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(PKV_SHARED_WAVES(D))))
void attn_shared_kernel(AttnParams p) {
  attn_shared_body<T, KT, D, NW, false>(p);
}

template <class T, class KT, int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(PKV_SHARED_WAVES(D))))
void attn_shared_append_kernel(AttnParams p) {
  attn_shared_body<T, KT, D, NW, true>(p);
}

// Waves per workgroup.  The grid is one workgroup per (group, kv head), often
// only a few per compute unit.  With plain K/V loads 2 waves measured faster
// (every wave of such a grid resident from the start, walking twice the
// blocks).  With the non-temporal loads, on the shared-prefix E4M3 workload
// (1280 workgroups): 2 waves 129.8-130.1 us, 4 waves 128.7-129.6 us, 3 waves
// 127.9-128.0 us, 8 waves 129.6-129.9 us.
#ifndef PKV_SHARED_NW
#define PKV_SHARED_NW 3
#endif
template <class T, class KT, int D>
static hipError_t launch_shared(const AttnParams& p, bool append, hipStream_t stream) {
  constexpr int NW = PKV_SHARED_NW;
  if (append)
    hipLaunchKernelGGL((attn_shared_append_kernel<T, KT, D, NW>), dim3(p.total_wgs), dim3(NW * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_shared_kernel<T, KT, D, NW>), dim3(p.total_wgs), dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <class T, class KT>
static hipError_t launch_shared_d(const AttnParams& p, int d, bool append, hipStream_t stream) {
  if (d == 128) return launch_shared<T, KT, 128>(p, append, stream);
  if (d == 256) return launch_shared<T, KT, 256>(p, append, stream);
  return hipErrorInvalidValue;
}

bool shared_supported(int q_dtype, int kv_dtype, int d, int bs) {
  return (q_dtype == F16::kId || q_dtype == BF16::kId) &&
         (kv_dtype == q_dtype || kv_dtype == FP8::kId || kv_dtype == BF8::kId) && (d == 128 || d == 256) && bs == 16;
}

// (q dtype, kv dtype, head_dim) -> instantiation; the cases shared_supported accepts.
hipError_t launch_attention_shared(const AttnParams& p, int q_dtype, int kv_dtype, int d, bool append,
                                   hipStream_t stream) {
  if (q_dtype == BF16::kId) {
    if (kv_dtype == BF16::kId) return launch_shared_d<BF16, BF16>(p, d, append, stream);
    if (kv_dtype == FP8::kId) return launch_shared_d<BF16, FP8>(p, d, append, stream);
    if (kv_dtype == BF8::kId) return launch_shared_d<BF16, BF8>(p, d, append, stream);
  } else if (q_dtype == F16::kId) {
    if (kv_dtype == F16::kId) return launch_shared_d<F16, F16>(p, d, append, stream);
    if (kv_dtype == FP8::kId) return launch_shared_d<F16, FP8>(p, d, append, stream);
    if (kv_dtype == BF8::kId) return launch_shared_d<F16, BF8>(p, d, append, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
