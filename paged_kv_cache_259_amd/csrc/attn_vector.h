// attn_vector.h -- paged decode attention, one workgroup per (sequence, query
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
//
// Two kernels share the body: attn_vector_kernel (plain decode) and
// attn_vector_append_kernel (decode that first writes each sequence's new K/V
// row).  attn_vector.hip instantiates the first, attn_append.hip the second.
#pragma once
#include "pkv_device.h"

namespace pkv {

// How far (log2 domain) a row group's running max may rise above the reference
// the weights are taken against before the accumulator is rescaled.
constexpr float kLazyRescaleVec = 8.f;

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

// NT: the K/V tiles are loaded with the non-temporal policy (see load_tile).
template <class QT, class KT, int D, int BS, int NW, bool NT>
struct VectorAttention {
  static constexpr int ELT = KT::bytes;
  static constexpr int VEC = 16 / ELT;        // elements per 16-byte load
  static constexpr int LPR = D * ELT / 16;    // lanes per token row
  static constexpr int RPW = 64 / LPR;        // token rows per wave-wide load
  static constexpr int NI = BS / RPW;         // loads per lane per tile
  static constexpr size_t ROW_BYTES = (size_t)D * ELT;
  static constexpr size_t TILE_BYTES = ROW_BYTES * BS;
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "row must split into whole lanes");
  static_assert(NI >= 1 && BS % RPW == 0, "block must hold whole row groups");

  struct Smem {
    float m[NW], l[NW];
    float acc[NW][D];
    alignas(16) int prefix[kMaxSliceSeqs + 4];
    int wsum[NW];
  };

  // Running softmax state of one lane (shared by the LPR lanes of its row group).
  struct State {
    float m, l, acc[VEC];
    __device__ void init() {
      m = -__builtin_inff();
      l = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
    }
  };

  // One block's tiles in registers.
  struct Tiles {
    uint4 k[NI], v[NI];
    bool ok;
  };

  // Every lane loads unconditionally, so the compiler can count the loads in
  // flight and wait only for the tile being consumed (a load under a per-lane
  // condition makes it wait for every load, the next tile's too).  kpool /
  // vpool point at kv head kvh's tile of block 0 (wave-uniform), lane_off is
  // the lane's byte offset inside a tile.  A row at or past `valid` (the last
  // block's tail) reads the block's last real row instead -- the same cache
  // lines, no extra memory traffic -- and consume masks it.  A table entry
  // outside the pool, or a block loaded only to keep the loads unconditional
  // (!live), reads no memory (see load_tile); consume skips the former and
  // never sees the latter.
  __device__ static void issue(const AttnParams& p, const char* kpool, const char* vpool, size_t block_stride,
                               uint32_t lane_off, int blk, int valid, int row, bool live, Tiles& t) {
    t.ok = blk >= 0 && blk < p.num_blocks;                  // out-of-pool entries are skipped
    const size_t boff = (size_t)(t.ok ? blk : 0) * block_stride;
    const int bytes = t.ok && live ? TILE_BYTES : 0;
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kpool + boff, bytes), vr = buffer_rsrc(vpool + boff, bytes);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = i * RPW + row;                            // valid >= 1: every block has a real token
      const uint32_t off = lane_off + (uint32_t)(((r < valid ? r : valid - 1) - row) * ROW_BYTES);
      t.k[i] = load_tile<uint4, NT>(kr, off);
      t.v[i] = load_tile<uint4, NT>(vr, off);
    }
  }

  __device__ static void consume(const AttnParams& p, const QFrag<QT, KT, VEC>& qf, Tiles& t, int jb, int ctx,
                                 int last_partial, int row, State& st) {
    if (!t.ok) return;                                      // wave-uniform
    float s[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) s[i] = group_sum<LPR>(qf.dot(t.k[i])) * p.qk_scale;
    if (jb == last_partial) {                               // wave-uniform
      const int valid = ctx - jb * BS;                      // 1 .. BS-1 tokens of this block are real
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const bool v = i * RPW + row < valid;
        s[i] = v ? s[i] : -__builtin_inff();
        if (!v) t.v[i] = make_uint4(0u, 0u, 0u, 0u);        // tail slots may hold NaN: drop, never multiply
      }
    }
    float mb = s[0];
#pragma unroll
    for (int i = 1; i < NI; ++i) mb = fmaxf(mb, s[i]);
    // The reference max st.m moves only when the row group's max exceeds it by
    // more than kLazyRescaleVec (log2 domain), so the accumulator is rescaled on
    // few blocks (a wave-uniform branch); the weights stay below 2^kLazyRescaleVec
    // and the softmax does not depend on the reference.
    const bool grow = mb > st.m + kLazyRescaleVec;        // a row with no token yet: mb = -inf, no growth
    if (__builtin_amdgcn_ballot_w64(grow)) {
      // 0 on a row group's first real block; rows that did not grow keep their
      // scale (and a row with no token yet, m = -inf, must not form -inf - -inf)
      const float alpha = grow ? exp2_fast(st.m - mb) : 1.f;
      const float mn = grow ? mb : st.m;
      st.l *= alpha;
#pragma unroll
      for (int e = 0; e < VEC; ++e) st.acc[e] *= alpha;
      st.m = mn;
    }
    const bool live = st.m != -__builtin_inff();          // false only for a row with no token yet
    float pr[NI];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      pr[i] = live ? exp2_fast(s[i] - st.m) : 0.f;
      psum += pr[i];
    }
    st.l += psum;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float vf[VEC];
      Unpack<KT>::run(t.v[i], vf);
#pragma unroll
      for (int e = 0; e < VEC; ++e) st.acc[e] = __builtin_fmaf(pr[i], vf[e], st.acc[e]);
    }
  }

  // Blocks [j0, j1) of sequence `seq` for query head `head`; wave w takes
  // blocks j0 + w, j0 + w + NW, ...  Software-pipelined: the next block's
  // tiles are in flight while the current one is consumed.  The wave's block
  // ids are read 64 at a time into one VGPR (lane t holds the t-th id) and
  // taken out with readlane, so no table load sits on the critical path.
  __device__ static void attend(const AttnParams& p, int seq, int head, int ctx, int j0, int j1, int w, int row,
                                int col, State& st) {
    const int first = j0 + w;
    const int n = first < j1 ? (j1 - first + NW - 1) / NW : 0;   // blocks of this wave
    if (n == 0) return;                                      // wave-uniform
    const int kvh = head / p.group;
    QFrag<QT, KT, VEC> qf;
    qf.load(p.q, ((size_t)seq * p.num_heads + head) * D + (size_t)col * VEC);
    const int32_t* table = p.block_tables + (size_t)seq * p.max_blocks_per_seq;
    const char* kpool = reinterpret_cast<const char*>(p.k_cache) + (size_t)kvh * TILE_BYTES;
    const char* vpool = reinterpret_cast<const char*>(p.v_cache) + (size_t)kvh * TILE_BYTES;
    const uint32_t lane_off = (uint32_t)(row * ROW_BYTES + col * 16);
    const size_t block_stride = TILE_BYTES * (size_t)p.num_kv_heads;
    const int last_partial = (ctx % BS) ? (ctx + BS - 1) / BS - 1 : -1;
    const int lane = threadIdx.x & 63;
    auto load_ids = [&](int chunk) -> int {
      const int i = chunk * 64 + lane;
      return i < n ? table[first + i * NW] : -1;
    };
    int ids = load_ids(0);
    int ids_next = n > 64 ? load_ids(1) : -1;
    int chunk = 0;
    auto id_of = [&](int i) -> int {                         // called with i = 0, 1, 2, ... in order
      if ((i >> 6) != chunk) {
        chunk = i >> 6;
        ids = ids_next;
        ids_next = (chunk + 1) * 64 < n ? load_ids(chunk + 1) : -1;
      }
      return __builtin_amdgcn_readlane(ids, i & 63);
    };
    auto valid_of = [&](int i) -> int {                      // real tokens in the wave's i-th block
      const int r = ctx - (first + i * NW) * BS;
      return r < BS ? r : BS;
    };
    // Both tile sets are refilled on every pass, also past the wave's last
    // block (issued for block n - 1 again but reading no memory, never
    // consumed): loads under a branch would make the compiler wait for all
    // loads in flight before each consume instead of only the consumed tile's.
    Tiles a, b;
    issue(p, kpool, vpool, block_stride, lane_off, id_of(0), valid_of(0), row, true, a);
    for (int i = 0; i < n; i += 2) {
      const int i1 = i + 1 < n ? i + 1 : n - 1;
      const int i2 = i + 2 < n ? i + 2 : n - 1;
      issue(p, kpool, vpool, block_stride, lane_off, id_of(i1), valid_of(i1), row, i + 1 < n, b);
      consume(p, qf, a, first + i * NW, ctx, last_partial, row, st);
      issue(p, kpool, vpool, block_stride, lane_off, id_of(i2), valid_of(i2), row, i + 2 < n, a);
      if (i + 1 < n) consume(p, qf, b, first + (i + 1) * NW, ctx, last_partial, row, st);
    }
  }

  // Merge row groups (shuffles) and waves (LDS), then write the normalised
  // output row (prow < 0) or the fp32 summary row `prow` of the workspace.
  // Every thread of the workgroup calls it; it ends with a barrier so the LDS
  // can be reused.
  __device__ static void finish(const AttnParams& p, State& st, Smem& sm, int seq, int head, int64_t prow, int tid,
                                int w, int row, int col) {
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(st.m, off, 64);
      const float l2 = __shfl_xor(st.l, off, 64);
      const float mn = fmaxf(st.m, m2);
      const float a = (st.m == -__builtin_inff()) ? 0.f : exp2_fast(st.m - mn);
      const float b = (m2 == -__builtin_inff()) ? 0.f : exp2_fast(m2 - mn);
      st.l = st.l * a + l2 * b;
#pragma unroll
      for (int e = 0; e < VEC; ++e) st.acc[e] = st.acc[e] * a + __shfl_xor(st.acc[e], off, 64) * b;
      st.m = mn;
    }
    if (row == 0) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) sm.acc[w][col * VEC + e] = st.acc[e];
      if (col == 0) { sm.m[w] = st.m; sm.l[w] = st.l; }
    }
    __syncthreads();
    float M = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < NW; ++i) M = fmaxf(M, sm.m[i]);
    float wgt[NW];
    float Lsum = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      wgt[i] = (sm.m[i] == -__builtin_inff()) ? 0.f : exp2_fast(sm.m[i] - M);
      Lsum += wgt[i] * sm.l[i];
    }
    if (prow < 0) {
      const size_t sh = (size_t)seq * p.num_heads + head;
      const float inv = Lsum > 0.f ? p.v_scale / Lsum : 0.f;
      for (int d = tid; d < D; d += NW * 64) {
        float o = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) o += wgt[i] * sm.acc[i][d];
        store_elem<QT>(p.out, sh * D + d, o * inv);
      }
    } else {
      for (int d = tid; d < D; d += NW * 64) {
        float o = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) o += wgt[i] * sm.acc[i][d];
        p.ws_o[(size_t)prow * D + d] = o * p.v_scale;
      }
      if (tid == 0) { p.ws_m[prow] = M; p.ws_l[prow] = Lsum; }
    }
    __syncthreads();
  }
};

// Waves per SIMD the register budget allows: two tiles (K and V, NI 16-byte
// loads each) in flight, the accumulator and the query slice, plus ~40 others.
template <class KT, int D, int BS>
constexpr int vector_waves_per_eu() {
  constexpr int VEC = 16 / KT::bytes;
  constexpr int NI = BS / (64 / (D * KT::bytes / 16));
  constexpr int est = 16 * NI + 3 * VEC + 40;
  constexpr int w = 512 / est;
  return w < 1 ? 1 : (w > 8 ? 8 : w);
}
#ifndef PKV_VEC_WAVES_PER_EU
#define PKV_VEC_WAVES_PER_EU 0   // 0: from the tile size
#endif
template <class QT, class KT, int D, int BS, int NW, bool NT, bool APPEND>
__device__ __forceinline__ void attn_vector_body(AttnParams p) {
  using A = VectorAttention<QT, KT, D, BS, NW, NT>;
  __shared__ typename A::Smem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane / A::LPR;
  const int col = lane % A::LPR;
  const uint32_t L = p.head_run_units ? head_runs(blockIdx.x, p.head_run_units)
                                       : xcd_remap(blockIdx.x, p.total_wgs, p.xcd_chunk);
  typename A::State st;

  if (p.num_slices > 0) {
    // balanced slices: head fastest, then slice
    const int head = (int)(L % (uint32_t)p.num_heads);
    apply_head_scales(p, head / p.group);
    const int k = (int)(L / (uint32_t)p.num_heads);
    const int S = p.num_seqs;
    block_prefix<NW * 64>(p.context_lens, S, p.ctx_cap, BS, sm.prefix, sm.wsum);
    if (blockIdx.x == 0)
      for (int i = tid; i <= S; i += NW * 64) p.ws_prefix[i] = sm.prefix[i];
    const int64_t total = sm.prefix[S];
    const int64_t a = slice_begin(k, total, p.num_slices), b = slice_begin(k + 1, total, p.num_slices);
    if (a >= b) return;                                     // empty slice (uniform)
    int lo = 1, hi = S;                                     // first i with prefix[i] > a
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sm.prefix[mid] > a) hi = mid; else lo = mid + 1;
    }
    int s = lo - 1;
    int64_t pos = a;
    while (pos < b) {
      const int start = sm.prefix[s], end = sm.prefix[s + 1];
      const int j0 = (int)(pos - start);
      const int j1 = (int)((b < end ? b : end) - start);
      const bool complete = start >= a && end <= b;
      const int which = start <= a ? 0 : 1;              // first or last segment of this slice
      int ctx = p.context_lens[s];
      ctx = ctx < 0 ? 0 : (ctx > p.ctx_cap ? p.ctx_cap : ctx);
      if (APPEND && j1 == end - start)                      // this segment holds the sequence's last block
        append_new_row<QT, KT, D, BS, NW * 64>(p, s, head / p.group, (j1 - 1 - j0) % NW);
      st.init();
      A::attend(p, s, head, ctx, j0, j1, w, row, col, st);
      const int64_t prow = complete ? -1 : ((int64_t)k * 2 + which) * p.num_heads + head;
      A::finish(p, st, sm, s, head, prow, tid, w, row, col);
      pos = end;
      ++s;
      while (s < S && sm.prefix[s + 1] <= pos) ++s;        // skip empty contexts
    }
    return;
  }

  // fixed partitions of partition_blocks blocks (one pass when num_partitions == 1)
  int seq, head, part;
  decode_work_id(L, p.num_seqs, p.num_heads, seq, head, part);
  // Fixed partitions: the last partition index first.  Shorter contexts have
  // no partition at the high indices, so the workgroups that find nothing to do
  // are dispatched while the GPU fills, and the grid ends with low partitions,
  // which every context has.
  if (p.num_partitions > 1 && PKV_PARTITIONS_REVERSED) part = p.num_partitions - 1 - part;
  apply_head_scales(p, head / p.group);
  if (p.longest_first) {                                    // one pass only
    if (p.seq_order) {
      const int o = p.seq_order[seq];
      seq = o < 0 ? 0 : (o >= p.num_seqs ? p.num_seqs - 1 : o);
    } else {
      seq = seq_of_rank<NW * 64>(p.context_lens, p.num_seqs, p.ctx_cap, BS, seq, sm.prefix, sm.wsum);
    }
  }
  int ctx = p.context_lens[seq];
  ctx = ctx < 0 ? 0 : (ctx > p.ctx_cap ? p.ctx_cap : ctx);
  const int nblk = (ctx + BS - 1) / BS;
  const int b_begin = part * p.partition_blocks;
  // a context that fits in one partition is finished here; the reduce skips it
  const bool direct = p.num_partitions == 1 || nblk <= p.partition_blocks;
  if (b_begin >= nblk && (part > 0 || !direct)) return;     // empty partition
  int b_end = b_begin + p.partition_blocks;
  b_end = b_end < nblk ? b_end : nblk;
  if (APPEND && nblk > 0 && b_end == nblk)                  // this workgroup reads the last block
    append_new_row<QT, KT, D, BS, NW * 64>(p, seq, head / p.group, (nblk - 1 - b_begin) % NW);
  st.init();
  A::attend(p, seq, head, ctx, b_begin, b_end, w, row, col, st);
  const int64_t prow = direct ? -1 : ((int64_t)seq * p.num_heads + head) * p.num_partitions + part;
  A::finish(p, st, sm, seq, head, prow, tid, w, row, col);
}

template <class QT, class KT, int D, int BS, int NW, bool NT>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(PKV_VEC_WAVES_PER_EU ? PKV_VEC_WAVES_PER_EU : vector_waves_per_eu<KT, D, BS>())))
void attn_vector_kernel(AttnParams p) {
  attn_vector_body<QT, KT, D, BS, NW, NT, false>(p);
}

template <class QT, class KT, int D, int BS, int NW, bool NT>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(PKV_VEC_WAVES_PER_EU ? PKV_VEC_WAVES_PER_EU : vector_waves_per_eu<KT, D, BS>())))
void attn_vector_append_kernel(AttnParams p) {
  attn_vector_body<QT, KT, D, BS, NW, NT, true>(p);
}

// ---------------------------------------------------------------------------
// launcher: (q dtype, kv dtype, head_dim, block_size) -> instantiation
// ---------------------------------------------------------------------------
#ifndef PKV_VEC_NW
#define PKV_VEC_NW 4
#endif
template <bool APPEND, class QT, class KT, int D, int BS, bool NT>
static hipError_t launch_vec_nt(const AttnParams& p, hipStream_t stream) {
  constexpr int NW = PKV_VEC_NW;
  if constexpr (APPEND)
    hipLaunchKernelGGL((attn_vector_append_kernel<QT, KT, D, BS, NW, NT>), dim3(p.total_wgs), dim3(NW * 64), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((attn_vector_kernel<QT, KT, D, BS, NW, NT>), dim3(p.total_wgs), dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <bool APPEND, class QT, class KT, int D, int BS>
static hipError_t launch_vec(const AttnParams& p, hipStream_t stream) {
  return p.kv_cached ? launch_vec_nt<APPEND, QT, KT, D, BS, false>(p, stream)
                     : launch_vec_nt<APPEND, QT, KT, D, BS, true>(p, stream);
}

template <bool APPEND, class QT, class KT, int D>
static hipError_t launch_vec_bs(const AttnParams& p, int bs, hipStream_t stream) {
  constexpr int LPR = D * KT::bytes / 16;
  constexpr int RPW = 64 / LPR;
  switch (bs) {
    case 8: if constexpr (8 % RPW == 0 && 8 / RPW <= 16) return launch_vec<APPEND, QT, KT, D, 8>(p, stream); break;
    case 16: if constexpr (16 % RPW == 0 && 16 / RPW <= 16) return launch_vec<APPEND, QT, KT, D, 16>(p, stream); break;
    case 32: if constexpr (32 % RPW == 0 && 32 / RPW <= 16) return launch_vec<APPEND, QT, KT, D, 32>(p, stream); break;
  }
  return hipErrorInvalidValue;
}

template <bool APPEND, class QT, class KT>
static hipError_t launch_vec_d(const AttnParams& p, int d, int bs, hipStream_t stream) {
  switch (d) {
    case 64: return launch_vec_bs<APPEND, QT, KT, 64>(p, bs, stream);
    case 128: return launch_vec_bs<APPEND, QT, KT, 128>(p, bs, stream);
    case 256: return launch_vec_bs<APPEND, QT, KT, 256>(p, bs, stream);
  }
  return hipErrorInvalidValue;
}

// (q dtype, kv dtype) -> instantiation; the combinations vector_supported accepts.
template <bool APPEND>
static hipError_t launch_vector_family(const AttnParams& p, int q_dtype, int kv_dtype, int d, int bs,
                                       hipStream_t stream) {
  if (q_dtype == 0 && kv_dtype == 0) return launch_vec_d<APPEND, F32, F32>(p, d, bs, stream);
  if (q_dtype == 1 && kv_dtype == 1) return launch_vec_d<APPEND, F16, F16>(p, d, bs, stream);
  if (q_dtype == 2 && kv_dtype == 2) return launch_vec_d<APPEND, BF16, BF16>(p, d, bs, stream);
  if (q_dtype == 1 && kv_dtype == 3) return launch_vec_d<APPEND, F16, FP8>(p, d, bs, stream);
  if (q_dtype == 2 && kv_dtype == 3) return launch_vec_d<APPEND, BF16, FP8>(p, d, bs, stream);
  if (q_dtype == 1 && kv_dtype == 4) return launch_vec_d<APPEND, F16, BF8>(p, d, bs, stream);
  if (q_dtype == 2 && kv_dtype == 4) return launch_vec_d<APPEND, BF16, BF8>(p, d, bs, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
