// attn_mfma.h -- paged decode attention for grouped-query heads on the
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
//   PV:  O^T[dim][head] += sum_k V^T[dim][tok_k] P^T[tok_k][head]
//        v_mfma_f32_16x16x16 (f16/bf16), one per 16 dims.  B = P^T: the
//        contraction index of lane group l/16 is tokens 4(l/16) .. +3, which
//        are exactly the lane's four QK results, so nothing moves between the
//        two products.  P enters as its 16-bit rounding plus the 16-bit
//        rounding of the remainder (two MFMAs), about 16 bits of each weight.
//        A = V^T: each wave stages its V tile (row-major, q's type) in its own
//        LDS rows and reads it back with the transposing ds_read_b64_tr_b16.
//        O[dt]: lane l holds O[head l%16][dim 16 dt + 4(l/16) + r], r = 0..3.
//
// 8-bit caches (E4M3, E5M2; "PagedAttention", Ultralytics glossary, section
// "Các kỹ thuật liên quan": an 8-bit KV cache) read half the bytes.  K codes are
// converted exactly to q's 16-bit type for the QK MFMA (lane group l/16 then
// holds dims D/4 (l/16) .. +D/4 of its token, two 16-byte loads at D = 128, and
// the query operand follows that contraction order); V codes likewise before
// they are staged for the PV MFMA.  k_scale scales the logits, v_scale the
// output.
//
// Two kernels share the body: attn_mfma_kernel (plain decode) and
// attn_mfma_append_kernel (decode that first writes each sequence's new K/V
// row).  attn_mfma.hip instantiates the first, attn_append.hip the second.
#pragma once
#include <type_traits>

#include "pkv_device.h"

namespace pkv {

// How far (log2 domain) a head's running max may rise above the reference the
// weights are taken against before the accumulators are rescaled.
constexpr float kLazyRescale = 8.f;

template <class T> struct MfmaOp;
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
template <> struct MfmaOp<BF16> {
  typedef bf16x8_t vec;
  __device__ __forceinline__ static f32x4_t qk(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(vec, a), __builtin_bit_cast(vec, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static f32x4_t pv(const uint2& a, const uint2& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b), c,
                                                     0, 0, 0);
  }
  // p rounded to bf16, and what that rounding left out, rounded again
  __device__ __forceinline__ static void split(const float* p, uint2& hi, uint2& lo) {
    bf16x4_t h = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};
    bf16x4_t l = {(__bf16)(p[0] - (float)h[0]), (__bf16)(p[1] - (float)h[1]), (__bf16)(p[2] - (float)h[2]),
                  (__bf16)(p[3] - (float)h[3])};
    hi = __builtin_bit_cast(uint2, h);
    lo = __builtin_bit_cast(uint2, l);
  }
};
template <> struct MfmaOp<F16> {
  typedef f16x8_t vec;
  __device__ __forceinline__ static f32x4_t qk(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(vec, a), __builtin_bit_cast(vec, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static f32x4_t pv(const uint2& a, const uint2& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a), __builtin_bit_cast(f16x4_t, b), c, 0,
                                                 0, 0);
  }
  __device__ __forceinline__ static void split(const float* p, uint2& hi, uint2& lo) {
    f16x4_t h = {(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
    f16x4_t l = {(_Float16)(p[0] - (float)h[0]), (_Float16)(p[1] - (float)h[1]), (_Float16)(p[2] - (float)h[2]),
                 (_Float16)(p[3] - (float)h[3])};
    hi = __builtin_bit_cast(uint2, h);
    lo = __builtin_bit_cast(uint2, l);
  }
};

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
// ds_read_b64_tr_b16 (8-byte aligned LDS address): within each 16-lane group,
// output lane j gets element j%4 of the 4 elements at lane 4m + j/4's address,
// m = 0..3.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* lds) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds)));
}

// T: the q type and MFMA operand type (f16 / bf16); KT: the cache type, T itself
// or one of the 8-bit formats.
// NT: the K/V tiles are loaded with the non-temporal policy (see load_tile).
template <class T, class KT, int D, int NW, bool PIPE, bool NT>
struct MfmaAttention {
  static constexpr int BS = 16;
  static constexpr int NC = D / 32;                 // QK steps of 32 dims
  static constexpr int NH = D / 128;                // 128-element halves of a V row (16 lanes x 8)
  static constexpr bool KV8 = KT::bytes == 1;
  static constexpr size_t ROW_BYTES = (size_t)D * KT::bytes;
  static constexpr size_t TILE_BYTES = ROW_BYTES * BS;
  static constexpr int NK = KV8 ? NC / 2 : NC;      // 16-byte K loads per lane per block
  // QK contraction order.  16-bit: MFMA step c takes dims 32c + 8 g4 .. +8 of
  // lane group g4 (one 16-byte load per step).  8-bit: lane group g4 holds the
  // contiguous dims g4 D/4 .. +D/4 (D/4 bytes, whole 16-byte loads) and step c
  // takes 8 of them; the query operand follows the same order.
  __device__ __forceinline__ static int k_dim(int c, int g4) { return KV8 ? g4 * (D / 4) + 8 * c : 32 * c + 8 * g4; }
  static constexpr int RS = D + 1;                  // padded LDS row stride against bank conflicts
  static constexpr int ND = D / 16;                 // PV output tiles of 16 dims
  static constexpr int VRS = D + 16;                // LDS row stride of a staged V tile (elements): the
                                                    // 16 rows x 32 bytes of a transposing read cover every bank
  static_assert(D % 128 == 0, "MFMA family needs head_dim 128 or 256");

  struct Smem {
    float m[NW][16], l[NW][16];
    union {                                         // attend uses vt, finish o (after a barrier)
      float o[NW][16 * RS];
      alignas(16) uint16_t vt[NW][16 * VRS];        // each wave's V tile in q's type, row-major
    };
    alignas(16) int prefix[kMaxSliceSeqs + 4];
    int wsum[NW];
  };

  struct State {
    float m;                 // reference max of head c16 (same in all four row groups; within 2^8 of the running max)
    float lsum;              // this lane's share of the running exp-sum of head c16
    f32x4_t O[ND];           // O[dt]: lane l holds O[head l%16][dim 16 dt + 4(l/16) + r], r = 0..3
    __device__ void init() {
      m = -__builtin_inff();
      lsum = 0.f;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) O[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };

  // One block's tiles in registers: K as the QK A operand (token c16, NK
  // 16-byte loads), V as row-major loads of 8 elements of tokens 4*g4 + tg.
  typedef typename std::conditional<KV8, uint2, uint4>::type VLoad;
  struct Tiles {
    uint4 k[NK];
    VLoad v[4][NH];
    bool ok;
  };

  // Every lane loads unconditionally, so the compiler can count the loads in
  // flight and wait only for the tile being consumed (a load under a per-lane
  // condition makes it wait for every load, the next tile's too).  kpool /
  // vpool point at kv head kvh's tile of block 0 (wave-uniform); klane / vlane
  // are the lane's byte offsets inside a tile.  A row at or past `valid` (the
  // last block's tail) is masked by consume; with 16-bit caches it reads the
  // block's last real row instead (the same cache lines, no extra memory
  // traffic), with 8-bit ones the resource ends after row valid - 1 so that it
  // reads zeros and no memory (measured 1 % faster there, 0.2 % slower with
  // 16-bit caches).  A table entry outside the pool, or a block loaded only to
  // keep the loads unconditional (!live), gets an empty resource and reads no
  // memory at all (see load_tile); consume skips the former and never sees
  // the latter.
  __device__ static void issue(const AttnParams& p, const char* kpool, const char* vpool, size_t block_stride,
                               uint32_t klane, uint32_t vlane, int blk, int valid, bool live, int c16, int g4,
                               Tiles& t) {
    t.ok = blk >= 0 && blk < p.num_blocks;
    const size_t boff = (size_t)(t.ok ? blk : 0) * block_stride;
    const int bytes = !(t.ok && live && valid > 0) ? 0 : KV8 ? valid * (int)ROW_BYTES : (int)TILE_BYTES;
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kpool + boff, bytes), vr = buffer_rsrc(vpool + boff, bytes);
    // 16-bit caches: row r is read (min(r, valid - 1) - r) rows from its place
    auto shift = [&](int r) -> uint32_t { return KV8 ? 0u : (uint32_t)(((r < valid ? r : valid - 1) - r) * ROW_BYTES); };
    const uint32_t kof = klane + shift(c16);
#pragma unroll
    for (int c = 0; c < NK; ++c) t.k[c] = load_tile<uint4, NT>(kr, kof + c * (KV8 ? 16 : 64));
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const uint32_t vof = vlane + (uint32_t)(tg * ROW_BYTES) + shift(g4 * 4 + tg);
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
        t.v[tg][hh] = load_tile<VLoad, NT>(vr, vof + hh * 128 * KT::bytes);
    }
  }

  // MASK: only the lanes' columns with col_on take part in this block (the
  // others keep their state: no score, no weight, no rescale).
  template <bool MASK = false>
  __device__ static void consume(const AttnParams& p, const uint4* qop, Tiles& t, int valid, int c16, int g4,
                                 uint16_t* vt, State& st, bool col_on = true) {
    if (!t.ok) return;                                  // wave-uniform
    f32x4_t S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if constexpr (KV8) {
        const uint4& k = t.k[c / 2];
        S = MfmaOp<T>::qk((c & 1) ? kv8x8_to_16<T, KT>(k.z, k.w) : kv8x8_to_16<T, KT>(k.x, k.y), qop[c], S);
      } else {
        S = MfmaOp<T>::qk(t.k[c], qop[c], S);
      }
    }
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = S[r] * p.qk_scale;
    if constexpr (MASK) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s[r] = col_on ? s[r] : -__builtin_inff();
    }
    if (valid < BS) {                                   // wave-uniform: the last, partial block
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool v = g4 * 4 + r < valid;
        s[r] = v ? s[r] : -__builtin_inff();
        if (!v) {
#pragma unroll
          for (int hh = 0; hh < NH; ++hh) t.v[r][hh] = VLoad{};
        }
      }
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));   // finite: every block has a real token
                                                                // (-inf in a masked column, which never grows)
    mx = max_over_rows(mx);
    // The reference max st.m moves only when a head's block max exceeds it by
    // more than kLazyRescale (log2 domain): the weights stay below 2^kLazyRescale,
    // and the accumulators are rescaled on few blocks (a wave-uniform branch)
    // instead of on every block.  The softmax does not depend on the reference.
    const bool grow = mx > st.m + kLazyRescale;         // always on the first block (st.m = -inf)
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? exp2_fast(st.m - mx) : 1.f;   // 0 on the first block
      const float mn = grow ? mx : st.m;
      st.lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) st.O[dt] *= alpha;
      st.m = mn;
    }
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = exp2_fast(s[r] - st.m);
    if constexpr (MASK) {                               // a masked column may have no reference yet (-inf - -inf)
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[r] = col_on ? pr[r] : 0.f;
    }
    st.lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    // PV on 16x16x16 MFMAs.  B = P^T: the contraction index of lane group g4 is
    // tokens 4 g4 .. +3, exactly the lane's four weights; P enters as a 16-bit
    // part and the 16-bit rounding of what it left out, so the product keeps
    // about 16 bits of each weight.  A = V^T: the wave stages its tile in LDS
    // (row-major, q's type) and reads it back transposed: lane 4m + q of group
    // g4 points at token 4 g4 + m, dims 16 dt + 4q .. +3, so output lane j
    // receives V[4 g4 + m][16 dt + j] for m = 0..3.
#pragma unroll
    for (int tg = 0; tg < 4; ++tg)
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        uint4 v16;
        if constexpr (KV8) v16 = kv8x8_to_16<T, KT>(t.v[tg][hh].x, t.v[tg][hh].y);
        else v16 = t.v[tg][hh];
        *reinterpret_cast<uint4*>(vt + (4 * g4 + tg) * VRS + 128 * hh + 8 * c16) = v16;
      }
    uint2 phi, plo;
    MfmaOp<T>::split(pr, phi, plo);
    const uint16_t* vr = vt + (4 * g4 + (c16 >> 2)) * VRS + 4 * (c16 & 3);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      const uint2 a = lds_read_tr16(vr + 16 * dt);
      st.O[dt] = MfmaOp<T>::pv(a, phi, st.O[dt]);
      st.O[dt] = MfmaOp<T>::pv(a, plo, st.O[dt]);
    }
  }

  // B operand of QK for column c16: Q[row][k_dim(c, g4) .. +8] of the query
  // row at element offset `qrow` (q is [rows][D]); zero for a padding column.
  __device__ static void load_q(const AttnParams& p, bool real, size_t qrow, int g4, uint4* qop) {
    const uint16_t* qr = reinterpret_cast<const uint16_t*>(p.q) + (real ? qrow : 0);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qop[c] = real ? *reinterpret_cast<const uint4*>(qr + k_dim(c, g4)) : make_uint4(0u, 0u, 0u, 0u);
  }

  // Blocks [j0, j1) of sequence `seq` for the query heads of kv head `kvh`.
  __device__ static void attend(const AttnParams& p, int seq, int kvh, int ctx, int j0, int j1, int w, int c16,
                                int g4, uint16_t* vt, State& st) {
    if (j0 + w >= j1) return;                           // wave-uniform: no block for this wave
    const int G = p.group;
    uint4 qop[NC];
    load_q(p, c16 < G, ((size_t)seq * p.num_heads + (size_t)kvh * G + c16) * D, g4, qop);
    walk<false>(p, p.block_tables + (size_t)seq * p.max_blocks_per_seq, kvh, ctx, j0, j1, w, c16, g4, vt, st, qop,
                true);
  }

  // Blocks [j0, j1) of the table `table` (a context of ctx tokens) under the
  // query operand qop; wave w takes blocks j0 + w, j0 + w + NW, ...  With PIPE
  // the next block's tiles are in flight while the current one is consumed.
  // Block ids come 64 at a time from one VGPR (lane t holds the t-th id)
  // through readlane.  MASK / col_on: see consume.
  template <bool MASK>
  __device__ static void walk(const AttnParams& p, const int32_t* table, int kvh, int ctx, int j0, int j1, int w,
                              int c16, int g4, uint16_t* vt, State& st, const uint4* qop, bool col_on) {
    const int first = j0 + w;
    const int n = first < j1 ? (j1 - first + NW - 1) / NW : 0;
    if (n == 0) return;                                 // wave-uniform
    const char* kpool = reinterpret_cast<const char*>(p.k_cache) + (size_t)kvh * TILE_BYTES;
    const char* vpool = reinterpret_cast<const char*>(p.v_cache) + (size_t)kvh * TILE_BYTES;
    const uint32_t klane = (uint32_t)(c16 * ROW_BYTES + (KV8 ? g4 * (D / 4) : g4 * 16));
    const uint32_t vlane = (uint32_t)((g4 * 4) * ROW_BYTES + c16 * 8 * KT::bytes);
    const size_t block_stride = TILE_BYTES * (size_t)p.num_kv_heads;
    const int lane = threadIdx.x & 63;
    auto load_ids = [&](int chunk) -> int {
      const int i = chunk * 64 + lane;
      return i < n ? table[first + i * NW] : -1;
    };
    int ids = load_ids(0);
    int ids_next = n > 64 ? load_ids(1) : -1;
    int chunk = 0;
    auto id_of = [&](int i) -> int {                    // called with i = 0, 1, 2, ... in order
      if ((i >> 6) != chunk) {
        chunk = i >> 6;
        ids = ids_next;
        ids_next = (chunk + 1) * 64 < n ? load_ids(chunk + 1) : -1;
      }
      return __builtin_amdgcn_readlane(ids, i & 63);
    };
    auto valid_of = [&](int i) -> int {                 // real tokens in the wave's i-th block
      const int r = ctx - (first + i * NW) * BS;
      return r < BS ? r : BS;
    };
    Tiles a;
    issue(p, kpool, vpool, block_stride, klane, vlane, id_of(0), valid_of(0), true, c16, g4, a);
    if constexpr (PIPE) {
      // Both tile sets are refilled on every pass, also past the wave's last
      // block (issued for block n - 1 again but reading no memory, never
      // consumed): loads under a branch would make the compiler wait for all
      // loads in flight before each consume instead of only the consumed tile's.
      Tiles b;
      for (int i = 0; i < n; i += 2) {
        const int i1 = i + 1 < n ? i + 1 : n - 1;
        const int i2 = i + 2 < n ? i + 2 : n - 1;
        issue(p, kpool, vpool, block_stride, klane, vlane, id_of(i1), valid_of(i1), i + 1 < n, c16, g4, b);
        consume<MASK>(p, qop, a, valid_of(i), c16, g4, vt, st, col_on);
        issue(p, kpool, vpool, block_stride, klane, vlane, id_of(i2), valid_of(i2), i + 2 < n, c16, g4, a);
        if (i + 1 < n) consume<MASK>(p, qop, b, valid_of(i + 1), c16, g4, vt, st, col_on);
      }
    } else {
      for (int i = 0; i < n; ++i) {
        if (i > 0) issue(p, kpool, vpool, block_stride, klane, vlane, id_of(i), valid_of(i), true, c16, g4, a);
        consume<MASK>(p, qop, a, valid_of(i), c16, g4, vt, st, col_on);
      }
    }
  }

  // Merge the waves' states of columns 0 .. ncols-1 through LDS and hand each
  // (column h, dim d) to store(h, d, M, L, o): M the merged max (log2 domain),
  // L the merged exp-sum, o the unnormalised output.  Called by every thread;
  // ends with a barrier.
  template <class Store>
  __device__ static void merge(State& st, Smem& sm, int ncols, int tid, int w, int c16, int g4, Store store) {
    float lsum = st.lsum;
    lsum = sum_over_rows(lsum);
    __syncthreads();                                    // every wave is done with its V tile (o shares it)
    if (c16 < ncols) {
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.o[w][c16 * RS + 16 * dt + 4 * g4 + r] = st.O[dt][r];
      if (g4 == 0) { sm.m[w][c16] = st.m; sm.l[w][c16] = lsum; }
    }
    __syncthreads();
    for (int idx = tid; idx < ncols * D; idx += NW * 64) {
      const int h = idx / D;
      const int d = idx - h * D;
      float M = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < NW; ++i) M = fmaxf(M, sm.m[i][h]);
      float o = 0.f, Lsum = 0.f;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const float wt = (sm.m[i][h] == -__builtin_inff()) ? 0.f : exp2_fast(sm.m[i][h] - M);
        Lsum += wt * sm.l[i][h];
        o += wt * sm.o[i][h * RS + d];
      }
      store(h, d, M, Lsum, o);
    }
    __syncthreads();
  }

  // Merge the waves (only the G real heads) and write the normalised outputs
  // (prow_base < 0) or the fp32 summary row prow_base + h * prow_stride of the
  // workspace for head h of the group.  Called by every thread; ends with a
  // barrier.
  __device__ static void finish(const AttnParams& p, State& st, Smem& sm, int seq, int kvh, int64_t prow_base,
                                int64_t prow_stride, int tid, int w, int c16, int g4) {
    const int G = p.group;
    merge(st, sm, G, tid, w, c16, g4, [&](int h, int d, float M, float Lsum, float o) {
      if (prow_base < 0) {
        const size_t sh = (size_t)seq * p.num_heads + (size_t)kvh * G + h;
        store_elem<T>(p.out, sh * D + d, Lsum > 0.f ? o * (p.v_scale / Lsum) : 0.f);
      } else {
        const int64_t prow = prow_base + h * prow_stride;
        p.ws_o[(size_t)prow * D + d] = o * p.v_scale;
        if (d == 0) { p.ws_m[prow] = M; p.ws_l[prow] = Lsum; }
      }
    });
  }
};

#ifndef PKV_MFMA_WAVES_PER_EU
#define PKV_MFMA_WAVES_PER_EU 4
#endif
#ifndef PKV_MFMA_WAVES_PER_EU_PIPE
#define PKV_MFMA_WAVES_PER_EU_PIPE 3
#endif
template <class T, class KT, int D, int NW, bool PIPE, bool NT, bool APPEND>
__device__ __forceinline__ void attn_mfma_body(AttnParams p) {
  using A = MfmaAttention<T, KT, D, NW, PIPE, NT>;
  __shared__ typename A::Smem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15;   // QK: token row of A / head column of B and of the result
  const int g4 = lane >> 4;    // 0..3
  const uint32_t L = p.head_run_units ? head_runs(blockIdx.x, p.head_run_units)
                                       : xcd_remap(blockIdx.x, p.total_wgs, p.xcd_chunk);
  typename A::State st;

  if (p.num_slices > 0) {
    const int kvh = (int)(L % (uint32_t)p.num_kv_heads);
    apply_head_scales(p, kvh);
    const int k = (int)(L / (uint32_t)p.num_kv_heads);
    const int S = p.num_seqs;
    block_prefix<NW * 64>(p.context_lens, S, p.ctx_cap, A::BS, sm.prefix, sm.wsum);
    if (blockIdx.x == 0)
      for (int i = tid; i <= S; i += NW * 64) p.ws_prefix[i] = sm.prefix[i];
    const int64_t total = sm.prefix[S];
    const int64_t a = slice_begin(k, total, p.num_slices), b = slice_begin(k + 1, total, p.num_slices);
    if (a >= b) return;
    int lo = 1, hi = S;
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
      const int which = start <= a ? 0 : 1;
      int ctx = p.context_lens[s];
      ctx = ctx < 0 ? 0 : (ctx > p.ctx_cap ? p.ctx_cap : ctx);
      if (APPEND && j1 == end - start)                      // this segment holds the sequence's last block
        append_new_row<T, KT, D, A::BS, NW * 64>(p, s, kvh, (j1 - 1 - j0) % NW);
      st.init();
      A::attend(p, s, kvh, ctx, j0, j1, w, c16, g4, sm.vt[w], st);
      const int64_t prow = complete ? -1 : ((int64_t)k * 2 + which) * p.num_heads + (int64_t)kvh * p.group;
      A::finish(p, st, sm, s, kvh, prow, 1, tid, w, c16, g4);
      pos = end;
      ++s;
      while (s < S && sm.prefix[s + 1] <= pos) ++s;
    }
    return;
  }

  int seq, kvh, part;
  if (p.compact_partitions) {
    // Fixed partitions: work id -> (kv head, position in the stream of
    // (sequence, partition) units of that head), sequence by sequence, where
    // sequence s owns max(1, its partitions) consecutive units (an empty
    // context keeps one, which writes its zero output).  Only units with work
    // exist; ids past the stream's end leave at once.
    const int S = p.num_seqs;
    kvh = (int)(L % (uint32_t)p.num_kv_heads);
    const int pos = (int)(L / (uint32_t)p.num_kv_heads);
    block_prefix<NW * 64>(p.context_lens, S, p.ctx_cap, p.partition_blocks * A::BS, sm.prefix, sm.wsum, true);
    if (pos >= sm.prefix[S]) return;                        // uniform: past the stream
    int lo = 1, hi = S;                                     // first i with prefix[i] > pos
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sm.prefix[mid] > pos) hi = mid; else lo = mid + 1;
    }
    seq = lo - 1;
    part = pos - sm.prefix[seq];
  } else {
    decode_work_id(L, p.num_seqs, p.num_kv_heads, seq, kvh, part);
    // Fixed partitions: the last partition index first.  Shorter contexts have
    // no partition at the high indices, so the workgroups that find nothing to
    // do are dispatched while the GPU fills, and the grid ends with low
    // partitions, which every context has.
    if (p.num_partitions > 1 && PKV_PARTITIONS_REVERSED) part = p.num_partitions - 1 - part;
  }
  apply_head_scales(p, kvh);
  if (p.longest_first) {                                    // one pass only
    if (p.seq_order) {
      const int o = p.seq_order[seq];
      seq = o < 0 ? 0 : (o >= p.num_seqs ? p.num_seqs - 1 : o);
    } else {
      seq = seq_of_rank<NW * 64>(p.context_lens, p.num_seqs, p.ctx_cap, A::BS, seq, sm.prefix, sm.wsum);
    }
  }
  int ctx = p.context_lens[seq];
  ctx = ctx < 0 ? 0 : (ctx > p.ctx_cap ? p.ctx_cap : ctx);
  const int nblk = (ctx + A::BS - 1) / A::BS;
  const int b_begin = part * p.partition_blocks;
  // a context that fits in one partition is finished here; the reduce skips it
  const bool direct = p.num_partitions == 1 || nblk <= p.partition_blocks;
  if (b_begin >= nblk && (part > 0 || !direct)) return;     // empty partition
  int b_end = b_begin + p.partition_blocks;
  b_end = b_end < nblk ? b_end : nblk;
  if (APPEND && nblk > 0 && b_end == nblk)                  // this workgroup reads the last block
    append_new_row<T, KT, D, A::BS, NW * 64>(p, seq, kvh, (nblk - 1 - b_begin) % NW);
  st.init();
  A::attend(p, seq, kvh, ctx, b_begin, b_end, w, c16, g4, sm.vt[w], st);
  // partition rows are [seq][head][partition]
  const int64_t prow = direct ? -1 : ((int64_t)seq * p.num_heads + (int64_t)kvh * p.group) * p.num_partitions + part;
  A::finish(p, st, sm, seq, kvh, prow, p.num_partitions, tid, w, c16, g4);
}

#define PKV_MFMA_WAVES(D, PIPE) ((D) == 128 ? ((PIPE) ? PKV_MFMA_WAVES_PER_EU_PIPE : PKV_MFMA_WAVES_PER_EU) : 1)
template <class T, class KT, int D, int NW, bool PIPE, bool NT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(PKV_MFMA_WAVES(D, PIPE))))
void attn_mfma_kernel(AttnParams p) {
  attn_mfma_body<T, KT, D, NW, PIPE, NT, false>(p);
}

template <class T, class KT, int D, int NW, bool PIPE, bool NT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(PKV_MFMA_WAVES(D, PIPE))))
void attn_mfma_append_kernel(AttnParams p) {
  attn_mfma_body<T, KT, D, NW, PIPE, NT, true>(p);
}

#ifndef PKV_MFMA_NW
#define PKV_MFMA_NW 4             // waves per workgroup: one pass and balanced slices
#endif
#ifndef PKV_MFMA_NW_PARTITIONS
#define PKV_MFMA_NW_PARTITIONS 2  // waves per workgroup: fixed partitions
#endif
#ifndef PKV_MFMA_PIPE
#define PKV_MFMA_PIPE 1
#endif
template <bool APPEND, class T, class KT, int D, int NW, bool NT>
static hipError_t launch_mfma_nt(const AttnParams& p, hipStream_t stream) {
  constexpr bool PIPE = PKV_MFMA_PIPE != 0;
  if constexpr (APPEND)
    hipLaunchKernelGGL((attn_mfma_append_kernel<T, KT, D, NW, PIPE, NT>), dim3(p.total_wgs), dim3(NW * 64), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<T, KT, D, NW, PIPE, NT>), dim3(p.total_wgs), dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <bool APPEND, class T, class KT, int D, int NW>
static hipError_t launch_mfma_nw(const AttnParams& p, hipStream_t stream) {
  return p.kv_cached ? launch_mfma_nt<APPEND, T, KT, D, NW, false>(p, stream)
                     : launch_mfma_nt<APPEND, T, KT, D, NW, true>(p, stream);
}

// Fixed partitions run with fewer waves per workgroup: a partition of a few
// dozen blocks split over 4 waves leaves each wave a short walk whose fixed
// costs (the head's prefix, the query fragments, the merge of the waves'
// summaries through LDS) weigh more; 2 waves per partition measured faster on
// 512-token partitions of long contexts, 4 faster for one pass and slices.
template <bool APPEND, class T, class KT, int D>
static hipError_t launch_mfma(const AttnParams& p, hipStream_t stream) {
  if (p.num_slices == 0 && p.num_partitions > 1)
    return launch_mfma_nw<APPEND, T, KT, D, PKV_MFMA_NW_PARTITIONS>(p, stream);
  return launch_mfma_nw<APPEND, T, KT, D, PKV_MFMA_NW>(p, stream);
}

template <bool APPEND, class T, class KT>
static hipError_t launch_mfma_d(const AttnParams& p, int d, hipStream_t stream) {
  if (d == 128) return launch_mfma<APPEND, T, KT, 128>(p, stream);
  if (d == 256) return launch_mfma<APPEND, T, KT, 256>(p, stream);
  return hipErrorInvalidValue;
}

// (q dtype, kv dtype, head_dim) -> instantiation; the cases mfma_supported accepts.
template <bool APPEND>
static hipError_t launch_mfma_family(const AttnParams& p, int q_dtype, int kv_dtype, int d, hipStream_t stream) {
  if (q_dtype == BF16::kId) {
    if (kv_dtype == BF16::kId) return launch_mfma_d<APPEND, BF16, BF16>(p, d, stream);
    if (kv_dtype == FP8::kId) return launch_mfma_d<APPEND, BF16, FP8>(p, d, stream);
    if (kv_dtype == BF8::kId) return launch_mfma_d<APPEND, BF16, BF8>(p, d, stream);
  } else if (q_dtype == F16::kId) {
    if (kv_dtype == F16::kId) return launch_mfma_d<APPEND, F16, F16>(p, d, stream);
    if (kv_dtype == FP8::kId) return launch_mfma_d<APPEND, F16, FP8>(p, d, stream);
    if (kv_dtype == BF8::kId) return launch_mfma_d<APPEND, F16, BF8>(p, d, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
