// prefill_mfma.hip -- chunked prefill attention over the paged cache on the
// CDNA4 matrix cores.  The prefill of a long prompt is split into chunks
// ("vLLM PagedAttention: uma revolução no throughput de inferência de LLMs",
// feature list: chunked prefill); each chunk's queries are the sequence's last
// n positions and attend causally to every token cached so far, the chunk's own
// K/V included (written to the pool by reshape_and_cache first).  Unlike decode
// this is a dense contraction: a 128-query tile reuses every K/V tile 128 times.
//
// One workgroup of 4 waves per (sequence, 128-query tile, query head); wave w
// owns query rows 32w .. 32w+31 of the tile as two 16-row groups.  Per step of
// 64 tokens (four 16-token blocks):
//   staging  the step's K and V rows go from the pool straight into LDS, one
//            step ahead, with global_load_lds_dwordx4: each instruction of a
//            wave fills 1 KiB of LDS (lane i's 16 bytes at 16 i), so a wave
//            chooses which 16-byte chunk of which token row each lane fetches
//            (through the block table).  Rows are D elements with no padding;
//            the chunk order inside a row is XOR-swizzled (K and V differently)
//            so the fragment reads below hit distinct LDS banks.  No register
//            staging and no LDS store instructions; each wave waits for its own
//            loads before the step's barrier.
//   QK       S^T[token][query] = sum_k K[token][k] Q[query][k]
//            v_mfma_f32_16x16x32 (f16/bf16), A = K rows from LDS (read once,
//            used by both row groups), B = Q^T held in registers; lane l gets
//            tokens 4(l/16)+r and 16+4(l/16)+r (r = 0..3) of query l%16.
//   softmax  causal / context mask (only on steps that straddle a boundary),
//            max over the step's 64 tokens (the lane's 16 values, then lanes
//            l^16 and l^32), exp2 in the log2 domain against a reference max
//            that moves only when a row's max grows by more than 2^8.
//   PV       O^T[dim][query] += sum_k V^T[dim][token_k] P^T[token_k][query]
//            v_mfma_f32_16x16x32 again: the contraction index k of lane group
//            l/16 is its 8 tokens above, so B = P^T is exactly the lane's own
//            8 softmax weights rounded to the input type.  A = V^T comes from
//            the row-major V tile through the transposing LDS read
//            ds_read_b64_tr_b16: within a 16-lane group, output lane j gets
//            element j%4 of the 4 values at lane 4m + j/4's address, for
//            m = 0..3; lane (c16, g4) points at token 4 g4 + c16/4, dims
//            d0 + 4 (c16%4) .. +3, so it receives V[4 g4 + m][d0 + c16].
// An 8-bit cache ("PagedAttention", Ultralytics glossary, section "Các kỹ thuật
// liên quan": FP8 keys and values) is staged the same way as bytes, into two
// stage buffers per tensor, and a convert pass turns each step's codes into the
// 16-bit tiles above (exact for E4M3 and E5M2); its scales go to the logits
// (K) and to the output (V).
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

template <class T> struct PrefillOp;
template <> struct PrefillOp<BF16> {
  __device__ __forceinline__ static f32x4_t mma(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  }
  __device__ __forceinline__ static uint32_t pack(float x, float y) {      // round to nearest even
    const bf162_t h = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, h);
  }
  __device__ __forceinline__ static uint4 ones() { return make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u); }
};
template <> struct PrefillOp<F16> {
  __device__ __forceinline__ static f32x4_t mma(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
  }
  __device__ __forceinline__ static uint32_t pack(float x, float y) {
    const half2_t h = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, h);
  }
  __device__ __forceinline__ static uint4 ones() { return make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u); }
};

constexpr float kRescale = 8.f;

#ifndef PKV_PREFILL_RW
#define PKV_PREFILL_RW 2      // 16-row query groups per wave
#endif
#ifndef PKV_PREFILL_NS
#define PKV_PREFILL_NS 2      // 32-token PV k-steps per pipeline step
#endif
#ifndef PKV_PREFILL_NW
#define PKV_PREFILL_NW 4      // waves per workgroup
#endif
#ifndef PKV_PREFILL_RING
#define PKV_PREFILL_RING 2    // stage buffers per tensor: loads run RING - 1 steps ahead
#endif
#ifndef PKV_PREFILL_WAVES_PER_EU
#define PKV_PREFILL_WAVES_PER_EU 2   // occupancy the register allocation must allow
#endif

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;


// Source of the 16-byte chunks of tokens that are not loaded (past the keys, or
// in a block outside the pool): zeros, so V rows that get weight 0 stay finite.
static __device__ __align__(16) const uint16_t kZeroChunk[8] = {0, 0, 0, 0, 0, 0, 0, 0};

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima): this wave's
// loads into LDS have landed
__device__ __forceinline__ void wait_lds_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// One global_load_lds_dwordx4: lane l's 16 bytes at src go to LDS bytes
// dst + 16 l .. +15 (dst wave-uniform).  The LDS it fills is read only after
// wait_lds_loads() and a barrier, and is filled only after the barrier that
// ends the step that last read it.
__device__ __forceinline__ void load_lds16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)dst, 16, 0, 0);
}

// The same through a buffer resource (buffer_rsrc): the 16 bytes at byte `off`
// (per lane) of the resource's range go to LDS bytes dst + 16 l .. +15.  The
// address is the resource's base plus the 32-bit lane offset, so no 64-bit
// address is formed per lane.  Every offset passed is inside the range.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t off, void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 16, off, 0, 0, 0);
}

// ds_read_b64_tr_b16 on an LDS address (8-byte aligned)
__device__ __forceinline__ uint2 read_tr16(const uint16_t* lds) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds));
  return __builtin_bit_cast(uint2, v);
}

template <class T, int D, int RW>
struct Prefill {
  static constexpr int BS = 16;                 // tokens per block
  static constexpr int NS = PKV_PREFILL_NS;     // PV k-steps (32 tokens each) per step
  static constexpr int STEP = 32 * NS;          // tokens per step
  static constexpr int KT = STEP / 16;          // blocks per step
  static constexpr int NW = PKV_PREFILL_NW;
  static constexpr int BM = NW * 16 * RW;       // query rows per workgroup
  static constexpr int NC = D / 32;             // QK k-steps of 32 dims
  static constexpr int ND = D / 16;             // PV output tiles of 16 dims
  static constexpr int CPR = D / 8;             // 16-byte chunks per token row
  static constexpr int RPI = 1024 / (2 * D);    // token rows per load instruction (64 lanes x 16 bytes)
  static constexpr int NQ = STEP / RPI;         // load instructions per tensor per step
  static constexpr int QPW = NQ / NW;           // ... per wave
  static constexpr int RPB = 256 / (2 * D);     // token rows per 256 bytes (one pass over the 64 LDS banks)
  static_assert(NQ % NW == 0 && RPI <= BS && BS % RPI == 0, "staging shape");
  static constexpr int TILE = STEP * D;         // elements of one K or V buffer

  // Chunk swizzles: logical chunk c of row r sits at chunk c ^ f(r) of the row.
  // K fragment reads take rows r0..r0+15 at one logical chunk: f_K spreads them
  // over all bank groups.  The transposing V reads take 8 consecutive rows x 2
  // adjacent chunks per 32 lanes: f_V is even, so a chunk pair stays a pair,
  // and distinct per row.
  __device__ __forceinline__ static int swz_k(int r) { return (r / RPB) % CPR; }
  __device__ __forceinline__ static int swz_v(int r) { return 2 * ((r / RPB) % (CPR / 2)); }
};

template <class T, class CT, int D, int RW>
__global__ __launch_bounds__(PKV_PREFILL_NW * 64) __attribute__((amdgpu_waves_per_eu(PKV_PREFILL_WAVES_PER_EU)))
void prefill_mfma_kernel(PrefillParams p) {
  using P = Prefill<T, D, RW>;
  using Op = PrefillOp<T>;
  constexpr int STEP = P::STEP, BS = P::BS, NC = P::NC, ND = P::ND, CPR = P::CPR, KT = P::KT,
                NS = P::NS;
  // CT, the cache type: T itself, or an 8-bit format (E4M3 / E5M2) whose
  // codes are staged as bytes and converted, exactly, to T in LDS
  constexpr bool kQuant = CT::bytes == 1;
  static_assert(kQuant || CT::kId == T::kId, "a 16-bit cache has q's type");
  struct StepIds { int b[KT]; };                            // block ids of one step (-1 past the keys)
  // RING stage buffers per tensor as separate objects: the compiler then sees
  // that loads into one never alias reads of another and adds no wait between them
  constexpr int R = PKV_PREFILL_RING;
  static_assert(R >= 2 && R <= 4, "2 to 4 stage buffers");
  __shared__ __align__(16) uint16_t sK0[P::TILE], sV0[P::TILE];
  __shared__ __align__(16) uint16_t sK1[kQuant ? 1 : P::TILE], sV1[kQuant ? 1 : P::TILE];
  __shared__ __align__(16) uint16_t sK2[R > 2 && !kQuant ? P::TILE : 1], sV2[R > 2 && !kQuant ? P::TILE : 1];
  __shared__ __align__(16) uint16_t sK3[R > 3 && !kQuant ? P::TILE : 1], sV3[R > 3 && !kQuant ? P::TILE : 1];
  // 8-bit cache: two stage buffers of codes per tensor, converted into sK0 / sV0
  constexpr int TILE8 = kQuant ? STEP * D : 16;
  __shared__ __align__(16) uint8_t qK0[TILE8], qK1[TILE8], qV0[TILE8], qV1[TILE8];
  auto kbuf = [&](auto b) -> uint16_t* {
    constexpr int k = decltype(b)::value;
    if constexpr (k == 0) return sK0; else if constexpr (k == 1) return sK1; else if constexpr (k == 2) return sK2; else return sK3;
  };
  auto vbuf = [&](auto b) -> uint16_t* {
    constexpr int k = decltype(b)::value;
    if constexpr (k == 0) return sV0; else if constexpr (k == 1) return sV1; else if constexpr (k == 2) return sV2; else return sV3;
  };
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15;
  const int g4 = lane >> 4;

  // work id: query tiles fastest (last tile first), then head, then sequence;
  // sequences in decreasing context length (longest first) when asked
  const uint32_t L = xcd_remap(blockIdx.x, p.total_wgs, p.xcd_chunk);
  const int tile = p.q_tiles - 1 - (int)(L % (uint32_t)p.q_tiles);
  const uint32_t rest = L / (uint32_t)p.q_tiles;
  const int h = (int)(rest % (uint32_t)p.num_heads);
  int seq = (int)(rest / (uint32_t)p.num_heads);
  if (p.longest_first)   // LDS scratch borrowed from the K tiles, which are first written after its last barrier
    seq = seq_of_rank<P::NW * 64>(p.context_lens, p.num_seqs, p.ctx_cap, BS, seq, reinterpret_cast<int*>(sK0),
                                  reinterpret_cast<int*>(sK1));
  const int kvh = h / p.group;
  // logit scale, and with an 8-bit cache the K scale folded into it (the
  // converted codes are the cache's values divided by the scale) and the V
  // scale applied to the output
  float qk_scale = p.qk_scale, out_scale = 1.f;
  if constexpr (kQuant) {
    qk_scale *= p.k_scales ? p.k_scales[kvh] : p.k_scale;
    out_scale = p.v_scales ? p.v_scales[kvh] : p.v_scale;
  }

  // rows [q0, q1) of q / out; offsets are clamped to the num_tokens rows that exist
  int q0 = p.query_start_loc[seq];
  int q1 = p.query_start_loc[seq + 1];
  q0 = q0 < 0 ? 0 : (q0 > p.num_tokens ? p.num_tokens : q0);
  q1 = q1 < q0 ? q0 : (q1 > p.num_tokens ? p.num_tokens : q1);
  const int n_all = q1 - q0;                                // the chunk's query tokens
  const int n = n_all < p.max_query_len ? n_all : p.max_query_len;   // rows this launch covers
  const int row0 = tile * P::BM;
  if (row0 >= n) return;                                    // workgroup-uniform
  int ctx = p.context_lens[seq];
  ctx = ctx < 0 ? 0 : (ctx > p.ctx_cap ? p.ctx_cap : ctx);
  const int base = ctx - n_all;                             // position of query row 0 (< 0: no position)
  const int rows_here = (n - row0) < P::BM ? (n - row0) : P::BM;
  int nkeys = base + row0 + rows_here;                      // keys 0 .. nkeys-1 serve this tile
  nkeys = __builtin_amdgcn_readfirstlane(nkeys > ctx ? ctx : (nkeys < 0 ? 0 : nkeys));   // uniform: scalar loop bounds and table reads
  const int nsteps = (nkeys + STEP - 1) / STEP;
  const int wrow0 = row0 + 16 * RW * w;                     // the wave's first row
  const int wave_first_pos = base + wrow0;
  const int wave_last_pos = wave_first_pos + 16 * RW - 1;   // causal limit of the wave's rows

  // B operand of QK: Q^T, lane l holds query row wrow0 + 16 g + c16, dims 32c + 8 g4 .. +8.
  // With a negative scale Q enters negated (sign bits flipped, exact), so the
  // logit scale qs applied to the products is never negative.
  const uint32_t qsign = qk_scale < 0.f ? 0x80008000u : 0u;
  const float qs = fabsf(qk_scale);
  uint4 qf[RW][NC];
  int qpos[RW];
  bool qreal[RW];
#pragma unroll
  for (int g = 0; g < RW; ++g) {
    const int qrow = wrow0 + 16 * g + c16;
    qreal[g] = qrow < n;
    qpos[g] = base + qrow;
    const uint16_t* qp =
        reinterpret_cast<const uint16_t*>(p.q) + ((size_t)(q0 + (qreal[g] ? qrow : 0)) * p.num_heads + h) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint4 v = qreal[g] ? *reinterpret_cast<const uint4*>(qp + c * 32 + g4 * 8) : make_uint4(0u, 0u, 0u, 0u);
      qf[g][c] = make_uint4(v.x ^ qsign, v.y ^ qsign, v.z ^ qsign, v.w ^ qsign);
    }
  }

  float m[RW];
  f32x4_t lsum[RW];   // row sums of the rounded weights, from the PV MFMA with an all-ones A (every element equal)
  f32x4_t O[RW][ND];
#pragma unroll
  for (int g = 0; g < RW; ++g) {
    m[g] = -__builtin_inff();
    lsum[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) O[g][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // The table is read through the constant address space: it is not written
  // during the launch, so its (uniform) entries come with scalar loads, whose
  // waits do not wait for the K/V loads in flight.
  typedef const __attribute__((address_space(4))) int32_t const_i32_t;
  const_i32_t* table = (const_i32_t*)(p.block_tables + (size_t)seq * p.max_blocks_per_seq);
  const size_t block_stride = (size_t)p.num_kv_heads * BS * D;             // elements
  const uint16_t* kpool = reinterpret_cast<const uint16_t*>(p.k_cache) + (size_t)kvh * BS * D;
  const uint16_t* vpool = reinterpret_cast<const uint16_t*>(p.v_cache) + (size_t)kvh * BS * D;

  const int nkblk = (nkeys + BS - 1) / BS;
  // block ids of step st; uniform, so scalar loads
  // (every read is in the row's first nkblk entries; all KT issue before any is used)
  auto ids_of = [&](int st) -> StepIds {
    StepIds r;
    const int last = nkblk > 0 ? nkblk - 1 : 0;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int j = KT * st + kt;
      r.b[kt] = __builtin_amdgcn_readfirstlane(table[j < last ? j : last]);
    }
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) r.b[kt] = KT * st + kt < nkblk ? r.b[kt] : -1;
    return r;
  };
  // Load step i's K and V rows into LDS buffers kb, vb: instruction q of the
  // step (wave-uniform) fills rows q*RPI .. q*RPI+RPI-1; lane l fetches the
  // logical chunk that the swizzle puts at position l % CPR of row l / CPR.
  // A wave's QPW instructions cover QPW*RPI consecutive rows of one block of
  // the step (block WR*w/BS, from row WR*w % BS, WR = QPW*RPI), and the
  // swizzles repeat within a block, so a lane's offset inside the block is the
  // same on every step.  When every one of those rows is a key (all steps but
  // the last) and the block's table entry lies in the pool, the loads take the
  // block's base plus that offset; otherwise each lane checks its row and
  // reads a zero chunk past the keys.
  constexpr int WR = P::QPW * P::RPI;                       // rows per wave and step
  static_assert(BS % WR == 0 && KT * BS == P::NW * WR, "each wave loads part of one block of each step");
  static_assert(BS % (P::RPB * CPR) == 0, "the swizzles repeat within a block");
  const int dma_row = lane / CPR, dma_pos = lane % CPR;
  const int wkt = WR * w / BS, wrb = WR * w % BS;           // the wave's block of the step and first row in it
  auto load_step = [&](int i, StepIds ids, uint16_t* kb, uint16_t* vb) {
    int blk = ids.b[0];
#pragma unroll
    for (int kt = 1; kt < KT; ++kt) blk = wkt == kt ? ids.b[kt] : blk;   // the wave's block (uniform)
    const bool in_pool = blk >= 0 && blk < p.num_blocks;
    const size_t boff = (size_t)(in_pool ? blk : 0) * block_stride;
    const uint16_t* kblk = kpool + boff;
    const uint16_t* vblk = vpool + boff;
    if (in_pool && i * STEP + wkt * BS + wrb + WR <= nkeys) {   // uniform
      const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kblk, BS * D * 2), vr = buffer_rsrc(vblk, BS * D * 2);
#pragma unroll
      for (int j = 0; j < P::QPW; ++j) {                   // the block's tile + a fixed 32-bit lane offset
        const int rb = wrb + j * P::RPI + dma_row;          // row inside the block
        load_lds16(kr, (uint32_t)(rb * D + (dma_pos ^ P::swz_k(rb)) * 8) * 2u, kb + (w * P::QPW + j) * 512);
        load_lds16(vr, (uint32_t)(rb * D + (dma_pos ^ P::swz_v(rb)) * 8) * 2u, vb + (w * P::QPW + j) * 512);
      }
    } else {
#pragma unroll
      for (int j = 0; j < P::QPW; ++j) {
        const int rb = wrb + j * P::RPI + dma_row;
        const bool ok = in_pool && i * STEP + wkt * BS + rb < nkeys;
        load_lds16(ok ? kblk + rb * D + (dma_pos ^ P::swz_k(rb)) * 8 : kZeroChunk, kb + (w * P::QPW + j) * 512);
        load_lds16(ok ? vblk + rb * D + (dma_pos ^ P::swz_v(rb)) * 8 : kZeroChunk, vb + (w * P::QPW + j) * 512);
      }
    }
  };
  // 8-bit cache: a step's codes go into a stage buffer as rows of D bytes, in
  // order (row r of the step at byte r D).  One load instruction fills 1 KiB =
  // RPI8 rows, so wave w loads block w of the step (QPW8 instructions per
  // tensor), lane l the 16-byte chunk l % CPR8 of row l / CPR8 of its rows;
  // the same fast and checked paths as the 16-bit staging.
  constexpr int CPR8 = D / 16;                              // 16-byte chunks per row of codes
  constexpr int RPI8 = 64 / CPR8;                           // rows per load instruction
  constexpr int QPW8 = BS / RPI8;                           // load instructions per wave and tensor
  static_assert(!kQuant || (KT == P::NW && BS % RPI8 == 0), "8-bit staging: one block per wave and step");
  const int r8 = lane / CPR8, c8 = lane % CPR8;
  auto load_step8 = [&](int i, StepIds ids, uint8_t* kb, uint8_t* vb) {
    int blk = ids.b[0];
#pragma unroll
    for (int kt = 1; kt < KT; ++kt) blk = w == kt ? ids.b[kt] : blk;   // the wave's block (uniform)
    const bool in_pool = blk >= 0 && blk < p.num_blocks;
    const size_t boff = (size_t)(in_pool ? blk : 0) * block_stride + (size_t)kvh * BS * D;   // bytes
    const uint8_t* kblk = reinterpret_cast<const uint8_t*>(p.k_cache) + boff;
    const uint8_t* vblk = reinterpret_cast<const uint8_t*>(p.v_cache) + boff;
    if (in_pool && i * STEP + w * BS + BS <= nkeys) {       // uniform: the whole block is keys
      const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kblk, BS * D), vr = buffer_rsrc(vblk, BS * D);
#pragma unroll
      for (int j = 0; j < QPW8; ++j) {
        const uint32_t off = (uint32_t)((j * RPI8 + r8) * D + c8 * 16);
        load_lds16(kr, off, kb + (w * QPW8 + j) * 1024);
        load_lds16(vr, off, vb + (w * QPW8 + j) * 1024);
      }
    } else {
#pragma unroll
      for (int j = 0; j < QPW8; ++j) {
        const int rb = j * RPI8 + r8;                       // row inside the block
        const bool ok = in_pool && i * STEP + w * BS + rb < nkeys;
        load_lds16(ok ? kblk + rb * D + c8 * 16 : (const uint8_t*)kZeroChunk, kb + (w * QPW8 + j) * 1024);
        load_lds16(ok ? vblk + rb * D + c8 * 16 : (const uint8_t*)kZeroChunk, vb + (w * QPW8 + j) * 1024);
      }
    }
  };
  // Codes of one step -> the 16-bit tiles sK0 / sV0 in the layout the
  // fragment reads expect: the 16 codes of chunk c of row r are dims 16 c ..
  // 16 c + 15, logical 16-bit chunks 2c and 2c + 1, stored at their swizzled
  // positions.  Both formats convert exactly to f16 and bf16.
  auto convert8 = [&](const uint8_t* kq, const uint8_t* vq) __attribute__((always_inline)) {
    constexpr int CH = STEP * CPR8;                         // 16-byte chunks per tensor and step
    static_assert(CH % (P::NW * 64) == 0, "whole passes");
    if constexpr (kQuant) {
#pragma unroll
    for (int q = tid; q < CH; q += P::NW * 64) {
      const int r = q / CPR8, c = q % CPR8;
      const uint4 kx = *reinterpret_cast<const uint4*>(kq + q * 16);
      const uint4 vx = *reinterpret_cast<const uint4*>(vq + q * 16);
      const int sk = P::swz_k(r), sv = P::swz_v(r);
      *reinterpret_cast<uint4*>(sK0 + r * D + ((2 * c) ^ sk) * 8) = kv8x8_to_16<T, CT>(kx.x, kx.y);
      *reinterpret_cast<uint4*>(sK0 + r * D + ((2 * c + 1) ^ sk) * 8) = kv8x8_to_16<T, CT>(kx.z, kx.w);
      *reinterpret_cast<uint4*>(sV0 + r * D + ((2 * c) ^ sv) * 8) = kv8x8_to_16<T, CT>(vx.x, vx.y);
      *reinterpret_cast<uint4*>(sV0 + r * D + ((2 * c + 1) ^ sv) * 8) = kv8x8_to_16<T, CT>(vx.z, vx.w);
    }
    }
  };
  // Per-lane fragment addresses (elements) inside a buffer; the swizzles do not
  // change under the added multiples of 16 rows.
  // K: row c16 (+16 kt), logical chunk 4c + g4 -> chunk 4 (c ^ sk/4) + (g4 ^ sk%4)
  //    with sk = swz_k(c16).
  // V (transposing read): row vr = 4 g4 + c16/4 (+32 ns, +16 for the second
  //    half), dims 16 dt + 4 (c16 % 4) .. +3 = logical chunk 2 dt + (c16 % 4)/2,
  //    half c16 % 2; swz_v is even, so the chunk is 2 (dt ^ swz_v(vr)/2) + (c16 % 4)/2.
  const int kbase = c16 * D + (g4 ^ (P::swz_k(c16) & 3)) * 8, ksw = P::swz_k(c16) & ~3;
  const int vr = 4 * g4 + (c16 >> 2);
  const int vbase = vr * D + 8 * ((c16 & 3) >> 1) + 4 * (c16 & 1), vsw = P::swz_v(vr) / 2;
  // The lane's fragment offsets, once: every read of a step is then one of
  // these plus a compile-time offset (buffer, block, k-step), which the LDS
  // instruction takes as its immediate.
  int koff[NC], voff[ND];
#pragma unroll
  for (int c = 0; c < NC; ++c) koff[c] = kbase + ((4 * c) ^ ksw) * 8;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) voff[dt] = vbase + (dt ^ vsw) * 16;

  // One step of the wave's rows.  `masked` (a compile-time tag) selects the
  // variant with the per-element causal / context / skipped-block mask; steps
  // whose every key is visible to every row of the wave run the other one, so
  // interior steps carry no mask arithmetic at all.
  auto step_body = [&](int i, const uint16_t* kb, const uint16_t* vb, StepIds ids, auto masked) __attribute__((always_inline)) {
    constexpr bool interior = !decltype(masked)::value;
    const int k0 = i * STEP;
    {
      bool blk_ok[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) blk_ok[kt] = ids.b[kt] >= 0 && ids.b[kt] < p.num_blocks;
      f32x4_t S[RW][KT];
#pragma unroll
      for (int g = 0; g < RW; ++g)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) S[g][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const uint4 kf = *reinterpret_cast<const uint4*>(kb + kt * 16 * D + koff[c]);
#pragma unroll
          for (int g = 0; g < RW; ++g) S[g][kt] = Op::mma(kf, qf[g][c], S[g][kt]);
        }
      uint4 pk[RW][NS];
#pragma unroll
      for (int g = 0; g < RW; ++g) {
        // logits in the log2 domain are qs * S; on interior steps the scale is
        // folded into the exp2 argument (max commutes with qs >= 0)
        float s[KT][4];
        float mx = -__builtin_inff();
        if constexpr (interior) {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              s[kt][r] = S[g][kt][r];
              mx = fmaxf(mx, s[kt][r]);
            }
          mx *= qs;
        } else {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int kpos = k0 + kt * BS + g4 * 4 + r;
              const bool vis = blk_ok[kt] && kpos < nkeys && kpos <= qpos[g] && qreal[g];
              s[kt][r] = vis ? S[g][kt][r] * qs : -__builtin_inff();
              mx = fmaxf(mx, s[kt][r]);
            }
        }
        mx = max_over_rows(mx);
        // The reference max only moves when a row's max grows by more than
        // kRescale (log2 domain): softmax does not depend on the reference, the
        // weights stay <= 2^kRescale, and the accumulators are rescaled on few
        // steps (a wave-uniform branch) instead of every step.
        const bool grow = mx > m[g] + kRescale;
        if (__builtin_amdgcn_ballot_w64(grow)) {
          const float mn = grow ? mx : m[g];
          const float alpha = m[g] == -__builtin_inff() ? 0.f : exp2_fast(m[g] - mn);
          lsum[g] *= alpha;
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) O[g][dt] *= alpha;
          m[g] = mn;
        }
        const float mref = m[g] == -__builtin_inff() ? 0.f : m[g];   // nothing visible yet: weights are 0
        float pr[KT][4];
        if constexpr (interior) {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              pr[kt][r] = exp2_fast(fmaf(s[kt][r], qs, -mref));
            }
        } else {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              pr[kt][r] = exp2_fast(s[kt][r] - mref);
            }
        }
#pragma unroll
        for (int ns = 0; ns < NS; ++ns)
          pk[g][ns] = make_uint4(Op::pack(pr[2 * ns][0], pr[2 * ns][1]), Op::pack(pr[2 * ns][2], pr[2 * ns][3]),
                                 Op::pack(pr[2 * ns + 1][0], pr[2 * ns + 1][1]),
                                 Op::pack(pr[2 * ns + 1][2], pr[2 * ns + 1][3]));
      }
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
          const uint16_t* va = vb + 32 * ns * D + voff[dt];
          const uint2 lo = read_tr16(va);                   // tokens 32 ns + 4 g4 + m
          const uint2 hi = read_tr16(va + 16 * D);          // tokens 32 ns + 16 + 4 g4 + m
          const uint4 vf = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
          for (int g = 0; g < RW; ++g) O[g][dt] = Op::mma(vf, pk[g][ns], O[g][dt]);
        }
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
#pragma unroll
        for (int g = 0; g < RW; ++g) lsum[g] = Op::mma(Op::ones(), pk[g][ns], lsum[g]);
    }
  };
  // Steps [0, n_open) are open to every row of the workgroup: every key is
  // before the first row's position and inside the context.  With a table
  // whose entries all lie in the pool they run without the mask (padding rows
  // past the chunk are never written, so they need none either).
  bool table_ok = true;
  for (int b = tid; b < nkblk; b += P::NW * 64) table_ok = table_ok && table[b] >= 0 && table[b] < p.num_blocks;
  table_ok = __syncthreads_and(table_ok);
  int n_open = (base + row0 + 1 < nkeys ? base + row0 + 1 : nkeys) / STEP;
  n_open = __builtin_amdgcn_readfirstlane(table_ok && n_open > 0 ? n_open : 0);   // uniform (a scalar loop bound)
  auto compute_open = [&](int i, const uint16_t* kb, const uint16_t* vb, StepIds ids) __attribute__((always_inline)) {
    step_body(i, kb, vb, ids, std::false_type{});
  };
  auto compute = [&](int i, const uint16_t* kb, const uint16_t* vb, StepIds ids) __attribute__((always_inline)) {
    if (i * STEP > wave_last_pos) return;                   // wave-uniform: no key of the step is visible
    step_body(i, kb, vb, ids, std::true_type{});
  };

  if constexpr (!kQuant) {
    // Pipeline: a ring of R buffer pairs; step j's rows live in pair j % R and
    // are loaded R - 1 steps ahead, into the pair the previous step finished
    // with (its readers passed the barrier that ended that step).  At the end of
    // step i each wave waits until its loads of step i + 1 have landed (the
    // loads of later steps may stay in flight: vmcnt counts them, the loads of
    // one step are LPS instructions per wave), then meets the other waves at the
    // barrier.  The loops run R steps per pass from a multiple of R, so every
    // access names its buffers statically (open steps past the last multiple of
    // R run with the mask: same result).  Block ids come R steps ahead.
    constexpr int LPS = 2 * P::QPW;                           // load instructions per wave and step
    auto wait_step_after = [&](int i) __attribute__((always_inline)) {   // step i + 1's loads have landed
      const int later = (i + R - 1 < nsteps ? i + R - 1 : nsteps - 1) - (i + 1);   // later steps already issued
      if constexpr (R >= 4) { if (later >= 2) { __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * LPS)); return; } }
      if constexpr (R >= 3) { if (later >= 1) { __builtin_amdgcn_s_waitcnt(0x0F70 | LPS); return; } }
      wait_lds_loads();
    };
    static_assert((R - 2) * LPS <= 15, "vmcnt immediate");
    StepIds ids[R];
  #pragma unroll
    for (int k = 0; k < R; ++k) ids[k] = ids_of(k);
    // steps 0 .. R-2 into pairs 0 .. R-2
    if (0 < nsteps) load_step(0, ids[0], sK0, sV0);
    if constexpr (R > 2) { if (1 < nsteps) load_step(1, ids[1], sK1, sV1); }
    if constexpr (R > 3) { if (2 < nsteps) load_step(2, ids[2], sK2, sV2); }
    wait_step_after(-1);
    __syncthreads();
    auto one = [&](int i, auto open, auto cur) __attribute__((always_inline)) {
      constexpr int c = decltype(cur)::value, n = (c + R - 1) % R;
      const StepIds idn = ids_of(i + R);
      if (i + R - 1 < nsteps)
        load_step(i + R - 1, ids[R - 1], kbuf(std::integral_constant<int, n>{}), vbuf(std::integral_constant<int, n>{}));
      uint16_t* kc = kbuf(std::integral_constant<int, c>{});
      uint16_t* vc = vbuf(std::integral_constant<int, c>{});
      if constexpr (decltype(open)::value) compute_open(i, kc, vc, ids[0]); else compute(i, kc, vc, ids[0]);
      wait_step_after(i);
      __syncthreads();
  #pragma unroll
      for (int k = 0; k + 1 < R; ++k) ids[k] = ids[k + 1];
      ids[R - 1] = idn;
    };
    n_open -= n_open % R;
    auto steps = [&](int i, int end, auto open) __attribute__((always_inline)) {   // steps [i, end) from a multiple of R
      for (; i < end; i += R) {
        one(i, open, std::integral_constant<int, 0>{});
        if (i + 1 < end) one(i + 1, open, std::integral_constant<int, 1>{});
        if constexpr (R > 2) { if (i + 2 < end) one(i + 2, open, std::integral_constant<int, 2>{}); }
        if constexpr (R > 3) { if (i + 3 < end) one(i + 3, open, std::integral_constant<int, 3>{}); }
      }
    };
    steps(0, n_open, std::true_type{});
    steps(n_open, nsteps, std::false_type{});
  } else {
    // 8-bit cache, per step i (stage buffer i % 2 holds its codes, landed):
    // issue the codes of step i + 1 into the other stage buffer (its codes
    // were converted before the last barrier but one), convert step i into
    // sK0 / sV0 (their readers passed the barrier that ended step i - 1),
    // barrier, QK / softmax / PV, wait for this wave's loads of step i + 1,
    // barrier.  Steps run in pairs from an even index, so each stage buffer is
    // named statically.
    StepIds idc = ids_of(0), idn = ids_of(1);
    if (0 < nsteps) load_step8(0, idc, qK0, qV0);
    wait_lds_loads();
    __syncthreads();
    auto one8 = [&](int i, auto open, auto cur) __attribute__((always_inline)) {
      constexpr int c = decltype(cur)::value;
      const StepIds idnn = ids_of(i + 2);
      if (i + 1 < nsteps) load_step8(i + 1, idn, c ? qK0 : qK1, c ? qV0 : qV1);
      convert8(c ? qK1 : qK0, c ? qV1 : qV0);
      __syncthreads();
      if constexpr (decltype(open)::value) compute_open(i, sK0, sV0, idc); else compute(i, sK0, sV0, idc);
      wait_lds_loads();
      __syncthreads();
      idc = idn;
      idn = idnn;
    };
    const int open_end = n_open - n_open % 2;
    auto steps8 = [&](int i, int end, auto open) __attribute__((always_inline)) {   // steps [i, end) from an even index
      for (; i < end; i += 2) {
        one8(i, open, std::integral_constant<int, 0>{});
        if (i + 1 < end) one8(i + 1, open, std::integral_constant<int, 1>{});
      }
    };
    steps8(0, open_end, std::true_type{});
    steps8(open_end, nsteps, std::false_type{});
  }

  // normalise and write: lane l holds out[row wrow0 + 16 g + c16][dims 16 dt + 4 g4 + r]
#pragma unroll
  for (int g = 0; g < RW; ++g) {
    const float ls = lsum[g][0];
    if (qreal[g]) {
      float inv = ls > 0.f ? 1.f / ls : 0.f;
      if constexpr (kQuant) inv = ls > 0.f ? out_scale / ls : 0.f;
      const size_t orow = ((size_t)(q0 + wrow0 + 16 * g + c16) * p.num_heads + h) * D;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        const uint2 v = make_uint2(Op::pack(O[g][dt][0] * inv, O[g][dt][1] * inv),
                                   Op::pack(O[g][dt][2] * inv, O[g][dt][3] * inv));
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + orow + dt * 16 + g4 * 4) = v;
      }
    }
  }
}


bool prefill_supported(int q_dtype, int kv_dtype, int head_dim, int block_size) {
  return (q_dtype == F16::kId || q_dtype == BF16::kId) &&
         (kv_dtype == q_dtype || kv_dtype == FP8::kId || kv_dtype == BF8::kId) && (head_dim == 64 || head_dim == 128) &&
         block_size == 16;
}

int prefill_tile_rows() { return Prefill<F16, 128, PKV_PREFILL_RW>::BM; }

template <class T, class CT, int D>
static hipError_t launch_prefill_t(const PrefillParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_mfma_kernel<T, CT, D, PKV_PREFILL_RW>), dim3(p.total_wgs), dim3(PKV_PREFILL_NW * 64), 0,
                     stream, p);
  return hipGetLastError();
}

template <class T, class CT>
static hipError_t launch_prefill_d(const PrefillParams& p, int head_dim, hipStream_t stream) {
  return head_dim == 64 ? launch_prefill_t<T, CT, 64>(p, stream) : launch_prefill_t<T, CT, 128>(p, stream);
}

template <class T>
static hipError_t launch_prefill_kv(const PrefillParams& p, int kv_dtype, int head_dim, hipStream_t stream) {
  if (kv_dtype == T::kId) return launch_prefill_d<T, T>(p, head_dim, stream);
  if (kv_dtype == FP8::kId) return launch_prefill_d<T, FP8>(p, head_dim, stream);
  if (kv_dtype == BF8::kId) return launch_prefill_d<T, BF8>(p, head_dim, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillParams& p, int dtype, int kv_dtype, int head_dim, hipStream_t stream) {
  if (dtype == F16::kId) return launch_prefill_kv<F16>(p, kv_dtype, head_dim, stream);
  if (dtype == BF16::kId) return launch_prefill_kv<BF16>(p, kv_dtype, head_dim, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
