// prefill_mfma.hip -- chunked prefill attention over the paged cache on the
// CDNA4 matrix cores.  The prefill of a long prompt is split into chunks
// ("vLLM PagedAttention: uma revolução no throughput de inferência de LLMs",
// feature list: chunked prefill); each chunk's queries are the sequence's last
// n positions and attend causally to every token cached so far, the chunk's own
// K/V included (written to the pool by reshape_and_cache first).  Unlike decode
// this is a dense contraction: a 64-query tile reuses every K/V tile 64 times.
//
// One workgroup of 4 waves per (sequence, 64-query tile, query head); wave w
// owns query rows 16w .. 16w+15 of the tile.  Per step of 32 tokens (two
// 16-token blocks):
//   staging  256 threads load the step's K and V rows (16-byte loads through
//            the block table) into registers one step ahead, then store them to
//            LDS: K row-major [token][dim], V transposed [dim][token].
//   QK       S^T[token][query] = sum_k K[token][k] Q[query][k]
//            v_mfma_f32_16x16x32 (f16/bf16), A = K rows from LDS, B = Q^T held
//            in registers; lane l gets tokens 4(l/16)+r of query l%16.
//   softmax  causal / context mask, running max over the 32 tokens (the lane's
//            8 values, then lanes l^16 and l^32), exp2 in the log2 domain.
//   PV       O^T[dim][query] += sum_k V^T[dim][token_k] P^T[token_k][query]
//            v_mfma_f32_16x16x16 (f16/bf16), A = V^T rows from LDS (4 tokens =
//            8 bytes), B = P^T, which is exactly the lane's own 4 softmax
//            weights of the QK result rounded to the input type.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

template <class T> struct PrefillOp;
template <> struct PrefillOp<BF16> {
  __device__ __forceinline__ static f32x4_t qk(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  }
  __device__ __forceinline__ static f32x4_t pv(const uint2& a, const uint2& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, a), __builtin_bit_cast(bf16x4_t, b),
                                                     c, 0, 0, 0);
  }
  __device__ __forceinline__ static uint32_t pack(float x, float y) {
    return (uint32_t)f32_to_bf16_rne(x) | ((uint32_t)f32_to_bf16_rne(y) << 16);
  }
};
template <> struct PrefillOp<F16> {
  __device__ __forceinline__ static f32x4_t qk(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
  }
  __device__ __forceinline__ static f32x4_t pv(const uint2& a, const uint2& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a), __builtin_bit_cast(f16x4_t, b), c,
                                                 0, 0, 0);
  }
  __device__ __forceinline__ static uint32_t pack(float x, float y) {
    const half2_t h = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, h);
  }
};

template <class T, int D>
struct Prefill {
  static constexpr int BS = 16;                 // tokens per block
  static constexpr int STEP = 32;               // tokens per step (two blocks)
  static constexpr int NW = 4;
  static constexpr int BM = NW * 16;            // query rows per workgroup
  static constexpr int NC = D / 32;             // QK k-steps of 32 dims
  static constexpr int ND = D / 16;             // PV output tiles of 16 dims
  static constexpr int CPR = D / 8;             // 16-byte chunks per token row
  static constexpr int CH = STEP * CPR / (NW * 64);   // chunks per thread per tensor per step
  static constexpr int KSTR = D + 8;            // LDS row stride of K (elements)
  static constexpr int VSTR = STEP + 8;         // LDS row stride of V^T (elements)
  static_assert(CH >= 1 && STEP * CPR == CH * NW * 64, "staging must cover the step exactly");

  struct Smem {
    alignas(16) uint16_t k[2][STEP * KSTR];
    alignas(16) uint16_t vt[2][D * VSTR];
  };
};

template <class T, int D>
__global__ __launch_bounds__(256) void prefill_mfma_kernel(PrefillParams p) {
  using P = Prefill<T, D>;
  using Op = PrefillOp<T>;
  constexpr int STEP = P::STEP, BS = P::BS, NC = P::NC, ND = P::ND, CPR = P::CPR, CH = P::CH;
  __shared__ typename P::Smem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15;
  const int g4 = lane >> 4;

  // work id: query tiles fastest (longest first), then head, then sequence
  const uint32_t L = xcd_remap(blockIdx.x, p.total_wgs, p.xcd_chunk);
  const int tile = p.q_tiles - 1 - (int)(L % (uint32_t)p.q_tiles);
  const uint32_t rest = L / (uint32_t)p.q_tiles;
  const int h = (int)(rest % (uint32_t)p.num_heads);
  const int seq = (int)(rest / (uint32_t)p.num_heads);
  const int kvh = h / p.group;

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
  nkeys = nkeys > ctx ? ctx : (nkeys < 0 ? 0 : nkeys);
  const int nsteps = (nkeys + STEP - 1) / STEP;
  const int wave_last_pos = base + row0 + 16 * w + 15;      // causal limit of the wave's rows

  // B operand of QK: Q^T, lane l holds query row 16w + c16, dims 32c + 8 g4 .. +8
  const int qrow = row0 + 16 * w + c16;
  const bool qreal = qrow < n;
  const int qpos = base + qrow;
  uint4 qf[NC];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + ((size_t)(q0 + (qreal ? qrow : 0)) * p.num_heads + h) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qf[c] = qreal ? *reinterpret_cast<const uint4*>(qp + c * 32 + g4 * 8) : make_uint4(0u, 0u, 0u, 0u);
  }

  float m = -__builtin_inff(), lsum = 0.f;
  f32x4_t O[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) O[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int32_t* table = p.block_tables + (size_t)seq * p.max_blocks_per_seq;
  const size_t block_stride = (size_t)p.num_kv_heads * BS * D;             // elements
  const uint16_t* kpool = reinterpret_cast<const uint16_t*>(p.k_cache) + (size_t)kvh * BS * D;
  const uint16_t* vpool = reinterpret_cast<const uint16_t*>(p.v_cache) + (size_t)kvh * BS * D;

  uint4 kreg[CH], vreg[CH];
  auto load_step = [&](int i) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = tid + j * P::NW * 64;
      const int tok = c / CPR, col = c - tok * CPR;
      const int pos = i * STEP + tok;
      const int blk = pos < nkeys ? table[pos / BS] : -1;
      const bool ok = blk >= 0 && blk < p.num_blocks;
      const size_t off = (size_t)blk * block_stride + (size_t)(pos % BS) * D + col * 8;
      kreg[j] = ok ? *reinterpret_cast<const uint4*>(kpool + off) : make_uint4(0u, 0u, 0u, 0u);
      vreg[j] = ok ? *reinterpret_cast<const uint4*>(vpool + off) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = tid + j * P::NW * 64;
      const int tok = c / CPR, col = c - tok * CPR;
      *reinterpret_cast<uint4*>(&sm.k[buf][tok * P::KSTR + col * 8]) = kreg[j];
      const uint32_t u[4] = {vreg[j].x, vreg[j].y, vreg[j].z, vreg[j].w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sm.vt[buf][(col * 8 + e) * P::VSTR + tok] = (uint16_t)(u[e >> 1] >> (16 * (e & 1)));
    }
  };

  if (nsteps > 0) {
    load_step(0);
    store_step(0);
  }
  __syncthreads();
  for (int i = 0; i < nsteps; ++i) {
    const int buf = i & 1;
    if (i + 1 < nsteps) load_step(i + 1);
    if (i * STEP <= wave_last_pos) {                        // wave-uniform: some key of the step is visible
      // blocks of this step that the table maps outside the pool are skipped
      bool blk_ok[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int pos = i * STEP + kt * BS;
        const int b = pos < nkeys ? table[pos / BS] : -1;
        blk_ok[kt] = b >= 0 && b < p.num_blocks;
      }
      f32x4_t S[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        S[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const uint4 kf = *reinterpret_cast<const uint4*>(&sm.k[buf][(kt * 16 + c16) * P::KSTR + c * 32 + g4 * 8]);
          S[kt] = Op::qk(kf, qf[c], S[kt]);
        }
      }
      float s[2][4];
      float mx = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kpos = i * STEP + kt * BS + g4 * 4 + r;
          const bool vis = blk_ok[kt] && kpos < nkeys && kpos <= qpos && qreal;
          s[kt][r] = vis ? S[kt][r] * p.qk_scale : -__builtin_inff();
          mx = fmaxf(mx, s[kt][r]);
        }
      mx = fmaxf(mx, swz_xor16(mx));
      mx = fmaxf(mx, xor32(mx));
      const float mn = fmaxf(m, mx);
      const float mref = mn == -__builtin_inff() ? 0.f : mn;   // a row with nothing visible yet stays empty
      const float alpha = exp2_fast(m - mref);
      float pr[2][4];
      float ps = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pr[kt][r] = exp2_fast(s[kt][r] - mref);
          ps += pr[kt][r];
        }
      lsum = lsum * alpha + ps;
      m = mn;
      uint2 pk[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        pk[kt] = make_uint2(Op::pack(pr[kt][0], pr[kt][1]), Op::pack(pr[kt][2], pr[kt][3]));
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        O[dt] *= alpha;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const uint2 vf =
              *reinterpret_cast<const uint2*>(&sm.vt[buf][(dt * 16 + c16) * P::VSTR + kt * 16 + g4 * 4]);
          O[dt] = Op::pv(vf, pk[kt], O[dt]);
        }
      }
    }
    if (i + 1 < nsteps) store_step((i + 1) & 1);
    __syncthreads();
  }

  // normalise and write: lane l holds out[query 16w + c16][dims 16 dt + 4 g4 + r]
  lsum += swz_xor16(lsum);
  lsum += xor32(lsum);
  if (qreal) {
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const size_t orow = ((size_t)(q0 + qrow) * p.num_heads + h) * D;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      const size_t e = orow + dt * 16 + g4 * 4;
      uint2 v;
      if constexpr (T::kId == BF16::kId) {
        v = make_uint2((uint32_t)f32_to_bf16_rne(O[dt][0] * inv) | ((uint32_t)f32_to_bf16_rne(O[dt][1] * inv) << 16),
                       (uint32_t)f32_to_bf16_rne(O[dt][2] * inv) | ((uint32_t)f32_to_bf16_rne(O[dt][3] * inv) << 16));
      } else {
        v = make_uint2(PrefillOp<F16>::pack(O[dt][0] * inv, O[dt][1] * inv),
                       PrefillOp<F16>::pack(O[dt][2] * inv, O[dt][3] * inv));
      }
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + e) = v;
    }
  }
}

bool prefill_supported(int q_dtype, int kv_dtype, int head_dim, int block_size) {
  return q_dtype == kv_dtype && (q_dtype == F16::kId || q_dtype == BF16::kId) && (head_dim == 64 || head_dim == 128) &&
         block_size == 16;
}

int prefill_tile_rows() { return Prefill<F16, 128>::BM; }

template <class T, int D>
static hipError_t launch_prefill_t(const PrefillParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_mfma_kernel<T, D>), dim3(p.total_wgs), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams& p, int dtype, int head_dim, hipStream_t stream) {
  if (dtype == F16::kId) return head_dim == 64 ? launch_prefill_t<F16, 64>(p, stream) : launch_prefill_t<F16, 128>(p, stream);
  if (dtype == BF16::kId) return head_dim == 64 ? launch_prefill_t<BF16, 64>(p, stream) : launch_prefill_t<BF16, 128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
