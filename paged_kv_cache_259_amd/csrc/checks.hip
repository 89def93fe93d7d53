// checks.hip -- debug checks of the device-resident values each call takes on
// trust: block tables and context lengths, slots, block-copy pairs, the host
// order, the shared decode's groups, the prefill's query offsets and the
// per-kv-head scales of an 8-bit cache.
//
// The pages fix what these values mean: a sequence's table names its blocks in
// order and the token at position pos sits in block table[pos / bs] at offset
// pos % bs ("PagedAttention", Ultralytics glossary, section "Cách phân trang
// hoạt động"); a block shared by several sequences is copied to a fresh block
// before one of them writes into it ("KV cache paginado e batching contínuo
// para LLMs", section "Como funciona"; same glossary page, section "Chia sẻ
// block giữa các chuỗi").  The kernels never fault on values that break these
// rules (they clamp or skip them), but they then give wrong numbers.  With the
// checks on, every entry point first runs the matching check kernels on its
// stream, waits for them, and returns PKV_ERR_PRECONDITION without launching
// anything else when a value is out of place.
//
// Every check is a plain scan: one thread per value, or for "no two equal"
// one thread per value comparing it against all earlier ones through LDS
// tiles (quadratic, which is fine for a debug aid and needs no scratch).
// Violations go to a two-word report in a static device array: a count and the
// smallest (kind << 48 | index), both by atomics.
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

using u64 = unsigned long long;

// [0] violations, [1] smallest (kind << 48 | index); one copy per GPU
static __device__ __align__(256) u64 check_report[2];

constexpr long long kIndexMask = (1LL << 48) - 1;

__device__ __forceinline__ void flag(u64* r, int kind, long long index) {
  atomicAdd(&r[0], 1ull);
  atomicMin(&r[1], ((u64)kind << 48) | (u64)(index < 0 ? 0 : (index > kIndexMask ? kIndexMask : index)));
}

__global__ void check_clear_kernel(u64* r) {
  if (threadIdx.x == 0) {
    r[0] = 0ull;
    r[1] = ~0ull;
  }
}

// One workgroup per sequence: its context length, then the table entries a
// kernel reads for it (the first ceil(ctx / bs), at most max_blocks_per_seq).
__global__ __launch_bounds__(256) void check_tables_kernel(const int32_t* tables, int mbs, const int32_t* ctx_lens,
                                                            int bs, int num_blocks, int max_ctx, u64* r) {
  const int s = blockIdx.x;
  const int c = ctx_lens[s];
  const long long need = c <= 0 ? 0 : ((long long)c + bs - 1) / bs;
  if (threadIdx.x == 0 && (c < 0 || c > max_ctx || need > mbs)) flag(r, PKV_CHECK_CONTEXT_LEN, s);
  const long long nb = need < mbs ? need : mbs;
  for (long long j = threadIdx.x; j < nb; j += blockDim.x) {
    const int b = tables[(size_t)s * mbs + j];
    if (b < 0 || b >= num_blocks) flag(r, PKV_CHECK_BLOCK_ID, (long long)s * mbs + j);
  }
}

// Value i of a strided array: v[i * stride + off].
template <class T>
struct Strided {
  const T* v;
  int stride, off;
  __device__ __forceinline__ long long operator()(long long i) const { return (long long)v[i * stride + off]; }
};

// Values outside [lo, hi); negative values are allowed when neg_ok.
template <class T>
__global__ __launch_bounds__(256) void check_range_kernel(Strided<T> a, long long n, long long hi, bool neg_ok,
                                                          int kind, u64* r) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const long long x = a(i);
  if (x < 0 ? !neg_ok : x >= hi) flag(r, kind, i);
}

// Value j of `a`, inside [0, hi), equal to a value of `b`: to one at an index
// below j when earlier_only (b is then a itself: "no two equal", the later one
// flagged), to any of b's m values otherwise.  When m_dev is given, b holds
// min(m, max(0, *m_dev)) values (a bound only the device knows).
template <class T>
__global__ __launch_bounds__(256) void check_member_kernel(Strided<T> a, long long n, Strided<T> b, long long m,
                                                           const int32_t* m_dev, long long hi, bool earlier_only,
                                                           int kind, u64* r) {
  __shared__ long long tile[256];
  if (m_dev) {
    const long long md = *m_dev;
    m = md < 0 ? 0 : (md < m ? md : m);
  }
  if (earlier_only) n = n < m ? n : m;
  const long long j = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long x = j < n ? a(j) : -1;
  // block-uniform bound on the b values any thread of the block compares with
  long long end = m;
  if (earlier_only) {
    const long long last = (long long)blockIdx.x * blockDim.x + blockDim.x;
    end = last < m ? last : m;
  }
  bool hit = false;
  for (long long i0 = 0; i0 < end; i0 += 256) {
    __syncthreads();
    const long long i = i0 + threadIdx.x;
    tile[threadIdx.x] = i < end ? b(i) : -1;
    __syncthreads();
    long long lim = end - i0 < 256 ? end - i0 : 256;
    if (earlier_only && j - i0 < lim) lim = j - i0;       // only b values at indices below j
    for (long long k = 0; k < lim; ++k) hit |= tile[k] == x;
  }
  if (j < n && x >= 0 && x < hi && hit) flag(r, kind, j);
}

// Decode with append: the new token of sequence s (context c >= 1) goes to the
// slot of position c - 1, block table[s][(c - 1) / bs] at offset (c - 1) % bs.
// A negative slot (skipped by the write) is allowed.
__global__ __launch_bounds__(256) void check_append_slots_kernel(const int64_t* slots, const int32_t* tables, int mbs,
                                                                 const int32_t* ctx_lens, int S, int bs, u64* r) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= S) return;
  const int c = ctx_lens[s];
  const int64_t slot = slots[s];
  if (c < 1 || slot < 0) return;
  const long long j = (long long)(c - 1) / bs;
  if (j >= mbs) return;                                     // a bad context length, flagged by the table check
  const long long want = (long long)tables[(size_t)s * mbs + j] * bs + (c - 1) % bs;
  if (slot != want) flag(r, PKV_CHECK_APPEND_SLOT, s);
}

// Shared-block decode, one workgroup per group g: the offsets (group_offsets[0]
// == 0, non-decreasing, group_offsets[G] == S, at most max_group_size members),
// the shared count (>= 0), the members (in [0, S)), and that the tables of all
// the group's members agree on the blocks the kernel reads as shared: the first
// min(shared count, (c - 1) / bs) over the members' contexts c, read through
// the first member in range.  Member positions are clamped as the kernel
// clamps them.
__global__ __launch_bounds__(256) void check_groups_kernel(const int32_t* off, const int32_t* mem, const int32_t* shared,
                                                           int G, int gmax, const int32_t* tables, int mbs,
                                                           const int32_t* ctx_lens, int S, int bs, int ctx_cap,
                                                           u64* r) {
  __shared__ int s_lim, s_lead;
  const int g = blockIdx.x;
  const int a = off[g], b = off[g + 1];
  if (threadIdx.x == 0) {
    const bool bad = (g == 0 && a != 0) || (g == G - 1 && b != S) || a < 0 || b < a || b > S || b - a > gmax ||
                     shared[g] < 0;
    if (bad) flag(r, PKV_CHECK_GROUP, g);
    s_lim = 0x7fffffff;
    s_lead = -1;
  }
  __syncthreads();
  const int o0 = a < 0 ? 0 : (a > S ? S : a);
  const int o1max = o0 + gmax < S ? o0 + gmax : S;
  const int o1 = b < o0 ? o0 : (b > o1max ? o1max : b);
  for (int i = o0 + threadIdx.x; i < o1; i += blockDim.x) {
    const int s = mem[i];
    if (s < 0 || s >= S) {
      flag(r, PKV_CHECK_GROUP_MEMBER, i);
      continue;
    }
    int c = ctx_lens[s];
    c = c < 0 ? 0 : (c > ctx_cap ? ctx_cap : c);
    atomicMin(&s_lim, c > 0 ? (c - 1) / bs : 0);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = o0; i < o1; ++i) {
      const int s = mem[i];
      if (s >= 0 && s < S) { s_lead = s; break; }
    }
  }
  __syncthreads();
  const int lead = s_lead;
  if (lead < 0) return;
  int nsh = shared[g];
  nsh = nsh < 0 ? 0 : (nsh > s_lim ? s_lim : nsh);
  nsh = nsh < mbs ? nsh : mbs;
  const long long pairs = (long long)(o1 - o0) * nsh;
  for (long long t = threadIdx.x; t < pairs; t += blockDim.x) {
    const int s = mem[o0 + (int)(t / nsh)];
    const int j = (int)(t % nsh);
    if (s < 0 || s >= S || s == lead) continue;
    if (tables[(size_t)s * mbs + j] != tables[(size_t)lead * mbs + j]) flag(r, PKV_CHECK_SHARED_BLOCK, (long long)s * mbs + j);
  }
}

// Chunked prefill: query_start_loc[0] == 0, non-decreasing, inside
// [0, num_tokens], query_start_loc[S] == num_tokens, no chunk longer than
// max_query_len; entry s is flagged.
__global__ __launch_bounds__(256) void check_query_starts_kernel(const int32_t* qsl, int S, int num_tokens, int max_q,
                                                                 u64* r) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s > S) return;
  const int x = qsl[s];
  bool bad = x < 0 || x > num_tokens || (s == 0 && x != 0) || (s == S && x != num_tokens);
  if (s > 0) {
    const int prev = qsl[s - 1];
    bad = bad || x < prev || (long long)x - prev > max_q;
  }
  if (bad) flag(r, PKV_CHECK_QUERY_START, s);
}

// Per-kv-head scales of an 8-bit cache: positive and finite.  Entry i of
// k_scales is flagged as index i, of v_scales as n + i.
__global__ __launch_bounds__(256) void check_scales_kernel(const float* ks, const float* vs, int n, u64* r) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= 2 * n) return;
  const float* a = i < n ? ks : vs;
  if (!a) return;
  const float x = a[i < n ? i : i - n];
  if (!(x > 0.f && x <= 3.402823466e38f)) flag(r, PKV_CHECK_SCALE, i);
}

unsigned grid_of(long long n) { return (unsigned)((n + 255) / 256); }

// 1 on, 0 off, -1: the PKV_DEBUG environment variable decides
std::atomic<int> g_mode{-1};
std::mutex g_mu;
constexpr int kMaxDevices = 64;
std::atomic<void*> g_report_ptr[kMaxDevices];

struct LastReport {
  long long violations = 0;
  int kind = 0;
  long long index = -1;
};
thread_local LastReport t_last;

// Device address of the current device's report, looked up once per device.
u64* report_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_report_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(check_report)) != hipSuccess) return nullptr;
    g_report_ptr[dev].store(p, std::memory_order_release);
  }
  return static_cast<u64*>(p);
}

}  // namespace

bool debug_checks_on() {
  const int m = g_mode.load(std::memory_order_relaxed);
  if (m >= 0) return m != 0;
  const char* e = getenv("PKV_DEBUG");
  return e && *e && strcmp(e, "0") != 0;
}

struct DeviceChecks::Impl {
  std::unique_lock<std::mutex> lock{g_mu};
  hipStream_t stream;
  u64* r = nullptr;
  bool failed = false;
};

DeviceChecks::DeviceChecks(hipStream_t stream) : impl_(new Impl) {
  impl_->stream = stream;
  t_last = LastReport{};
  (void)hipGetLastError();
  impl_->r = report_ptr();
  if (!impl_->r) {
    impl_->failed = true;
    return;
  }
  hipLaunchKernelGGL(check_clear_kernel, dim3(1), dim3(64), 0, stream, impl_->r);
  note(hipGetLastError());
}

DeviceChecks::~DeviceChecks() { delete impl_; }

void DeviceChecks::note(hipError_t e) { impl_->failed = impl_->failed || e != hipSuccess; }

void DeviceChecks::tables(const int32_t* tables, int mbs, const int32_t* ctx_lens, int num_seqs, int bs,
                          int num_blocks, int max_ctx) {
  if (impl_->failed || num_seqs <= 0) return;
  hipLaunchKernelGGL(check_tables_kernel, dim3(num_seqs), dim3(256), 0, impl_->stream, tables, mbs, ctx_lens, bs,
                     num_blocks, max_ctx, impl_->r);
  note(hipGetLastError());
}

void DeviceChecks::permutation(const int32_t* order, int n) {
  if (impl_->failed || !order || n <= 0) return;
  const Strided<int32_t> a{order, 1, 0};
  hipLaunchKernelGGL(check_range_kernel<int32_t>, dim3(grid_of(n)), dim3(256), 0, impl_->stream, a, (long long)n,
                     (long long)n, false, (int)PKV_CHECK_SEQ_ORDER, impl_->r);
  note(hipGetLastError());
  hipLaunchKernelGGL(check_member_kernel<int32_t>, dim3(grid_of(n)), dim3(256), 0, impl_->stream, a, (long long)n, a,
                     (long long)n, (const int32_t*)nullptr, (long long)n, true, (int)PKV_CHECK_SEQ_ORDER, impl_->r);
  note(hipGetLastError());
}

void DeviceChecks::slots(const int64_t* slots, int n, long long num_slots) {
  if (impl_->failed || n <= 0) return;
  const Strided<int64_t> a{slots, 1, 0};
  hipLaunchKernelGGL(check_range_kernel<int64_t>, dim3(grid_of(n)), dim3(256), 0, impl_->stream, a, (long long)n,
                     num_slots, true, (int)PKV_CHECK_SLOT, impl_->r);
  note(hipGetLastError());
  hipLaunchKernelGGL(check_member_kernel<int64_t>, dim3(grid_of(n)), dim3(256), 0, impl_->stream, a, (long long)n, a,
                     (long long)n, (const int32_t*)nullptr, num_slots, true, (int)PKV_CHECK_DUPLICATE_SLOT, impl_->r);
  note(hipGetLastError());
}

void DeviceChecks::append_slots(const int64_t* slots, const int32_t* tables, int mbs, const int32_t* ctx_lens,
                                int num_seqs, int bs, long long num_slots) {
  if (impl_->failed || num_seqs <= 0) return;
  this->slots(slots, num_seqs, num_slots);
  hipLaunchKernelGGL(check_append_slots_kernel, dim3(grid_of(num_seqs)), dim3(256), 0, impl_->stream, slots, tables,
                     mbs, ctx_lens, num_seqs, bs, impl_->r);
  note(hipGetLastError());
}

void DeviceChecks::pairs(const int64_t* mapping, int n, int src_blocks, int dst_blocks, bool same_pool) {
  if (impl_->failed || n <= 0) return;
  const Strided<int64_t> src{mapping, 2, 0}, dst{mapping, 2, 1};
  hipLaunchKernelGGL(check_range_kernel<int64_t>, dim3(grid_of(n)), dim3(256), 0, impl_->stream, src, (long long)n,
                     (long long)src_blocks, false, (int)PKV_CHECK_PAIR_ID, impl_->r);
  note(hipGetLastError());
  hipLaunchKernelGGL(check_range_kernel<int64_t>, dim3(grid_of(n)), dim3(256), 0, impl_->stream, dst, (long long)n,
                     (long long)dst_blocks, false, (int)PKV_CHECK_PAIR_ID, impl_->r);
  note(hipGetLastError());
  hipLaunchKernelGGL(check_member_kernel<int64_t>, dim3(grid_of(n)), dim3(256), 0, impl_->stream, dst, (long long)n,
                     dst, (long long)n, (const int32_t*)nullptr, (long long)dst_blocks, true,
                     (int)PKV_CHECK_DUPLICATE_DST, impl_->r);
  note(hipGetLastError());
  if (same_pool) {
    hipLaunchKernelGGL(check_member_kernel<int64_t>, dim3(grid_of(n)), dim3(256), 0, impl_->stream, dst,
                       (long long)n, src, (long long)n, (const int32_t*)nullptr, (long long)dst_blocks, false,
                       (int)PKV_CHECK_DST_IS_SRC, impl_->r);
    note(hipGetLastError());
  }
}

void DeviceChecks::groups(const int32_t* offsets, const int32_t* members, const int32_t* shared, int num_groups,
                          int max_group_size, const int32_t* tables, int mbs, const int32_t* ctx_lens, int num_seqs,
                          int bs, int ctx_cap) {
  if (impl_->failed || num_groups <= 0 || num_seqs <= 0) return;
  hipLaunchKernelGGL(check_groups_kernel, dim3(num_groups), dim3(256), 0, impl_->stream, offsets, members, shared,
                     num_groups, max_group_size, tables, mbs, ctx_lens, num_seqs, bs, ctx_cap, impl_->r);
  note(hipGetLastError());
  // no sequence in two groups: the members listed, group_offsets[G] of them
  // (at most S), pairwise distinct
  const Strided<int32_t> a{members, 1, 0};
  hipLaunchKernelGGL(check_member_kernel<int32_t>, dim3(grid_of(num_seqs)), dim3(256), 0, impl_->stream, a,
                     (long long)num_seqs, a, (long long)num_seqs, offsets + num_groups, (long long)num_seqs, true,
                     (int)PKV_CHECK_GROUP_MEMBER, impl_->r);
  note(hipGetLastError());
}

void DeviceChecks::scales(const float* k_scales, const float* v_scales, int num_kv_heads) {
  if (impl_->failed || num_kv_heads <= 0 || (!k_scales && !v_scales)) return;
  hipLaunchKernelGGL(check_scales_kernel, dim3(grid_of(2LL * num_kv_heads)), dim3(256), 0, impl_->stream, k_scales,
                     v_scales, num_kv_heads, impl_->r);
  note(hipGetLastError());
}

void DeviceChecks::query_starts(const int32_t* qsl, int num_seqs, int num_tokens, int max_query_len) {
  if (impl_->failed || num_seqs <= 0) return;
  hipLaunchKernelGGL(check_query_starts_kernel, dim3(grid_of((long long)num_seqs + 1)), dim3(256), 0, impl_->stream,
                     qsl, num_seqs, num_tokens, max_query_len, impl_->r);
  note(hipGetLastError());
}

int DeviceChecks::finish() {
  if (impl_->failed) return PKV_ERR_LAUNCH;
  u64 host[2] = {0ull, ~0ull};
  if (hipMemcpyAsync(host, impl_->r, sizeof(host), hipMemcpyDeviceToHost, impl_->stream) != hipSuccess ||
      hipStreamSynchronize(impl_->stream) != hipSuccess)
    return PKV_ERR_LAUNCH;
  t_last.violations = (long long)host[0];
  if (host[0] == 0) return PKV_OK;
  t_last.kind = (int)(host[1] >> 48);
  t_last.index = (long long)(host[1] & (u64)kIndexMask);
  return PKV_ERR_PRECONDITION;
}

}  // namespace pkv

extern "C" {

int pkv_set_debug_checks(int mode) {
  const int m = mode > 0 ? 1 : (mode == 0 ? 0 : -1);
  return pkv::g_mode.exchange(m);
}

int pkv_debug_report(int64_t* violations, int* kind, int64_t* index) {
  if (violations) *violations = pkv::t_last.violations;
  if (kind) *kind = pkv::t_last.violations ? pkv::t_last.kind : 0;
  if (index) *index = pkv::t_last.violations ? pkv::t_last.index : -1;
  return PKV_OK;
}

}  // extern "C"
