// pkv_api.hip -- the attention half of the C ABI declared in include/pkv.h:
// host-side argument checks, the choice of kernel family and launch shape, and
// launches; plus the status strings and version.
// Nothing here allocates or frees; only the debug checks (checks.hip, off by
// default) synchronise.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "pkv.h"
#include "pkv_internal.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
#ifndef PKV_AUTO_PARTITION
#define PKV_AUTO_PARTITION 512
#endif
constexpr int kAutoPartitionTokens = PKV_AUTO_PARTITION;

#ifndef PKV_SLICE_WGS_VEC
#define PKV_SLICE_WGS_VEC 1280   // resident 4-wave workgroups of the vector kernel on 256 CUs
#endif
#ifndef PKV_SLICE_WGS_MFMA
#define PKV_SLICE_WGS_MFMA 1024  // resident 4-wave workgroups of the MFMA kernel on 256 CUs
#endif
constexpr int kSingleMaxTokens = 256;    // contexts this short: one pass, no split
#ifndef PKV_LONGEST_FIRST
#define PKV_LONGEST_FIRST 1
#endif
#ifndef PKV_PARTITION_XCD_CHUNK
#define PKV_PARTITION_XCD_CHUNK 64   // fixed partitions: runs of 64 work ids per XCD
#endif
#ifndef PKV_HEAD_RUNS
#define PKV_HEAD_RUNS 1              // one pass with 16+ head units, a multiple of 8: head_runs order
#endif

enum Mode { kSingle = 0, kPartitions = 1, kSlices = 2 };

struct Plan {
  int path;            // PKV_PATH_*
  int mode;            // Mode
  int part_tokens;     // tokens per partition (partitions / single pass), 0 for slices
  int num_parts;       // partitions per sequence, or number of slices
  int units;           // head units per sequence: query heads (vector) or kv heads (MFMA)
  bool longest_first;  // one pass in decreasing context order
  size_t rows;         // fp32 summary rows in the workspace
  size_t off_m, off_l, off_prefix;
  size_t ws_bytes;     // workspace needed (0 for a single pass)
};

// PKV_ATTN_PATH=vector forces the vector family; =mfma asks for the MFMA family.
int forced_path() {
  const char* e = getenv("PKV_ATTN_PATH");
  if (!e) return -1;
  if (!strcmp(e, "vector")) return PKV_PATH_VECTOR;
  if (!strcmp(e, "mfma")) return PKV_PATH_MFMA;
  return -1;
}

// PKV_XCD_CHUNK=<n> overrides the XCD run length of every launch (tuning).
int xcd_chunk_env() {
  const char* e = getenv("PKV_XCD_CHUNK");
  if (e && *e) {
    const int v = atoi(e);
    if (v >= 0 && v <= 4096) return v;
  }
  return -1;
}

// XCD run length of a launch (see xcd_remap): runs of 64 work ids for fixed
// partitions, the hardware order otherwise.
int xcd_chunk_for(int mode) {
  const int v = xcd_chunk_env();
  if (v >= 0) return v;
  return mode == kPartitions ? PKV_PARTITION_XCD_CHUNK : 0;
}

// One pass with U head units per sequence (U >= 16, a multiple of 8): the
// head_runs order, so each XCD reads U/8 neighbouring (block, head) tiles of a
// block -- one contiguous run -- instead of tiles 8 heads apart, and a head keeps
// its XCD across sequences (LLaMA-13B shape: 179.6 -> about 176 us).  With fewer
// units (grouped heads: 8 kv heads) it is the hardware order anyway.  0 = off.
uint32_t head_run_units_for(int mode, int units) {
  if (!PKV_HEAD_RUNS || mode != kSingle || xcd_chunk_env() >= 0) return 0;
  return units >= 16 && units % 8 == 0 ? (uint32_t)units : 0;
}

bool compact_partitions_env() {
  const char* e = getenv("PKV_COMPACT_PARTITIONS");
  return !(e && *e == '0');
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int make_plan(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size, int max_context_len,
              int partition_size, int q_dtype, int kv_dtype, Plan* out) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      max_context_len < 0)
    return PKV_ERR_BAD_SIZE;
  if (num_heads % num_kv_heads != 0) return PKV_ERR_HEAD_GROUPING;
  if (pkv::dtype_bytes(q_dtype) != 2 && q_dtype != PKV_F32) return PKV_ERR_UNSUPPORTED;
  if (pkv::dtype_bytes(kv_dtype) == 0) return PKV_ERR_UNSUPPORTED;
  if (partition_size < 0 || (partition_size > 0 && partition_size % block_size != 0)) return PKV_ERR_PARTITION;
  const int group = num_heads / num_kv_heads;
  const bool vec_ok = pkv::vector_supported(q_dtype, kv_dtype, head_dim, block_size);
  const bool mfma_ok = pkv::mfma_supported(q_dtype, kv_dtype, head_dim, block_size, group);
  int path;
  const int forced = forced_path();
  if (forced == PKV_PATH_VECTOR) path = PKV_PATH_VECTOR;
  else if (forced == PKV_PATH_MFMA) path = PKV_PATH_MFMA;
  else path = mfma_ok ? PKV_PATH_MFMA : PKV_PATH_VECTOR;
  if ((path == PKV_PATH_MFMA && !mfma_ok) || (path == PKV_PATH_VECTOR && !vec_ok)) return PKV_ERR_UNSUPPORTED;

  Plan pl{};
  pl.path = path;
  pl.units = path == PKV_PATH_MFMA ? num_kv_heads : num_heads;
  const int max_blocks = (max_context_len + block_size - 1) / block_size;
  if (partition_size > 0 || num_seqs > pkv::kMaxSliceSeqs) {
    // fixed partitions (the caller's size, or 512 tokens for very large batches)
    const int ptoks = partition_size > 0 ? partition_size : kAutoPartitionTokens / block_size * block_size;
    const int nparts = (max_context_len + ptoks - 1) / ptoks;
    if (nparts > 1) {
      pl.mode = kPartitions;
      pl.part_tokens = ptoks;
      pl.num_parts = nparts;
      pl.rows = (size_t)num_seqs * num_heads * nparts;
    } else {
      pl.mode = kSingle;
    }
  } else if (max_context_len > kSingleMaxTokens &&
             (long long)num_seqs * pl.units < 2LL * (path == PKV_PATH_MFMA ? PKV_SLICE_WGS_MFMA : PKV_SLICE_WGS_VEC)) {
    // few (sequence, head) units for the resident workgroups: balanced slices,
    // about one round of resident workgroups, at least two blocks per slice
    const int target = path == PKV_PATH_MFMA ? PKV_SLICE_WGS_MFMA : PKV_SLICE_WGS_VEC;
    long long ns = (target + pl.units - 1) / pl.units;
    const long long items = (long long)num_seqs * max_blocks;
    if (ns > items / 2) ns = items / 2;
    if (ns > 1) {
      pl.mode = kSlices;
      pl.num_parts = (int)ns;
      pl.rows = (size_t)ns * 2 * num_heads;
    } else {
      pl.mode = kSingle;
    }
  } else {
    pl.mode = kSingle;
  }
  if (pl.mode == kSingle) {
    // one pass: one partition covering the whole (rounded-up) context; with
    // enough units, workgroups take sequences longest first
    pl.part_tokens = max_blocks > 0 ? max_blocks * block_size : block_size;
    pl.num_parts = 1;
    pl.longest_first = PKV_LONGEST_FIRST && num_seqs > 1 && num_seqs <= pkv::kMaxSliceSeqs;
  }
  if (pl.mode != kSingle) {
    pl.off_m = align_up(pl.rows * head_dim * sizeof(float), 256);
    pl.off_l = pl.off_m + align_up(pl.rows * sizeof(float), 256);
    pl.off_prefix = pl.off_l + align_up(pl.rows * sizeof(float), 256);
    pl.ws_bytes = pl.off_prefix + (pl.mode == kSlices ? align_up((size_t)(num_seqs + 1) * sizeof(int), 256) : 0);
  }
  const long long wgs = pl.mode == kSlices ? (long long)pl.num_parts * pl.units
                                           : (long long)num_seqs * pl.units * pl.num_parts;
  if (wgs > 2147483647LL) return PKV_ERR_BAD_SIZE;
  *out = pl;
  return PKV_OK;
}

}  // namespace

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL_POINTER: return "a required pointer is NULL";
    case PKV_ERR_BAD_SIZE: return "a size argument is out of range";
    case PKV_ERR_HEAD_GROUPING: return "num_heads is not a multiple of num_kv_heads";
    case PKV_ERR_UNSUPPORTED: return "unsupported head_dim / block_size / dtype combination or misaligned buffer";
    case PKV_ERR_PARTITION: return "partition_size must be 0 or a positive multiple of block_size";
    case PKV_ERR_WORKSPACE: return "workspace missing or smaller than pkv_attention_workspace_bytes()";
    case PKV_ERR_LAUNCH: return "HIP kernel launch failed";
    case PKV_ERR_SCALE: return "FP8 scale must be a positive finite number";
    case PKV_ERR_MEMORY_KIND: return "buffer is neither device memory nor pinned host memory";
    case PKV_ERR_SCRATCH_LIMIT:
      return "the call needs more split-context scratch than the library's static scratch holds "
             "(PKV_STATIC_SCRATCH_BYTES); call pkv_paged_attention_decode with a workspace instead";
    case PKV_ERR_PRECONDITION:
      return "debug checks: a device-resident value (block table, context length, slot, pair, order, group, "
             "query offset or per-head scale) breaks the call's preconditions; nothing was launched "
             "(see pkv_debug_report)";
  }
  return "unknown status";
}

int pkv_version(void) { return 200; }

int pkv_attention_plan(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                       int max_context_len, int partition_size, int q_dtype, int kv_dtype, int* path,
                       int* partition_tokens, int* num_partitions) {
  Plan pl;
  const int st = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len,
                           partition_size, q_dtype, kv_dtype, &pl);
  if (st != PKV_OK) return st;
  if (path) *path = pl.path;
  if (partition_tokens) *partition_tokens = pl.mode == kSlices ? 0 : pl.part_tokens;
  if (num_partitions) *num_partitions = pl.num_parts;
  return PKV_OK;
}

size_t pkv_attention_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                                     int max_context_len, int partition_size, int q_dtype, int kv_dtype) {
  Plan pl;
  if (make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len, partition_size, q_dtype,
                kv_dtype, &pl) != PKV_OK)
    return 0;
  return pl.ws_bytes;
}

}  // extern "C"

namespace {

// The calling thread's K/V load policy (pkv_set_kv_load_policy).
thread_local int t_kv_load_policy = PKV_KV_LOADS_STREAM;

// Decode, optionally writing each sequence's new token first (new_k != NULL).
int decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache, const void* new_k,
                const void* new_v, const int64_t* slot_mapping, const int32_t* block_tables, int max_blocks_per_seq,
                const int32_t* context_lens, const int32_t* seq_order, int num_seqs, int num_heads, int num_kv_heads,
                int head_dim, int block_size, int num_blocks, int max_context_len, float scale, float k_scale,
                float v_scale, const float* k_scales, const float* v_scales, int q_dtype, int kv_dtype,
                int partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  int st = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len, partition_size,
                     q_dtype, kv_dtype, &pl);
  if (st != PKV_OK) return st;
  if (max_blocks_per_seq <= 0 || num_blocks <= 0) return PKV_ERR_BAD_SIZE;
  if (!isfinite(scale)) return PKV_ERR_BAD_SIZE;
  const bool fp8 = kv_dtype == PKV_FP8_E4M3 || kv_dtype == PKV_FP8_E5M2;
  if (fp8 && !((k_scales || pkv::good_scale(k_scale)) && (v_scales || pkv::good_scale(v_scale)))) return PKV_ERR_SCALE;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PKV_ERR_NULL_POINTER;
  if (!pkv::aligned16(out) || !pkv::aligned16(q) || !pkv::aligned16(k_cache) || !pkv::aligned16(v_cache)) return PKV_ERR_UNSUPPORTED;
  if (new_k) {
    if (!new_v || !slot_mapping) return PKV_ERR_NULL_POINTER;
    if (!pkv::aligned16(new_k) || !pkv::aligned16(new_v)) return PKV_ERR_UNSUPPORTED;
  }
  if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes || !pkv::aligned16(workspace)))
    return PKV_ERR_WORKSPACE;

  pkv::AttnParams p{};
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  char* ws = reinterpret_cast<char*>(workspace);
  if (pl.mode != kSingle) {
    p.ws_o = reinterpret_cast<float*>(ws);
    p.ws_m = reinterpret_cast<float*>(ws + pl.off_m);
    p.ws_l = reinterpret_cast<float*>(ws + pl.off_l);
    p.ws_prefix = pl.mode == kSlices ? reinterpret_cast<int*>(ws + pl.off_prefix) : nullptr;
  }
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_heads / num_kv_heads;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  long long cap_table = (long long)max_blocks_per_seq * block_size;
  long long cap;
  if (pl.mode == kSlices) {
    p.num_slices = pl.num_parts;
    p.longest_first = 0;
    p.partition_blocks = 0;
    p.num_partitions = 0;
    cap = ((long long)max_context_len + block_size - 1) / block_size * block_size;
  } else {
    p.num_slices = 0;
    p.longest_first = pl.longest_first ? 1 : 0;
    p.seq_order = pl.longest_first ? seq_order : nullptr;
    p.partition_blocks = pl.part_tokens / block_size;
    p.num_partitions = pl.num_parts;
    cap = (long long)pl.part_tokens * pl.num_parts;
  }
  if (cap > cap_table) cap = cap_table;
  p.ctx_cap = (int)(cap < 2147483647LL ? cap : 2147483647LL);
  p.new_k = new_k;
  p.new_v = new_v;
  p.slot_mapping = new_k ? slot_mapping : nullptr;
  p.enc_k_scale = k_scale;
  p.enc_v_scale = v_scale;
  p.k_scales = fp8 ? k_scales : nullptr;
  p.v_scales = fp8 ? v_scales : nullptr;
  p.qk_scale = scale * kLog2e * (fp8 && !k_scales ? k_scale : 1.f);
  p.v_scale = fp8 && !v_scales ? v_scale : 1.f;
  p.total_wgs = (uint32_t)(pl.mode == kSlices ? (size_t)pl.num_parts * pl.units
                                              : (size_t)num_seqs * pl.units * pl.num_parts);
  p.xcd_chunk = (uint32_t)xcd_chunk_for(pl.mode);
  // Fixed partitions on the matrix-core family walk the units that exist,
  // sequence by sequence, each XCD on one kv head (hardware order): long-context
  // split-K at 512-token partitions 474.5 -> 464.5 us against the reversed
  // partition-major grid.  PKV_COMPACT_PARTITIONS=0 keeps the grid.
  if (pl.mode == kPartitions && pl.path == PKV_PATH_MFMA && num_seqs <= pkv::kMaxSliceSeqs &&
      compact_partitions_env()) {
    p.compact_partitions = 1;
    if (xcd_chunk_env() < 0) p.xcd_chunk = 0;
  }
  p.head_run_units = head_run_units_for(pl.mode, pl.units);
  p.kv_cached = t_kv_load_policy == PKV_KV_LOADS_CACHED ? 1 : 0;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (pkv::debug_checks_on()) {
    pkv::DeviceChecks c(s);
    c.tables(block_tables, max_blocks_per_seq, context_lens, num_seqs, block_size, num_blocks, max_context_len);
    c.permutation(seq_order, num_seqs);
    if (fp8) c.scales(k_scales, v_scales, num_kv_heads);
    if (new_k)
      c.append_slots(slot_mapping, block_tables, max_blocks_per_seq, context_lens, num_seqs, block_size,
                     (long long)num_blocks * block_size);
    const int cst = c.finish();
    if (cst != PKV_OK) return cst;
  }
  (void)hipGetLastError();  // start from a clean error state
  hipError_t e;
  if (pl.path == PKV_PATH_MFMA)
    e = new_k ? pkv::launch_attention_mfma_append(p, q_dtype, kv_dtype, head_dim, s)
              : pkv::launch_attention_mfma(p, q_dtype, kv_dtype, head_dim, s);
  else
    e = new_k ? pkv::launch_attention_vector_append(p, q_dtype, kv_dtype, head_dim, block_size, s)
              : pkv::launch_attention_vector(p, q_dtype, kv_dtype, head_dim, block_size, s);
  if (e != hipSuccess) return PKV_ERR_LAUNCH;
  if (pl.mode != kSingle) {
    pkv::ReduceParams r{};
    r.out = out;
    r.context_lens = context_lens;
    r.ws_m = p.ws_m;
    r.ws_l = p.ws_l;
    r.ws_o = p.ws_o;
    r.ws_prefix = p.ws_prefix;
    r.num_seqs = num_seqs;
    r.num_heads = num_heads;
    r.num_partitions = p.num_partitions;
    r.partition_tokens = pl.part_tokens;
    r.num_slices = p.num_slices;
    r.ctx_cap = p.ctx_cap;
    e = pkv::launch_attention_reduce(r, q_dtype, head_dim, s);
  }
  return pkv::launch_status(e);
}

}  // namespace

extern "C" {

int pkv_set_kv_load_policy(int policy) {
  if (policy != PKV_KV_LOADS_STREAM && policy != PKV_KV_LOADS_CACHED) return PKV_ERR_BAD_SIZE;
  const int prev = t_kv_load_policy;
  t_kv_load_policy = policy;
  return prev;
}

int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                               const int32_t* seq_order, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                               int block_size, int num_blocks, int max_context_len, float scale, float k_scale,
                               float v_scale, const float* k_scales, const float* v_scales, int q_dtype, int kv_dtype,
                               int partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, nullptr, nullptr, nullptr, block_tables, max_blocks_per_seq,
                     context_lens, seq_order, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_context_len, scale, k_scale, v_scale, k_scales, v_scales, q_dtype, kv_dtype, partition_size,
                     workspace, workspace_bytes, stream);
}

int pkv_paged_attention_decode_append(void* out, const void* q, void* k_cache, void* v_cache, const void* key,
                                      const void* value, const int64_t* slot_mapping, const int32_t* block_tables,
                                      int max_blocks_per_seq, const int32_t* context_lens, const int32_t* seq_order,
                                      int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                                      int num_blocks, int max_context_len, float scale, float k_scale, float v_scale,
                                      const float* k_scales, const float* v_scales, int q_dtype, int kv_dtype,
                                      int partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && (!key || !value || !slot_mapping)) return PKV_ERR_NULL_POINTER;
  return decode_impl(out, q, k_cache, v_cache, num_seqs > 0 ? key : nullptr, value, slot_mapping, block_tables,
                     max_blocks_per_seq, context_lens, seq_order, num_seqs, num_heads, num_kv_heads, head_dim,
                     block_size, num_blocks, max_context_len, scale, k_scale, v_scale, k_scales, v_scales, q_dtype,
                     kv_dtype, partition_size, workspace, workspace_bytes, stream);
}

int pkv_paged_attention_decode_shared(void* out, const void* q, void* k_cache, void* v_cache, const void* key,
                                      const void* value, const int64_t* slot_mapping, const int32_t* block_tables,
                                      int max_blocks_per_seq, const int32_t* context_lens,
                                      const int32_t* group_offsets, const int32_t* group_members,
                                      const int32_t* group_shared_blocks, int num_groups, int max_group_size,
                                      int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                                      int num_blocks, int max_context_len, float scale, float k_scale, float v_scale,
                                      const float* k_scales, const float* v_scales, int q_dtype, int kv_dtype,
                                      void* stream) {
  if (num_seqs < 0 || num_groups < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      max_context_len < 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || max_group_size <= 0)
    return PKV_ERR_BAD_SIZE;
  if (num_heads % num_kv_heads != 0) return PKV_ERR_HEAD_GROUPING;
  const int group = num_heads / num_kv_heads;
  if ((long long)max_group_size * group > 16) return PKV_ERR_BAD_SIZE;   // one MFMA tile of columns
  if (!pkv::shared_supported(q_dtype, kv_dtype, head_dim, block_size)) return PKV_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return PKV_ERR_BAD_SIZE;
  const bool fp8 = kv_dtype == PKV_FP8_E4M3 || kv_dtype == PKV_FP8_E5M2;
  if (fp8 && !((k_scales || pkv::good_scale(k_scale)) && (v_scales || pkv::good_scale(v_scale)))) return PKV_ERR_SCALE;
  const long long wgs = (long long)num_groups * num_kv_heads;
  if (wgs > 2147483647LL) return PKV_ERR_BAD_SIZE;
  if (num_seqs == 0 || num_groups == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !group_offsets || !group_members ||
      !group_shared_blocks)
    return PKV_ERR_NULL_POINTER;
  if (!pkv::aligned16(out) || !pkv::aligned16(q) || !pkv::aligned16(k_cache) || !pkv::aligned16(v_cache))
    return PKV_ERR_UNSUPPORTED;
  if (key) {
    if (!value || !slot_mapping) return PKV_ERR_NULL_POINTER;
    if (!pkv::aligned16(key) || !pkv::aligned16(value)) return PKV_ERR_UNSUPPORTED;
  }
  pkv::AttnParams p{};
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = group;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.num_partitions = 1;
  const long long cap_table = (long long)max_blocks_per_seq * block_size;
  const long long cap = ((long long)max_context_len + block_size - 1) / block_size * block_size;
  const long long c = cap < cap_table ? cap : cap_table;
  p.ctx_cap = (int)(c < 2147483647LL ? c : 2147483647LL);
  p.new_k = key;
  p.new_v = value;
  p.slot_mapping = key ? slot_mapping : nullptr;
  p.enc_k_scale = k_scale;
  p.enc_v_scale = v_scale;
  p.k_scales = fp8 ? k_scales : nullptr;
  p.v_scales = fp8 ? v_scales : nullptr;
  p.qk_scale = scale * kLog2e * (fp8 && !k_scales ? k_scale : 1.f);
  p.v_scale = fp8 && !v_scales ? v_scale : 1.f;
  p.total_wgs = (uint32_t)wgs;
  p.xcd_chunk = (uint32_t)xcd_chunk_for(kSingle);                  // work ids are (group, kv head), head fastest
  p.head_run_units = head_run_units_for(kSingle, num_kv_heads);
  p.grp_off = group_offsets;
  p.grp_mem = group_members;
  p.grp_shared = group_shared_blocks;
  p.grp_max = max_group_size;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (pkv::debug_checks_on()) {
    pkv::DeviceChecks c(s);
    c.tables(block_tables, max_blocks_per_seq, context_lens, num_seqs, block_size, num_blocks, max_context_len);
    c.groups(group_offsets, group_members, group_shared_blocks, num_groups, max_group_size, block_tables,
             max_blocks_per_seq, context_lens, num_seqs, block_size, p.ctx_cap);
    if (fp8) c.scales(k_scales, v_scales, num_kv_heads);
    if (key)
      c.append_slots(slot_mapping, block_tables, max_blocks_per_seq, context_lens, num_seqs, block_size,
                     (long long)num_blocks * block_size);
    const int cst = c.finish();
    if (cst != PKV_OK) return cst;
  }
  (void)hipGetLastError();
  return pkv::launch_status(pkv::launch_attention_shared(p, q_dtype, kv_dtype, head_dim, key != nullptr, s));
}

int pkv_paged_prefill_attention(void* out, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                                const int32_t* query_start_loc, int num_seqs, int num_tokens, int num_heads,
                                int num_kv_heads,
                                int head_dim, int block_size, int num_blocks, int max_query_len,
                                int max_context_len, float scale, float k_scale, float v_scale,
                                const float* k_scales, const float* v_scales, int q_dtype, int kv_dtype,
                                void* stream) {
  if (num_seqs < 0 || num_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      max_query_len < 0 || max_context_len < 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
    return PKV_ERR_BAD_SIZE;
  if (num_heads % num_kv_heads != 0) return PKV_ERR_HEAD_GROUPING;
  if (!pkv::prefill_supported(q_dtype, kv_dtype, head_dim, block_size)) return PKV_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return PKV_ERR_BAD_SIZE;
  const bool fp8 = kv_dtype == PKV_FP8_E4M3 || kv_dtype == PKV_FP8_E5M2;
  if (fp8 && !((k_scales || pkv::good_scale(k_scale)) && (v_scales || pkv::good_scale(v_scale)))) return PKV_ERR_SCALE;
  const int bm = pkv::prefill_tile_rows();
  const long long tiles = ((long long)max_query_len + bm - 1) / bm;
  const long long wgs = (long long)num_seqs * num_heads * tiles;
  if (wgs > 2147483647LL) return PKV_ERR_BAD_SIZE;
  if (wgs == 0 || num_tokens == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc)
    return PKV_ERR_NULL_POINTER;
  if (!pkv::aligned16(out) || !pkv::aligned16(q) || !pkv::aligned16(k_cache) || !pkv::aligned16(v_cache))
    return PKV_ERR_UNSUPPORTED;
  pkv::PrefillParams p{};
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.query_start_loc = query_start_loc;
  p.num_seqs = num_seqs;
  p.num_tokens = num_tokens;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_heads / num_kv_heads;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.max_query_len = max_query_len;
  p.q_tiles = (int)tiles;
  const long long cap_table = (long long)max_blocks_per_seq * block_size;
  p.ctx_cap = (int)(max_context_len < cap_table ? max_context_len : cap_table);
  p.qk_scale = scale * kLog2e;
  p.k_scale = fp8 ? k_scale : 1.f;
  p.v_scale = fp8 ? v_scale : 1.f;
  p.k_scales = fp8 ? k_scales : nullptr;
  p.v_scales = fp8 ? v_scales : nullptr;
  p.longest_first = PKV_LONGEST_FIRST && num_seqs > 1 && num_seqs <= pkv::kMaxSliceSeqs;
  p.total_wgs = (uint32_t)wgs;
  // the query tiles and heads that read one kv head's K/V run on one XCD (shared L2)
  const char* e = getenv("PKV_PREFILL_XCD_CHUNK");
  long long chunk = (long long)tiles * p.group;
  if (e && *e) chunk = atoi(e);
  p.xcd_chunk = (uint32_t)(chunk < 0 ? 0 : (chunk > 4096 ? 4096 : chunk));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (pkv::debug_checks_on()) {
    pkv::DeviceChecks c(s);
    c.tables(block_tables, max_blocks_per_seq, context_lens, num_seqs, block_size, num_blocks, max_context_len);
    c.query_starts(query_start_loc, num_seqs, num_tokens, max_query_len);
    if (fp8) c.scales(k_scales, v_scales, num_kv_heads);
    const int cst = c.finish();
    if (cst != PKV_OK) return cst;
  }
  (void)hipGetLastError();
  return pkv::launch_status(pkv::launch_prefill(p, q_dtype, kv_dtype, head_dim, s));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Decode that allocates nothing: the split-context summaries go to a static
// device array instead of a caller workspace.
// ---------------------------------------------------------------------------
namespace {

// One copy per GPU, held from the library's first use on that GPU until the
// process ends.  In host code `scratch` names a host-side stand-in; kernels get
// the device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[PKV_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch, looked up once per device.
int static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PKV_ERR_LAUNCH;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return PKV_ERR_LAUNCH;
      g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, int max_blocks_per_seq,
                                       const int32_t* context_lens, const int32_t* seq_order, int num_seqs,
                                       int num_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                       int max_context_len, float scale, float k_scale, float v_scale,
                                       const float* k_scales, const float* v_scales, int q_dtype, int kv_dtype,
                                       int partition_size, void* stream) {
  Plan pl;
  const int st = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len, partition_size,
                           q_dtype, kv_dtype, &pl);
  if (st != PKV_OK) return st;
  if (pl.ws_bytes > PKV_STATIC_SCRATCH_BYTES) return PKV_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (pl.ws_bytes > 0 && num_seqs > 0) {
    const int e = static_scratch(&ws);
    if (e != PKV_OK) return e;
  }
  return decode_impl(out, q, k_cache, v_cache, nullptr, nullptr, nullptr, block_tables, max_blocks_per_seq,
                     context_lens, seq_order, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_context_len, scale, k_scale, v_scale, k_scales, v_scales, q_dtype, kv_dtype, partition_size,
                     ws, ws ? (size_t)PKV_STATIC_SCRATCH_BYTES : 0, stream);
}

}  // extern "C"
