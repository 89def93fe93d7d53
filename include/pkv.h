/*
 * pkv.h -- C ABI of the paged-KV decode library for AMD MI355X (gfx950).
 *
 * Six data-path calls and their helpers.  The library is stateless: the host
 * owns the block bookkeeping (which physical block holds which tokens,
 * reference counts, copy-on-write decisions); the library moves bytes and
 * attends.  Sources cited (page title, then section):
 *   [KVpag]      "KV cache paginado e batching contínuo para LLMs", "Como funciona"
 *   [PA/paging]  "PagedAttention" (Ultralytics glossary), "Cách phân trang hoạt động"
 *   [PA/sharing] same page, "Chia sẻ block giữa các chuỗi"
 *   [PA/related] same page, "Các kỹ thuật liên quan"
 *   [vLLM-rev]   "vLLM PagedAttention: uma revolução no throughput de inferência de LLMs"
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer argument is a DEVICE pointer (HIP device memory) unless noted.
 *   The caller allocates and owns every buffer, including the attention
 *   workspace.  The library never allocates, frees or synchronises.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *   call only enqueues work on it and returns; results are ready when the
 *   stream reaches that point.
 * - Pools (k_cache, v_cache): `[num_blocks][num_kv_heads][block_size][head_dim]`,
 *   row-major, element type `kv_dtype`.  One (block, kv head) tile is the
 *   contiguous `[block_size][head_dim]` block of [PA/paging]'s example.
 *   A flat slot is `block * block_size + offset`.
 * - Element types (`*_dtype`): PKV_F32, PKV_F16, PKV_BF16, PKV_FP8_E4M3 (OCP
 *   E4M3 "FN": bias 7, max +-448, no infinity, NaN = S.1111.111), PKV_FP8_E5M2
 *   (OCP E5M2: bias 15, max +-57344, S.11111.00 infinity, other S.11111.xx NaN).
 *   An 8-bit cache stores code * scale: one fp32 scale per pool (k_scale,
 *   v_scale), or one per kv head when the optional device arrays k_scales /
 *   v_scales ([num_kv_heads] fp32, positive finite; not checked on the host) are
 *   given -- then they replace the pool's scale.
 * - Return: PKV_OK (0) or a negative status (see pkv_status_string).  Every
 *   argument check runs on the host before anything is enqueued, so an error
 *   return means nothing was launched.  PKV_ERR_LAUNCH reports a HIP launch
 *   failure (the stream's earlier work is unaffected).
 * - Device-resident values (block ids, slots, context lengths) cannot be checked
 *   on the host.  They are preconditions; the kernels clamp or skip values that
 *   would address outside the buffers instead of faulting (each call says how),
 *   so a broken table gives wrong numbers, never an out-of-bounds access.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
#define PKV_F32 0
#define PKV_F16 1
#define PKV_BF16 2
#define PKV_FP8_E4M3 3
#define PKV_FP8_E5M2 4

/* status codes */
#define PKV_OK 0
#define PKV_ERR_NULL_POINTER (-1)   /* a required pointer is NULL                          */
#define PKV_ERR_BAD_SIZE (-2)       /* a size is negative / zero where it must be positive  */
#define PKV_ERR_HEAD_GROUPING (-3)  /* num_heads is not a multiple of num_kv_heads          */
#define PKV_ERR_UNSUPPORTED (-4)    /* head_dim / block_size / dtype combination not built  */
#define PKV_ERR_PARTITION (-5)      /* partition_size not a positive multiple of block_size */
#define PKV_ERR_WORKSPACE (-6)      /* workspace missing or smaller than required           */
#define PKV_ERR_LAUNCH (-7)         /* HIP reported a launch error                          */
#define PKV_ERR_SCALE (-8)          /* an FP8 scale is not a positive finite number         */
#define PKV_ERR_MEMORY_KIND (-9)    /* a buffer is neither device memory nor pinned host     */
                                    /* memory the device can address                         */
#define PKV_ERR_SCRATCH_LIMIT (-10) /* the call needs more than PKV_STATIC_SCRATCH_BYTES         */
#define PKV_ERR_PRECONDITION (-11)  /* debug checks: a device-resident value breaks the call's
                                       preconditions; nothing was launched (pkv_debug_report)  */

/* Size of the static device scratch of pkv_paged_attention_decode_noalloc (one copy per GPU). */
#define PKV_STATIC_SCRATCH_BYTES (48u << 20)

/* attention kernel families reported by pkv_attention_plan */
#define PKV_PATH_VECTOR 0  /* per-query-head vector kernel (wave shuffles, no MFMA)  */
#define PKV_PATH_MFMA 1    /* grouped-query kernel: one kv head's group on MFMA      */

/*
 * Debug checks of the device-resident values (pkv_set_debug_checks).
 *
 * The values a call reads from device memory -- block tables, context lengths,
 * slots, block-copy pairs, the host order, the shared decode's groups, the
 * prefill's query offsets -- cannot be checked on the host, and the kernels
 * take them on trust: a value out of place is clamped or skipped (never an
 * access outside the buffers) and gives wrong numbers.  With the checks on,
 * each entry point, after its host checks, runs check kernels over those values
 * on its stream, waits for them (the call then synchronises the stream), and
 * returns PKV_ERR_PRECONDITION without launching anything else when a value
 * breaks a rule below; pkv_debug_report then says which.  The rules restate
 * what the pages fix: a sequence's table lists its blocks in order and position
 * pos lives in block table[pos / bs] at offset pos % bs ("PagedAttention",
 * Ultralytics glossary, section "Cách phân trang hoạt động"); a block two
 * sequences share is copied to a fresh block before either writes into it
 * ("KV cache paginado e batching contínuo para LLMs", section "Como funciona").
 * Every value the kernels would clamp or skip counts as a violation here.
 * Violation kinds, each counted once per offending value:
 */
#define PKV_CHECK_CONTEXT_LEN 1    /* context_lens[s] < 0, > max_context_len, or needing more than
                                      max_blocks_per_seq blocks; index s                          */
#define PKV_CHECK_BLOCK_ID 2       /* block_tables[s][j] outside [0, num_blocks) for one of the first
                                      ceil(ctx_s / bs) entries; index s * max_blocks_per_seq + j  */
#define PKV_CHECK_SLOT 3           /* a slot >= num_blocks * block_size (negative slots are
                                      padding); index: the token                                   */
#define PKV_CHECK_DUPLICATE_SLOT 4 /* a slot equal to an earlier token's; index: the later token  */
#define PKV_CHECK_APPEND_SLOT 5    /* decode with append: slot_mapping[s] >= 0 is not the slot of
                                      position context_lens[s] - 1; index s                       */
#define PKV_CHECK_PAIR_ID 6        /* a copy / swap pair's src or dst outside its pool; index: pair */
#define PKV_CHECK_DUPLICATE_DST 7  /* a pair's dst equal to an earlier pair's; index: the later pair */
#define PKV_CHECK_DST_IS_SRC 8     /* copy_blocks: a pair's dst equal to some pair's src; index: pair */
#define PKV_CHECK_SEQ_ORDER 9      /* seq_order not a permutation of 0..num_seqs-1: an entry out of
                                      range or equal to an earlier one; index: the entry           */
#define PKV_CHECK_GROUP 10         /* shared decode: group_offsets[0] != 0, decreasing, past
                                      num_seqs, group_offsets[G] != num_seqs, a group larger than
                                      max_group_size, or a negative shared count; index: group     */
#define PKV_CHECK_GROUP_MEMBER 11  /* shared decode: a member outside [0, num_seqs) or listed twice;
                                      index: position in group_members                             */
#define PKV_CHECK_SHARED_BLOCK 12  /* shared decode: a member's table differs from the group's first
                                      member on a block read as shared; index s * max_blocks_per_seq + j */
#define PKV_CHECK_QUERY_START 13   /* prefill: query_start_loc[0] != 0, decreasing, outside
                                      [0, num_tokens], [num_seqs] != num_tokens, or a chunk longer
                                      than max_query_len; index: the entry                         */
#define PKV_CHECK_SCALE 14         /* 8-bit cache: a per-kv-head scale (k_scales / v_scales) that is
                                      not a positive finite number; index h for k_scales[h],
                                      num_kv_heads + h for v_scales[h]                             */

/*
 * pkv_set_debug_checks -- turn the debug checks on (mode 1), off (0), or leave
 * them to the PKV_DEBUG environment variable (-1, the default: on when it is set
 * and not "0", read at each call).  Process-wide; returns the previous mode.
 * Host-only.  With the checks on, calls serialise on one library-wide lock
 * while their checks run, and every call waits for its stream, so they do not
 * belong under HIP graph capture; results are unchanged.
 */
int pkv_set_debug_checks(int mode);

/*
 * pkv_debug_report -- the debug checks of the calling thread's most recent
 * checked call: the number of violations (0 if it passed or no call was
 * checked), and the kind (PKV_CHECK_*) and index of the first one in (kind,
 * index) order (0 and -1 when there is none).  Any pointer may be NULL.
 * Host-only; returns PKV_OK.
 */
int pkv_debug_report(int64_t* violations, int* kind, int64_t* index);

/*
 * K/V load policy of the decode calls (pkv_set_kv_load_policy).
 *
 * PKV_KV_LOADS_STREAM (the default): the K/V tiles are loaded with the
 *   non-temporal cache policy.  Right when a launch reads each block once --
 *   distinct contexts, or forks read through pkv_paged_attention_decode_shared --
 *   since the tiles then pass through the caches without displacing anything.
 * PKV_KV_LOADS_CACHED: the default cache policy.  Right when several sequences
 *   of one launch share blocks and are read by the plain decode ("KV cache
 *   paginado e batching contínuo para LLMs", section "Como funciona": forks
 *   share their prompt's blocks): the later readers of a shared block then find
 *   it in L2 or the Infinity Cache instead of HBM.
 * The policy changes only where the bytes come from, never a result.
 */
#define PKV_KV_LOADS_STREAM 0
#define PKV_KV_LOADS_CACHED 1

/*
 * pkv_set_kv_load_policy -- set the K/V load policy (PKV_KV_LOADS_*) of the
 * calling thread's later pkv_paged_attention_decode, ..._append and ..._noalloc
 * calls (pkv_paged_attention_decode_shared always streams: it reads each block
 * once per group).  Per host thread, PKV_KV_LOADS_STREAM until set.  Returns
 * the previous policy, or PKV_ERR_BAD_SIZE (policy unchanged) for any other
 * value.  Host-only.
 */
int pkv_set_kv_load_policy(int policy);

/* Human-readable text of a status code (static string, never NULL). */
const char* pkv_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int pkv_version(void);

/*
 * pkv_attention_plan -- how pkv_paged_attention_decode would run these shapes.
 *
 * Host-only; enqueues nothing.  Writes the kernel family (PKV_PATH_*), the
 * partition size in tokens and the number of partitions per sequence
 * (1 = single pass, no reduce kernel) through the three host pointers (any may
 * be NULL); balanced slices report partition size 0 and the number of slices.
 * `partition_size` 0 asks for the library's automatic choice.
 * Returns the same status pkv_paged_attention_decode would return for these
 * shapes (pointers aside).
 */
int pkv_attention_plan(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                       int block_size, int max_context_len, int partition_size,
                       int q_dtype, int kv_dtype,
                       int* path, int* partition_tokens, int* num_partitions);

/*
 * pkv_attention_workspace_bytes -- device workspace pkv_paged_attention_decode
 * needs for these shapes: the fp32 per-partition / per-slice summaries (running
 * max, exp-sum and unnormalised output vector) of a split context, plus the
 * block prefix of the sequences for balanced slices.  0 for a one-pass launch
 * and for invalid shapes.
 */
size_t pkv_attention_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                     int block_size, int max_context_len, int partition_size,
                                     int q_dtype, int kv_dtype);

/*
 * pkv_paged_attention_decode -- attention of each sequence's one new query token
 * over its paged KV cache ([PA/paging]: the kernel walks the request's block
 * table and gathers keys and values block by block; [KVpag]: decode consumes
 * the cache of every token seen so far).
 *
 * For every sequence s and query head h, with G = num_heads / num_kv_heads and
 * kv head g = h / G ([PA/related]: grouped-query heads share K/V heads):
 *   K_t = k_cache[block_tables[s][t / bs]][g][t % bs][:]   (V likewise), t < ctx_s
 *   logit_t = scale * <q[s][h][:], K_t>      (K_t, V_t times k_scale / v_scale for FP8)
 *   out[s][h][:] = sum_t softmax(logit)_t * V_t
 * computed in fp32 with an online (running max / running sum) softmax, so the
 * score row is never written to memory ([PA/related], FlashAttention-style).
 * ctx_s = context_lens[s] counts every cached token including the new one; a
 * sequence with ctx_s == 0 gets a zero output row.
 *
 * out          [num_seqs][num_heads][head_dim], q_dtype (fp32/f16/bf16); written, must
 *              not alias any input.  Rounded to nearest even from fp32.
 * q            [num_seqs][num_heads][head_dim], q_dtype.
 * k_cache, v_cache  pools as above, kv_dtype.  With an 8-bit kv_dtype the values
 *              are code * k_scale (resp. v_scale), or code * k_scales[g] with the
 *              per-head arrays; scales are ignored for 16/32-bit caches.
 * block_tables [num_seqs][max_blocks_per_seq] int32; entries past ceil(ctx/bs) are never read.
 * context_lens [num_seqs] int32.
 * seq_order    optional [num_seqs] int32 device array: the sequences longest
 *              context first (a permutation of 0..num_seqs-1).  It only decides
 *              which sequences start first in a one-pass launch -- any
 *              permutation gives the same results; the host that builds the
 *              block tables knows the lengths and can sort them for free.  NULL:
 *              every workgroup derives the order itself from context_lens.
 *              Entries are clamped to [0, num_seqs); a non-permutation leaves
 *              some output rows unwritten.
 * num_blocks   number of blocks in each pool.  A table entry outside
 *              [0, num_blocks) makes the kernel skip that block's tokens.
 * max_context_len  host-side upper bound of context_lens (sizes the partition grid).
 *              Tokens past min(ctx_s, max_context_len rounded up to a partition,
 *              max_blocks_per_seq * block_size) are ignored.
 * partition_size   tokens per split-context partition (multiple of block_size),
 *              or 0 for the automatic choice.  With partitions, each (sequence,
 *              head, partition) of a context longer than one partition writes an
 *              fp32 summary to `workspace` and a second kernel merges them:
 *              M = max_p m_p; out = sum_p e^(m_p - M) o_p / sum_p e^(m_p - M) l_p.
 *              The automatic choice is one pass when there are enough (sequence,
 *              head) units to fill the GPU (sequences dispatched longest first),
 *              else balanced
 *              slices: every workgroup gets the same number of blocks, contexts
 *              crossing a slice boundary are merged by the second kernel.
 * workspace    device buffer of at least pkv_attention_workspace_bytes(...) bytes
 *              (may be NULL when that is 0).  Contents on entry are ignored.
 * Supported: head_dim 64/128/256; block_size 8/16/32 (16 for the MFMA family);
 *   (q, kv) dtypes (f32,f32), (f16,f16), (bf16,bf16), and f16 or bf16 q over
 *   either 8-bit cache.
 *   Grouped heads (2 <= G <= 16, head_dim 128 or 256, block_size 16) with
 *   16-bit q over a cache of q's type or either 8-bit format run on the matrix
 *   cores; everything else on the vector family.
 * The K/V loads follow the calling thread's load policy (pkv_set_kv_load_policy).
 */
int pkv_paged_attention_decode(void* out, const void* q,
                               const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* context_lens, const int32_t* seq_order,
                               int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                               int block_size, int num_blocks, int max_context_len,
                               float scale, float k_scale, float v_scale,
                               const float* k_scales, const float* v_scales,
                               int q_dtype, int kv_dtype, int partition_size,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_paged_attention_decode_noalloc -- pkv_paged_attention_decode for callers
 * that cannot allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.
 *
 * Same arguments, results and launches as pkv_paged_attention_decode without
 * `workspace` / `workspace_bytes`: when the plan splits contexts, the fp32
 * summaries go to a static device array of PKV_STATIC_SCRATCH_BYTES (48 MiB)
 * inside the library instead.  Each GPU the library runs on holds its own copy
 * from the first use until the process ends; its device address is looked up
 * once per device, on the first call with that device current.  The call
 * itself allocates nothing (no hipMalloc, no allocating library routine).
 *
 * A call whose plan needs more than PKV_STATIC_SCRATCH_BYTES
 * (pkv_attention_workspace_bytes of the same shapes) returns
 * PKV_ERR_SCRATCH_LIMIT and launches nothing.  PKV_ERR_LAUNCH also reports a
 * failed address lookup.  Scratch contents on entry are ignored (nothing needs
 * clearing).  Every call on one GPU shares that GPU's scratch: two calls whose
 * kernels overlap on one GPU (different streams, no ordering between them)
 * race on it and may give wrong outputs; calls on one stream are ordered and
 * safe.
 */
int pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, int max_blocks_per_seq,
                                       const int32_t* context_lens, const int32_t* seq_order,
                                       int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                       int block_size, int num_blocks, int max_context_len,
                                       float scale, float k_scale, float v_scale,
                                       const float* k_scales, const float* v_scales,
                                       int q_dtype, int kv_dtype, int partition_size, void* stream);

/*
 * pkv_paged_attention_decode_append -- one decode step in one launch: each
 * sequence's new token is written into the pool and then attended over, with
 * the new token included ([KVpag]: decode produces one token at a time and
 * attends over the cache of every token seen so far, its own included).
 *
 * Same result as pkv_reshape_and_cache(key, value, k_cache, v_cache,
 * slot_mapping, num_tokens = num_seqs, ...) followed by
 * pkv_paged_attention_decode(...) with the same arguments, without the second
 * launch: for each sequence s the workgroup that reads s's last block first
 * writes row s of key / value (each [num_seqs][num_kv_heads][head_dim], q_dtype;
 * bit copy or the 8-bit encode of pkv_reshape_and_cache) into slot
 * slot_mapping[s], then attends.
 * Preconditions: slot_mapping[s] is the slot of position context_lens[s] - 1
 * of sequence s (the host's block manager returns exactly that), and no two
 * sequences share it.  Slots < 0 or past the pool are skipped; a sequence with
 * context 0 writes nothing.  k_cache / v_cache are written, so they are not const.
 */
int pkv_paged_attention_decode_append(void* out, const void* q, void* k_cache, void* v_cache,
                                      const void* key, const void* value, const int64_t* slot_mapping,
                                      const int32_t* block_tables, int max_blocks_per_seq,
                                      const int32_t* context_lens, const int32_t* seq_order,
                                      int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                      int block_size, int num_blocks, int max_context_len,
                                      float scale, float k_scale, float v_scale,
                                      const float* k_scales, const float* v_scales,
                                      int q_dtype, int kv_dtype, int partition_size,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_paged_attention_decode_shared -- the decode of pkv_paged_attention_decode
 * (or, with key != NULL, of pkv_paged_attention_decode_append) for groups of
 * sequences whose block tables start with the same physical blocks, as the
 * samples forked from one prompt do ([KVpag] "Como funciona": forks share
 * blocks through reference counts; [PA/sharing] "Chia sẻ block giữa các
 * chuỗi": parallel samples share the prompt's blocks).  The outputs are the
 * same attention (up to rounding order); a shared block is read once for all
 * the members of its group instead of once per member.
 *
 * Groups: group g's members are group_members[group_offsets[g] ..
 * group_offsets[g+1]) (device int32 arrays; group_offsets has num_groups + 1
 * entries, each group at most max_group_size members).  The first
 * group_shared_blocks[g] entries of every member's table must name the same
 * physical blocks; the kernel reads them through the first member's table.
 * Every sequence must belong to exactly one group (a sequence sharing nothing
 * is a group of one, with 0 shared blocks); a sequence in no group gets no
 * output row, one in two groups an unspecified one.  The kernel lowers the
 * shared count to keep it below every member's newest token: shared blocks are
 * always full, and a member's last block is always read as its own.  Out-of-
 * range offsets and members are clamped or skipped.
 *
 * One workgroup per (group, kv head); the group's query rows for that kv head
 * are the columns of the matrix-core tile, so max_group_size * G <= 16
 * (G = num_heads / num_kv_heads, 1 for multi-head attention).
 * Other arguments as pkv_paged_attention_decode_append (key, value,
 * slot_mapping may all be NULL for a plain decode; k_cache / v_cache are
 * written only when key is given).  No workspace, no split context: a group's
 * work stays in its workgroups.
 * Supported: f16 or bf16 q over a cache of q's type or either 8-bit format,
 *   head_dim 128 or 256, block_size 16.
 */
int pkv_paged_attention_decode_shared(void* out, const void* q, void* k_cache, void* v_cache,
                                      const void* key, const void* value, const int64_t* slot_mapping,
                                      const int32_t* block_tables, int max_blocks_per_seq,
                                      const int32_t* context_lens,
                                      const int32_t* group_offsets, const int32_t* group_members,
                                      const int32_t* group_shared_blocks, int num_groups,
                                      int max_group_size,
                                      int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                      int block_size, int num_blocks, int max_context_len,
                                      float scale, float k_scale, float v_scale,
                                      const float* k_scales, const float* v_scales,
                                      int q_dtype, int kv_dtype, void* stream);

/*
 * pkv_reshape_and_cache -- write each new token's key and value into the pool
 * slot the host chose for it ([PA/paging] example: the token at position pos
 * goes to block table[pos / bs], offset pos % bs).
 *
 * For token i with sigma = slot_mapping[i] >= 0, for every kv head h:
 *   k_cache[sigma / bs][h][sigma % bs][:] = enc(key[i][h][:])   (value likewise)
 * enc is a bit copy when src_dtype == kv_dtype, and for an 8-bit cache the code
 * of nearest(clamp(fp32(x) / scale, -max, max)) with IEEE fp32 division, ties to
 * even mantissa, NaN -> 0x7F | sign (max 448 for E4M3, 57344 for E5M2; the scale
 * is the pool's, or k_scales[h] / v_scales[h] for kv head h).  sigma < 0
 * (padding) and sigma >= num_blocks * block_size are skipped.
 *
 * key, value   [num_tokens][num_kv_heads][head_dim], src_dtype (f32/f16/bf16).
 * slot_mapping [num_tokens] int64.  Slots must be distinct within one call
 *              (two tokens to one slot leave either value).
 * k_scale, v_scale  8-bit encode scales (positive, finite); ignored otherwise, and
 *              replaced by k_scales / v_scales (device, [num_kv_heads]) when given.
 * Supported: src_dtype == kv_dtype, or src f32/f16/bf16 -> an 8-bit kv_dtype;
 *   head_dim a multiple of 16 up to 1024; any block_size >= 1.
 * num_tokens == 0 is a no-op returning PKV_OK.
 */
int pkv_reshape_and_cache(const void* key, const void* value,
                          void* k_cache, void* v_cache, const int64_t* slot_mapping,
                          int num_tokens, int num_kv_heads, int head_dim, int block_size,
                          int num_blocks, int src_dtype, int kv_dtype,
                          float k_scale, float v_scale, const float* k_scales, const float* v_scales,
                          void* stream);

/*
 * pkv_copy_blocks -- block-level copy-on-write ([KVpag]: before writing into a
 * block still shared by other sequences, take a new block and copy the old
 * one; [PA/sharing]).  The host decides the pairs; this call moves the bytes.
 *
 * For each pair p: k_cache[dst] = k_cache[src] and v_cache[dst] = v_cache[src],
 * whole blocks (every kv head, every slot, raw bytes).
 * block_mapping [num_pairs][2] int64 (src, dst).  Destination ids must be
 *              distinct and disjoint from all source ids (then pair order does
 *              not matter).  Pairs with an id outside [0, num_blocks) are skipped.
 * num_pairs == 0 is a no-op returning PKV_OK.
 */
int pkv_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping, int num_pairs,
                    int num_kv_heads, int head_dim, int block_size, int num_blocks,
                    int kv_dtype, void* stream);

/*
 * pkv_paged_prefill_attention -- chunked prefill over the paged cache
 * ([vLLM-rev] feature list: a long prompt's prefill is split into chunks;
 * [PA/paging]: keys and values are gathered block by block through the table).
 *
 * Sequence s contributes n_s = query_start_loc[s+1] - query_start_loc[s] query
 * tokens, rows query_start_loc[s] .. of q and out.  They are the sequence's
 * last n_s positions: ctx_s = context_lens[s] counts every cached token
 * including the chunk, whose K/V the caller wrote into the pool first
 * (pkv_reshape_and_cache).  Query i sits at position p = ctx_s - n_s + i and
 * attends causally to positions 0..p; for each query head h (kv head g = h / G):
 *   out[row][h][:] = sum_{t<=p} softmax_t(scale * <q[row][h], K_t>) V_t
 * in fp32 with an online softmax; the probabilities enter the PV product
 * rounded to the q dtype.  A row with p < 0 (more queries than context) is zero.
 * Over an 8-bit cache ([PA/related] FP8 cache) K_t and V_t are the stored
 * values, code * k_scale (resp. v_scale) or code * k_scales[g] with the
 * per-head arrays, as for pkv_paged_attention_decode.
 *
 * out, q       [num_tokens][num_heads][head_dim], q_dtype.
 * query_start_loc  [num_seqs + 1] int32, non-decreasing, from 0 to num_tokens;
 *              entries are clamped to [0, num_tokens] (a broken array gives wrong
 *              rows, never an access outside q / out).
 * k_cache, v_cache, block_tables, num_blocks  as for pkv_paged_attention_decode
 *              (blocks the table maps outside [0, num_blocks) are skipped).
 * context_lens [num_seqs] int32.
 * max_query_len    host bound on every n_s (sizes the grid); rows past it are
 *              not written.  max_context_len: host bound on context_lens (larger
 *              values are clamped, giving wrong positions but no stray access).
 * k_scale, v_scale, k_scales, v_scales  the 8-bit cache's scales, as for
 *              pkv_paged_attention_decode (checked the same way, PKV_ERR_SCALE);
 *              ignored for a 16-bit cache.
 * Supported: q_dtype in {PKV_F16, PKV_BF16} over a cache of q's type or either
 *   8-bit format, head_dim 64 or 128, block_size 16.  Needs no workspace.
 *   max_query_len, num_seqs or num_tokens == 0 is a no-op returning PKV_OK.
 */
int pkv_paged_prefill_attention(void* out, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, int max_blocks_per_seq,
                                const int32_t* context_lens, const int32_t* query_start_loc,
                                int num_seqs, int num_tokens, int num_heads, int num_kv_heads, int head_dim,
                                int block_size, int num_blocks, int max_query_len, int max_context_len,
                                float scale, float k_scale, float v_scale,
                                const float* k_scales, const float* v_scales,
                                int q_dtype, int kv_dtype, void* stream);

/*
 * pkv_swap_blocks -- whole-block copies between two pools, for preemption by
 * swapping ([KVpag]: when physical blocks run out, the most recent requests are
 * preempted, all or nothing, and their blocks are recovered by swapping them to
 * CPU memory and back).  The host decides the pairs (which GPU block goes to
 * which host block, and back); this call moves the bytes in one launch.
 *
 * For each pair p = (src, dst):
 *   dst_k[dst] = src_k[src] and dst_v[dst] = src_v[src]
 * whole blocks (every kv head, every slot, raw bytes), the two pools having the
 * same block shape [num_kv_heads][block_size][head_dim] of kv_dtype.
 *
 * src_k, src_v   source pools, [src_num_blocks] blocks each.
 * dst_k, dst_v   destination pools, [dst_num_blocks] blocks each; must not
 *                overlap the source pools.
 * Each pool, and block_mapping, is either device memory or pinned host memory
 * (hipHostMalloc, e.g. torch's pin_memory=True) that the device addresses over
 * the host link; the library looks each pointer up with the HIP runtime and
 * returns PKV_ERR_MEMORY_KIND, launching nothing, for any other memory
 * (pageable host memory).  A swap-out is device -> host, a swap-in host -> device.
 * block_mapping  [num_pairs][2] int64 (src, dst).  Destination ids must be
 *                distinct.  Pairs with src outside [0, src_num_blocks) or dst
 *                outside [0, dst_num_blocks) are skipped.
 * num_pairs == 0 is a no-op returning PKV_OK.
 * The host must not touch a host pool until the stream has passed this call.
 */
int pkv_swap_blocks(const void* src_k, const void* src_v, int src_num_blocks,
                    void* dst_k, void* dst_v, int dst_num_blocks,
                    const int64_t* block_mapping, int num_pairs,
                    int num_kv_heads, int head_dim, int block_size, int kv_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
