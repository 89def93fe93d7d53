/*
 * pkv_probe.h -- HBM read-rate probes of the benchmark (libpkv_probe.so).
 *
 * Not part of the paged-KV path.  The decode kernels are bound by HBM
 * bandwidth (decode reads every cached key and value once per step: "vLLM
 * PagedAttention: uma revolução no throughput de inferência de LLMs", feature
 * list, prefill compute-bound vs decode bandwidth-bound), and the 8 TB/s spec
 * figure is not what a read-only kernel reaches on a given machine.  These two
 * read-only kernels measure that ceiling in the same process as the decode
 * step: one streams a buffer, the other reads tiles of the size the decode
 * kernels read (one (block, kv head) tile of the pool) at pseudo-random tile
 * indices, as a block-table walk does.
 *
 * Conventions: `buf` and `sink` are device pointers the caller allocated;
 * `stream` is a hipStream_t passed as void* (NULL = the null stream).  Each call
 * only enqueues one kernel and returns 0, or a negative status (the codes of
 * pkv.h: -1 null pointer, -2 bad size, -7 launch error) with nothing launched.
 * The kernels only read `buf`; `sink` receives at most one word (written only
 * when the XOR of everything read equals `salt`, which keeps the loads alive
 * without write traffic).
 */
#ifndef PKV_PROBE_H_
#define PKV_PROBE_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pkv_probe_stream_read -- read `bytes` bytes of `buf` once: each wave of
 * `num_workgroups` workgroups of 4 waves reads whole 8 KiB chunks (eight 1 KiB
 * loads of consecutive bytes in flight), wave w taking chunks w, w + W, ...
 * (W waves), so the grid sweeps the buffer front to back.  `bytes` a positive
 * multiple of 16, `buf` 16-byte aligned.  `nontemporal` != 0: the loads carry
 * the non-temporal cache policy, as the decode kernels' K/V loads do; 0: plain
 * loads, which displace what the caches hold (a cache flush needs them).
 */
int pkv_probe_stream_read(const void* buf, size_t bytes, int num_workgroups, unsigned salt, unsigned* sink,
                          int nontemporal, void* stream);

/*
 * pkv_probe_tile_read -- each wave of `num_workgroups` workgroups of 4 waves
 * reads `tiles_per_wave` whole tiles of `tile_bytes` bytes (1024, 2048, 4096 or
 * 8192) of the T = bytes / tile_bytes tiles of `buf`, two tiles in flight,
 * 16-byte loads.  Read number n (n = wave * tiles_per_wave + i) takes tile
 * (n * P + salt) mod T for a fixed prime P that divides no such T: a
 * scattered order that is a bijection, so a launch of at most T reads reads
 * every tile at most once (none is served by the caches from an earlier read
 * of the same launch; beyond T reads the order repeats).  `nontemporal` as for
 * pkv_probe_stream_read.
 */
int pkv_probe_tile_read(const void* buf, size_t bytes, int tile_bytes, int num_workgroups, int tiles_per_wave,
                        unsigned salt, unsigned* sink, int nontemporal, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H_ */
