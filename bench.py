"""Benchmark of one paged decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama13b_f16]

With a prefill workload (prefill_llama13b_f16, prefill_gqa_bf16, and
prefill_gqa_fp8 over an E4M3 cache) the step is
reshape_and_cache of the chunks' K/V followed by paged_prefill_attention, and
the roofline is the dense MFMA peak instead of HBM.  prefix_cache_llama13b_f16
times a prefill step of requests sharing a system prompt with the host prefix
cache off and on (value = the speedup).  shared_prefix_fp8 times the next
decode step of parallel samples that share their prompts' blocks, over fp8
(E4M3) pools: the copy-on-write copies the step needs plus the decode with
append, KV bytes counted logical (per sample) and unique (per physical block).
stream_probe measures what HBM delivers to plain read-only kernels here.

A step is one pass of the hot path over one synthetic decode batch, inputs
resident in HBM: every sequence's new key/value goes into the slot the block
manager gave it and each sequence attends over its paged context, the new
token included -- one paged_attention_decode_append launch (the split-context
reduce included when the plan uses one).  The block manager's host
bookkeeping (tables, slots, the longest-first sequence order) is built before
the timed region.

Timing: K steps, each bracketed by HIP events on the stream the kernels run
on.  Before every timed step 512 MiB are written and another 512 MiB read,
outside the events, so L2 and the 256 MB Infinity Cache hold nothing of the
step's inputs and no dirty lines of the flush itself (the headline); the same
steps back to back are reported beside it.  Warm-up runs at least --warmup
steps and at least 50 ms of GPU work (the first launches after the host-bound
set-up run at low clocks); the JSON gives the count.

Reported beside the step under "components" (not part of it): the same step
as two launches (reshape_and_cache, then paged_attention_decode); copy_blocks
on copy-on-write pairs shaped like the shared-prefix workload; swap_blocks of
the 16 most recent sequences to a pinned host pool and back; for a workload
that states its partition size (long-context split-K), the same step under the
library's automatic plan; the HBM read probes (a streaming read and random
2/4/8 KiB tile reads, libpkv_probe.so); and, with the default workload, the
GQA bf16 step (flushed and back to back, its roofline fraction and oracle
parity), so one default run covers both decode shapes the 70 % target names.

Prints one JSON line:
* value      algorithmic KV bytes read per step / step time (GB/s);
* roofline   the step's launch against MI355X's 8 TB/s HBM; achieved =
             algorithmic bytes per call (K/V of every context token, q, out,
             table entries, lengths, the new tokens read and written) / mean call
             time;
* pct_of_measured_stream_bw  achieved / the streaming-read probe's rate;
* slot_utilisation  sum(ctx) / (block_size * blocks held);
* cpu_baseline  the fp64 CPU oracle on a bounded sample of the same workload;
  the GPU rows it recomputed give max_abs_err / max_rel_err.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_traffic.json")
# sources of the kernels each kind of workload times (a change to any of them
# retires that kind's recorded HBM traffic)
KERNEL_SOURCES = {
    "decode": ["attn_vector.h", "attn_vector.hip", "attn_mfma.h", "attn_mfma.hip", "attn_append.hip",
               "attn_reduce.hip", "attn_shared.hip", "pkv_device.h", "pkv_api.hip"],
    "prefill": ["prefill_mfma.hip", "pkv_device.h", "pkv_api.hip"],
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama13b_f16")
    ap.add_argument("--partition", type=int, default=None, help="override the workload's partition size")
    ap.add_argument("--group-size", type=int, default=0,
                    help="shared-prefix workload: samples per shared-block group (0: as many as one tile holds)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-components", action="store_true",
                    help="default workload: skip the GQA step timed beside the headline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="bound on the oracle sample's CPU time")
    ap.add_argument("--calibrate-copy", type=int, default=0,
                    help="also run one copy_blocks of this many blocks (HBM counter calibration); such a run "
                         "skips the automatic-plan comparison, so its counters hold only the timed step")
    return ap.parse_args()


WARMUP_MIN_S = 0.05


def warm_up(fn, steps):
    """Run ``fn`` at least ``steps`` times and for at least WARMUP_MIN_S of GPU time.

    After the host-bound set-up (inputs, block tables) the GPU needs a few
    milliseconds of work to return to full clocks; a fixed count of short steps
    does not always cover that.  Returns the number of warm-up steps run.
    """
    import torch
    n, t0 = 0, time.perf_counter()
    while n < steps or time.perf_counter() - t0 < WARMUP_MIN_S:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


FLUSH_BYTES = 1 << 30          # 512 MiB written, then another 512 MiB read, between flushed steps


class Flusher:
    """Clears L2 and the 256 MB Infinity Cache between timed steps, outside the timed events.

    Writes 512 MiB (torch fill) and then reads another 512 MiB (the probe's
    streaming read, plain loads): the write evicts whatever the caches held, and
    the read leaves them holding clean lines of an unrelated buffer, so no
    write-back of the flush's own dirty lines lands inside the next timed step.
    (A non-temporal read would not displace those dirty lines: their write-back
    then lands in the timed step, which cost the decodes 2-8 %.)
    """

    def __init__(self, stream):
        import torch
        from paged_kv_cache_259_amd import probe
        self.buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        self.sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        self.half = FLUSH_BYTES // 2
        self.stream, self.probe, self.n = stream, probe, 0

    def __call__(self):
        self.n += 1
        self.buf[: self.half].fill_(self.n % 251)
        self.probe.stream_read(self.buf[self.half:], self.half, 2048, self.sink, nontemporal=False, stream=self.stream)


def timed_steps(fn, K, stream, flush=None):
    """Per-step times (ms) of K calls of fn, each bracketed by HIP events on ``stream``; with ``flush``,
    the caches are cleared before every step, outside the events."""
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        if flush is not None:
            flush()
        ev[i][0].record(stream)
        fn()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def hbm_probe(stream, reps=10, flush=None):
    """What HBM delivers to read-only kernels on this machine: a streaming read of 1 GiB (best of three grid
    sizes) and reads of scattered 2/4/8 KiB tiles (0.75 GB per launch, no tile read twice in a launch), GB/s
    from HIP events around each launch; with ``flush`` (the decode steps' cache flush) the caches are cleared
    before every launch, as before every timed decode step."""
    import torch
    from paged_kv_cache_259_amd import probe
    buf = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def rate(fn, nbytes):
        for _ in range(3):
            fn()
        ms = timed_steps(fn, reps, stream, flush)
        return nbytes / (float(np.mean(ms)) * 1e-3) / 1e9

    stream_rates = {}
    for wgs in (1024, 2048, 4096):
        stream_rates[wgs] = rate(lambda: probe.stream_read(buf, buf.numel(), wgs, sink, stream=stream), buf.numel())
    tiles, tiles_plain = {}, {}
    wgs = 2048
    salt = [0]

    def tile_launch(tb, per_wave, nt=True):
        salt[0] += 1                                    # another scattered order on every launch
        probe.tile_read(buf, tb, wgs, per_wave, sink, salt=salt[0] * 7919, nontemporal=nt, stream=stream)

    for tb in (2048, 4096, 8192):
        per_wave = (768 << 20) // (wgs * 4 * tb)
        tiles[tb] = rate(lambda: tile_launch(tb, per_wave), wgs * 4 * per_wave * tb)
        tiles_plain[tb] = rate(lambda: tile_launch(tb, per_wave, False), wgs * 4 * per_wave * tb)
    best = max(stream_rates, key=stream_rates.get)
    plain = rate(lambda: probe.stream_read(buf, buf.numel(), best, sink, nontemporal=False, stream=stream), buf.numel())
    del buf
    return {"stream_read_gbps": round(stream_rates[best], 1), "stream_read_workgroups": best,
            "stream_read_gbps_by_grid": {str(k): round(v, 1) for k, v in stream_rates.items()},
            "tile_read_gbps": {f"{k // 1024}KiB": round(v, 1) for k, v in tiles.items()},
            "plain_loads": {"stream_read_gbps": round(plain, 1),
                            "tile_read_gbps": {f"{k // 1024}KiB": round(v, 1) for k, v in tiles_plain.items()}},
            "flushed": flush is not None,
            "probe": "libpkv_probe.so: 16-byte non-temporal loads (plain loads under plain_loads), 1 GiB buffer, "
                     "mean of per-launch HIP-event times"
                     + (", caches flushed before each launch" if flush is not None else "")
                     + "; tiles in a scattered order that reads no tile twice per launch, two per wave in "
                     "flight, 2048 workgroups of 4 waves"}


def slot_utilisation(ctx, bs):
    """Share of the allocated slots holding a token: sum(ctx) / (bs * sum of blocks)."""
    ctx = np.asarray(ctx, np.int64)
    blocks = int(np.sum((ctx + bs - 1) // bs))
    return round(float(np.sum(ctx)) / (bs * blocks), 5) if blocks else None


def parity_of(got_rows, ref_rows, atol, rtol):
    """max-abs / max-rel error of GPU rows against the oracle's, and the worst ratio to the tolerance.

    max_rel_err is taken over elements with |ref| >= 0.01 (smaller references make the ratio meaningless).
    """
    got = np.asarray(got_rows, np.float64)
    ref = np.asarray(ref_rows, np.float64)
    err = np.abs(got - ref)
    big = np.abs(ref) >= 1e-2
    return {"max_abs_err": float(err.max()) if err.size else 0.0,
            "max_rel_err": float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0,
            "tol_ratio": float((err / (atol + rtol * np.abs(ref))).max()) if err.size else 0.0,
            "tolerance": f"{atol:g} + {rtol:g} |ref| per element",
            "elements": int(err.size)}


TOLERANCE = {"f32": (1e-5, 1e-5)}    # 16-bit and 8-bit caches: (2e-3, 1e-2)


def kernel_kind(workload):
    return "prefill" if workload.startswith("prefill") else "decode"


def kernel_source_hash(workload):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel_kind(workload)]:
        with open(os.path.join(ROOT, "paged_kv_cache_259_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per attention call from committed counter runs, if taken on the current kernels."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get(workload)
    if not entry or entry.get("kernel_source_hash") != kernel_source_hash(workload):
        return None
    return entry.get("bytes_per_call")


def algorithmic_bytes(w, ctx, elt_q, elt_kv):
    """KV bytes each sequence's context reads, plus q, out, table entries and context lengths."""
    kv = int(np.sum(ctx)) * w.num_kv_heads * w.head_dim * 2 * elt_kv
    qo = 2 * w.num_seqs * w.num_heads * w.head_dim * elt_q
    tables = int(np.sum(-(-ctx // w.block_size))) * 4 + 4 * w.num_seqs
    return kv, kv + qo + tables


class _BlockSubset:
    """float64 host copy of some pool blocks, read as pool[block, kv_head] by the oracle.

    ``decode`` turns an 8-bit pool's codes into values (the oracle's decoder
    times the scale); other pools are widened to float64.
    """

    def __init__(self, pool, blocks, decode=None):
        import torch
        ids = sorted(set(int(b) for b in blocks))
        rows = pool.index_select(0, torch.tensor(ids, dtype=torch.int64, device=pool.device))
        host = decode(rows.cpu().numpy()) if decode else rows.cpu().to(torch.float64).numpy()
        self._rows = {b: host[i] for i, b in enumerate(ids)}
        self.shape = tuple(pool.shape)
        self.dtype = np.float64

    def __getitem__(self, key):
        return self._rows[int(key[0])][key[1]]


def cpu_baseline(w, inp, tables, ctx, budget_s, gpu_out=None):
    """Time the oracle on whole sequences (all heads) until the wall-time budget is spent.

    The oracle runs as it stands: numpy in float64, its BLAS calls free to use
    the BLAS library's thread pool (the thread count is reported as ``cores``).
    Host copies of the blocks each sequence uses are made outside the timing.
    With ``gpu_out`` (the timed step's output), the sequences the oracle ran are
    also compared with the GPU rows (``parity``: max-abs / max-rel error).
    """
    import oracle
    import torch
    from threadpoolctl import threadpool_info
    q = inp["q"].cpu().to(torch.float64).numpy()
    elt = inp["k"].element_size()
    decode = None
    if getattr(w, "kv8", False):                      # E4M3 codes -> values, as the oracle reads them
        decode = lambda c: oracle.decode_e4m3(c) * np.float64(np.float32(w.kv_scale))
    done, kv_bytes, spent, refs = 0, 0, 0.0, []
    for s in range(w.num_seqs):
        n = int(ctx[s])
        blocks = tables[s, : -(-n // w.block_size)]
        kp = _BlockSubset(inp["k"], blocks, decode)
        vp = _BlockSubset(inp["v"], blocks, decode)
        t0 = time.perf_counter()
        refs.append(oracle.attend_ref(q[s:s + 1], kp, vp, tables[s:s + 1], ctx[s:s + 1], w.softmax_scale,
                                      w.block_size))
        spent += time.perf_counter() - t0
        done += 1
        kv_bytes += n * w.num_kv_heads * w.head_dim * 2 * elt
        if spent > budget_s:
            break
    blas_threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    res = {
        "value": round(kv_bytes / spent / 1e9, 6), "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
        "seq_per_s": round(done / spent, 3),
        "sample": f"first {done} of {w.num_seqs} sequences of the same decode step, all {w.num_heads} heads "
                  f"({kv_bytes / 1e6:.1f} MB of KV), fp64 numpy oracle, {spent:.1f} s wall",
        "host_cores_available": len(os.sched_getaffinity(0)),
    }
    if gpu_out is not None:
        got = gpu_out[:done].cpu().to(torch.float64).numpy()
        res["parity"] = parity_of(got, np.concatenate(refs), *TOLERANCE.get(w.kv_dtype, (2e-3, 1e-2)))
        res["parity"]["rows"] = f"all {done * w.num_heads} (sequence, head) rows of the first {done} sequences"
    return res


MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}     # dense MFMA, MI355X


def calibration_copy(w, dtype, nb, stream):
    """One copy_blocks call over nb block pairs: a plain copy of known size for the HBM counters."""
    import torch
    from paged_kv_cache_259_amd import ops
    big_k = torch.zeros((2 * nb, w.num_kv_heads, w.block_size, w.head_dim), dtype=dtype, device="cuda")
    big_v = torch.zeros_like(big_k)
    cal = torch.from_numpy(np.stack([np.arange(nb), np.arange(nb, 2 * nb)], 1).astype(np.int64)).to("cuda")
    ops.copy_blocks(big_k, big_v, cal, stream=stream)
    torch.cuda.synchronize()
    del big_k, big_v


def prefill_flops(w, ctx, chunk):
    """QK and PV flops of the visible (query, key) pairs: 4 * d * H per pair."""
    pairs = 0
    for c, n in zip(ctx.tolist(), chunk.tolist()):
        first = c - n + 1                          # keys visible to the chunk's first query
        pairs += n * first + n * (n - 1) // 2
    return 4 * w.head_dim * w.num_heads * pairs


def cpu_baseline_prefill(w, inp, tables, ctx, budget_s, gpu_out=None):
    """The oracle's prefill_ref, one whole sequence (all rows, all heads) at a time, until the budget is spent;
    with ``gpu_out``, the rows it recomputed are compared with the GPU's (``parity``)."""
    import oracle
    import torch
    from threadpoolctl import threadpool_info
    qsl = inp.query_start_loc
    decode = None
    if w.kv8:                                         # E4M3 codes -> values, as the oracle reads them
        decode = lambda c: oracle.dequant_e4m3(c, w.kv_scale)
    done, flops, spent, refs = 0, 0, 0.0, []
    for s in range(w.num_seqs):
        n, c = int(inp.chunk_lens[s]), int(ctx[s])
        blocks = tables[s, : -(-c // w.block_size)]
        kp = _BlockSubset(inp.k_cache, blocks, decode)
        vp = _BlockSubset(inp.v_cache, blocks, decode)
        q = inp.q[int(qsl[s]):int(qsl[s + 1])].cpu().to(torch.float64).numpy()
        t0 = time.perf_counter()
        refs.append(oracle.prefill_ref(q, kp, vp, tables[s:s + 1], ctx[s:s + 1], np.array([0, n]), w.softmax_scale,
                                       w.block_size))
        spent += time.perf_counter() - t0
        done += 1
        flops += prefill_flops(w, ctx[s:s + 1].astype(np.int64), inp.chunk_lens[s:s + 1].astype(np.int64))
        if spent > budget_s:
            break
    blas_threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    res = {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
           "sample": f"first {done} of {w.num_seqs} sequences of the same prefill step, all rows and heads, "
                     f"fp64 numpy oracle, {spent:.1f} s wall",
           "host_cores_available": len(os.sched_getaffinity(0))}
    if gpu_out is not None:
        got = gpu_out[: int(qsl[done])].cpu().to(torch.float64).numpy()
        res["parity"] = parity_of(got, np.concatenate(refs), 2e-3, 1e-2)
        res["parity"]["rows"] = f"every query row and head of the first {done} sequences"
    return res


def main_prefill(args, w):
    """One chunked-prefill step: reshape_and_cache of the chunk's K/V, then prefill attention."""
    import torch
    from paged_kv_cache_259_amd import ops, synth
    from paged_kv_cache_259_amd.block_manager import BlockManager

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = synth.make_prefill_inputs(w, device=dev)
    bm = BlockManager(inp.num_blocks, w.block_size, inp.free_list)
    seqs = list(range(w.num_seqs))
    slots = []
    for s in seqs:
        bm.add_sequence(s, int(inp.context_lens[s] - inp.chunk_lens[s]))
        slots += [bm.append_slot(s)[0] for _ in range(int(inp.chunk_lens[s]))]
    slots = torch.tensor(slots, dtype=torch.int64, device=dev)
    tables_np = bm.block_table_array(seqs, w.max_blocks_per_seq)
    tables = torch.from_numpy(tables_np).to(dev)
    ctx_np = bm.context_lens_array(seqs)
    ctx = torch.from_numpy(ctx_np).to(dev)
    qsl = torch.from_numpy(inp.query_start_loc.astype(np.int32)).to(dev)
    max_q, max_ctx = int(inp.chunk_lens.max()), int(ctx_np.max())
    out = torch.empty_like(inp.q)
    stream = torch.cuda.current_stream()

    sc = dict(k_scale=w.kv_scale, v_scale=w.kv_scale) if w.kv8 else {}

    def reshape():
        ops.reshape_and_cache(inp.k_new, inp.v_new, inp.k_cache, inp.v_cache, slots, stream=stream, **sc)

    def attend():
        ops.paged_prefill_attention(out, inp.q, inp.k_cache, inp.v_cache, tables, ctx, qsl, w.softmax_scale, max_q,
                                    max_ctx, stream=stream, **sc)

    warm = warm_up(lambda: (reshape(), attend()), args.warmup)
    K = args.steps
    flusher = Flusher(stream)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        flusher()
        ev[i][0].record(stream)
        reshape()
        ev[i][1].record(stream)
        attend()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    t_attn = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in range(K)])
    t_step = np.array([ev[i][0].elapsed_time(ev[i][2]) for i in range(K)])
    out_step = out.clone()
    flops = prefill_flops(w, ctx_np.astype(np.int64), inp.chunk_lens.astype(np.int64))
    attn_ms, step_ms = float(np.mean(t_attn)), float(np.mean(t_step))
    tokens = int(inp.chunk_lens.sum())
    if args.calibrate_copy:
        calibration_copy(w, inp.k_cache.dtype, args.calibrate_copy, stream)
    achieved = flops / (attn_ms * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    result = {
        "metric": "paged chunked-prefill attention TFLOP/s (% of dense MFMA peak) + prefill tokens/s per layer step",
        "value": round(flops / (step_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": warm, "ms_per_step": round(step_ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) q/K/V" + (", E4M3 pool codes" if w.kv8 else "")
                + ", uniform prior context lengths, shuffled block tables)",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                   "query_tokens": tokens, "sum_context": int(ctx_np.sum()), "max_context": max_ctx},
        "timing": "mean of K steps, HIP events on the launch stream; before each step 512 MiB are written and "
                  "another 512 MiB read (L2 and Infinity Cache cleared), outside the events",
        "tokens_per_s": round(tokens / (step_ms * 1e-3), 1),
        "slot_utilisation": slot_utilisation(ctx_np, w.block_size),
        "max_abs_err": None,
        "max_rel_err": None,
        "components": {"reshape_and_cache_us": round(float(np.mean(t_step - t_attn)) * 1e3, 2),
                       "paged_prefill_attention_us": round(attn_ms * 1e3, 2),
                       "paged_prefill_attention_median_us": round(float(np.median(t_attn)) * 1e3, 2)},
        "roofline": {"bound": "mfma", "kernel": "paged_prefill_attention", "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(args.workload), "algorithmic_flops_per_call": int(flops),
                     "kv_bytes_per_call": int(ctx_np.sum()) * w.num_kv_heads * w.head_dim * 2 * inp.k_cache.element_size()},
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline_prefill(w, inp, tables_np, ctx_np, args.cpu_seconds, gpu_out=out_step)
        result["cpu_baseline"] = cb
        result["max_abs_err"], result["max_rel_err"] = cb["parity"]["max_abs_err"], cb["parity"]["max_rel_err"]
    print(json.dumps(result))


def main_prefix_cache(args, w):
    """A prefill step of requests sharing a system prompt, without and with the prefix cache.

    Without: every request writes and attends its whole prompt.  With: the first
    request does; the others hit the shared prompt's full blocks and write and
    attend only their own tokens as a chunk over the cached context.  Each flow
    is reshape_and_cache + one batched paged_prefill_attention call.
    """
    import torch
    from paged_kv_cache_259_amd import ops, synth
    from paged_kv_cache_259_amd.block_manager import BlockManager

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = synth.make_prefix_cache_inputs(w, device=dev)
    R, L = w.num_requests, w.shared_len + w.unique_len
    stream = torch.cuda.current_stream()
    shape = (inp.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
    flows = {}
    for cache in (False, True):
        bm = BlockManager(inp.num_blocks, w.block_size, inp.free_list, prefix_cache=cache)
        slots, rows, chunk = [], [], []
        for r in range(R):
            if cache:
                sl, cached = bm.add_sequence_cached(r, inp.prompts[r])
            else:
                sl, cached = bm.add_sequence(r, L), 0
            slots += sl
            rows += list(range(r * L + cached, (r + 1) * L))
            chunk.append(L - cached)
        rows_t = torch.tensor(rows, dtype=torch.int64, device=dev)
        f = {"slots": torch.tensor(slots, dtype=torch.int64, device=dev), "q": inp.q.index_select(0, rows_t),
             "k": inp.k.index_select(0, rows_t), "v": inp.v.index_select(0, rows_t),
             "tables": torch.from_numpy(bm.block_table_array(list(range(R)), w.max_blocks_per_seq)).to(dev),
             "ctx": torch.full((R,), L, dtype=torch.int32, device=dev),
             "qsl": torch.from_numpy(np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)).to(dev),
             "chunk": np.array(chunk, np.int64), "kc": torch.empty(shape, dtype=inp.q.dtype, device=dev),
             "cached_blocks": bm.cached_blocks()}
        f["kv"] = torch.empty_like(f["kc"])
        f["out"] = torch.empty_like(f["q"])
        flows["cache" if cache else "no_cache"] = f

    def run(f):
        ops.reshape_and_cache(f["k"], f["v"], f["kc"], f["kv"], f["slots"], stream=stream)
        ops.paged_prefill_attention(f["out"], f["q"], f["kc"], f["kv"], f["tables"], f["ctx"], f["qsl"],
                                    w.softmax_scale, int(f["chunk"].max()), L, stream=stream)

    res, warms = {}, []
    for name, f in flows.items():
        warms.append(warm_up(lambda: run(f), args.warmup))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            run(f)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        flops = prefill_flops(w, np.full(R, L, np.int64), f["chunk"])
        res[name] = {"ms_per_step": round(ms, 4), "query_tokens": int(f["chunk"].sum()),
                     "kv_tokens_written": int(f["chunk"].sum()), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                     "cached_blocks": f["cached_blocks"]}
    speedup = res["no_cache"]["ms_per_step"] / res["cache"]["ms_per_step"]
    fc = flows["cache"]
    flops_c = prefill_flops(w, np.full(R, L, np.int64), fc["chunk"])
    result = {
        "metric": "prefill step time of requests sharing a system prompt, prefix cache off / on",
        "value": round(speedup, 3), "unit": "x", "n_gpus": 1, "steps": args.steps, "warmup": min(warms),
        "ms_per_step": res["cache"]["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded token ids and N(0,1) q/K/V; shared-prefix K/V identical across requests)",
        "config": {"workload": w.name, "requests": R, "shared_len": w.shared_len, "unique_len": w.unique_len},
        "flows": res,
        "roofline": {"bound": "mfma", "kernel": "reshape_and_cache + paged_prefill_attention (prefix cache on)",
                     "achieved": round(flops_c / (res["cache"]["ms_per_step"] * 1e-3) / 1e12, 2),
                     "peak": MFMA_PEAK_TFLOPS[w.dtype], "unit": "TFLOP/s",
                     "frac": round(flops_c / (res["cache"]["ms_per_step"] * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[w.dtype], 4),
                     "traffic": None, "algorithmic_flops_per_call": int(flops_c)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_prefix(w, inp, fc, args.cpu_seconds)
    print(json.dumps(result))


def cpu_baseline_prefix(w, inp, f, budget_s):
    """The oracle's prefill_ref on the cached flow's chunks, one request at a time, until the budget is spent."""
    import oracle
    import torch
    from threadpoolctl import threadpool_info
    L = w.shared_len + w.unique_len
    tables = f["tables"].cpu().numpy()
    qsl = f["qsl"].cpu().numpy()
    done, flops, spent = 0, 0, 0.0
    for r in range(w.num_requests):
        n = int(f["chunk"][r])
        kp = _BlockSubset(f["kc"], tables[r, : -(-L // w.block_size)])
        vp = _BlockSubset(f["kv"], tables[r, : -(-L // w.block_size)])
        q = f["q"][int(qsl[r]):int(qsl[r + 1])].cpu().to(torch.float64).numpy()
        t0 = time.perf_counter()
        oracle.prefill_ref(q, kp, vp, tables[r:r + 1], np.array([L]), np.array([0, n]), w.softmax_scale, w.block_size)
        spent += time.perf_counter() - t0
        done += 1
        flops += prefill_flops(w, np.array([L], np.int64), np.array([n], np.int64))
        if spent > budget_s:
            break
    blas_threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"first {done} of {w.num_requests} requests' chunks of the cached flow, fp64 numpy oracle, "
                      f"{spent:.1f} s wall",
            "host_cores_available": len(os.sched_getaffinity(0))}


def unique_kv_bytes(tables, ctx, bs, row_bytes):
    """KV bytes of the distinct physical blocks the step reads: each block once, with the most tokens any
    sequence uses of it."""
    used = {}
    for s in range(len(ctx)):
        n = int(ctx[s])
        for j in range(-(-n // bs)):
            b = int(tables[s, j])
            used[b] = max(used.get(b, 0), min(bs, n - j * bs))
    return sum(used.values()) * row_bytes


def main_shared_prefix(args, w):
    """The next decode step of every sample of the shared-prefix workload (fp8 pools, copy-on-write).

    Untimed set-up by the host driver: each prompt's K/V written once and shared
    by its samples; continuations appended one token per step, copying a shared
    partly filled block on a sample's first write into it; one decode over every
    sample.  The timed step: the block manager gives every sample the slot of
    its next token (copy-on-write pairs where that slot's block is still
    shared), then copy_blocks over those pairs (when any) and one
    paged_attention_decode_append launch that writes each sample's new token and
    attends.  Repeating the step rewrites the same bytes, so every timed step
    does the same work.

    The attention of the step is paged_attention_decode_shared: the samples of
    a prompt form one group (BlockManager.shared_groups), and each block the
    group shares is read once for all of them.  The same step through
    paged_attention_decode_append (every sample reads its whole context) is
    reported beside it.
    """
    import torch
    from paged_kv_cache_259_amd import ops, synth
    from paged_kv_cache_259_amd.shared_prefix import run_shared_prefix

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = synth.make_shared_prefix_inputs(w, device=dev)
    t_setup = time.perf_counter()
    res = run_shared_prefix(inp, dev)
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup
    bm, kc, vc = res["block_manager"], res["k_cache"], res["v_cache"]
    ks, vs = res["k_scale"], res["v_scale"]
    seqs = list(range(w.num_seqs))
    slots, pairs = [], []
    for s in seqs:
        slot, pair = bm.append_slot(s)
        slots.append(slot)
        if pair is not None:
            pairs.append(pair)
    tables_np = bm.block_table_array(seqs, w.max_blocks_per_seq)
    ctx_np = bm.context_lens_array(seqs)
    tables, ctx = torch.from_numpy(tables_np).to(dev), torch.from_numpy(ctx_np).to(dev)
    order = torch.from_numpy(bm.longest_first(seqs, group_shared=True)).to(dev)   # forks of a prompt together
    slot_t = torch.tensor(slots, dtype=torch.int64, device=dev)
    pair_t = torch.tensor(pairs, dtype=torch.int64, device=dev).reshape(-1, 2)
    k_new, v_new = synth.draw_step_kv(inp, len(seqs), dev)
    q = synth.draw_query(inp, len(seqs), dev)
    out = torch.empty_like(q)
    max_ctx = int(ctx_np.max())
    qd, kvd = ops.dtype_code(q.dtype), ops.dtype_code(kc.dtype)
    plan = ops.attention_plan(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size, max_ctx, 0, qd, kvd)
    ws_bytes = ops.attention_workspace_bytes(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size,
                                             max_ctx, 0, qd, kvd)
    workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    g_off, g_mem, g_shared = bm.shared_groups(seqs, args.group_size or 16 // (w.num_heads // w.num_kv_heads))
    g_max = int(np.diff(g_off).max())
    groups = [torch.from_numpy(a).to(dev) for a in (g_off, g_mem, g_shared)]

    def cow():
        if len(pairs):
            ops.copy_blocks(kc, vc, pair_t, stream=stream)

    each_policy = bm.kv_load_policy(seqs)   # forks share their prompt's blocks: "cached"

    def attend_each(policy=each_policy):  # every sample reads its whole context
        with ops.kv_load_policy(policy):
            ops.paged_attention_decode_append(out, q, kc, vc, k_new, v_new, slot_t, tables, ctx, w.softmax_scale,
                                              max_ctx, k_scale=ks, v_scale=vs, workspace=workspace, seq_order=order,
                                              stream=stream)

    def attend():                        # shared blocks read once per group
        ops.paged_attention_decode_shared(out, q, kc, vc, tables, ctx, *groups, g_max, w.softmax_scale, max_ctx,
                                          key=k_new, value=v_new, slot_mapping=slot_t, k_scale=ks, v_scale=vs,
                                          stream=stream)

    warm = warm_up(lambda: (cow(), attend(), attend_each()), args.warmup)
    K = args.steps
    flusher = Flusher(stream)

    def timed(fn):
        return timed_steps(fn, K, stream, flusher)

    t_step = timed(lambda: (cow(), attend()))
    out_step = out.clone()
    t_attn = timed(attend)
    t_each = timed(attend_each)
    other_policy = "stream" if each_policy == "cached" else "cached"
    t_each_other = timed(lambda: attend_each(other_policy))
    t_cow = timed(cow) if len(pairs) else None
    t_hot = timed_steps(lambda: (cow(), attend()), K, stream)
    step_ms, attn_ms = float(np.mean(t_step)), float(np.mean(t_attn))
    if args.calibrate_copy:
        calibration_copy(w, kc.dtype, args.calibrate_copy, stream)

    row_bytes = w.num_kv_heads * w.head_dim * 2 * kc.element_size()
    kv_logical, alg_bytes = algorithmic_bytes(w, ctx_np.astype(np.int64), q.element_size(), kc.element_size())
    kv_unique = unique_kv_bytes(tables_np, ctx_np, w.block_size, row_bytes)
    append_bytes = 2 * w.num_seqs * w.num_kv_heads * w.head_dim * (k_new.element_size() + kc.element_size()) \
        + 8 * w.num_seqs
    unique_alg = alg_bytes - kv_logical + kv_unique
    result = {
        "metric": "paged decode KV-read GB/s (% of HBM peak) + sequences/sec per decode step",
        "value": round(kv_logical / (step_ms * 1e-3) / 1e9, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": warm, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3",
        "data": "synthetic (seeded N(0,1) prompt and continuation K/V in fp16, encoded to E4M3 with amax/448 "
                "scales; uniform continuation lengths)",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                   "q_dtype": w.q_dtype, "kv_dtype": w.kv_dtype, "sum_context": int(ctx_np.sum()),
                   "max_context": max_ctx, "num_blocks": w.num_blocks,
                   "plan": {"path": ["vector", "mfma"][plan[0]], "partition_tokens": plan[1],
                            "num_partitions": plan[2]}},
        "timing": "mean of K steps, HIP events on the launch stream; before each step 512 MiB are written and "
                  "another 512 MiB read (L2 and Infinity Cache cleared), outside the events",
        "pct_of_hbm_peak": round(100.0 * kv_logical / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        "seq_per_s": round(w.num_seqs / (step_ms * 1e-3), 1),
        "kv_bytes_per_step": {"logical": kv_logical, "unique": kv_unique},
        "slot_utilisation": slot_utilisation(ctx_np, w.block_size),
        "max_abs_err": None,
        "max_rel_err": None,
        "unique_gbps": round(kv_unique / (step_ms * 1e-3) / 1e9, 1),
        "sharing": {"logical_blocks": res["logical_blocks"], "unique_blocks": res["unique_blocks"],
                    "cow_pairs_during_generation": res["cow_pairs"], "cow_pairs_this_step": len(pairs),
                    "groups": len(g_shared), "max_group_size": g_max,
                    "shared_blocks_per_group": int(np.median(g_shared)) if len(g_shared) else 0,
                    "setup_s": round(t_setup, 2)},
        "components": {"copy_blocks_us": None if t_cow is None else round(float(np.mean(t_cow)) * 1e3, 2),
                       "step_us_back_to_back": round(float(np.mean(t_hot)) * 1e3, 2),
                       "paged_attention_decode_shared_us": round(attn_ms * 1e3, 2),
                       "paged_attention_decode_shared_median_us": round(float(np.median(t_attn)) * 1e3, 2),
                       "paged_attention_decode_append_us": round(float(np.mean(t_each)) * 1e3, 2),
                       "paged_attention_decode_append_median_us": round(float(np.median(t_each)) * 1e3, 2),
                       "paged_attention_decode_append_kv_loads": each_policy,
                       f"paged_attention_decode_append_{other_policy}_us": round(float(np.mean(t_each_other)) * 1e3,
                                                                                 2)},
        "roofline": {
            "bound": "hbm",
            "kernel": "paged_attention_decode_shared with append over fp8 pools (achieved counts each physical block "
                      "once; the logical rate, each sample reading its whole context, is value)",
            "achieved": round((unique_alg + append_bytes) / (attn_ms * 1e-3) / 1e9, 1),
            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round((unique_alg + append_bytes) / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(args.workload),
            "algorithmic_bytes_per_call": unique_alg + append_bytes,
            "logical_bytes_per_call": alg_bytes + append_bytes,
        },
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline_shared(w, q, kc, vc, ks, vs, tables_np, ctx_np, args.cpu_seconds, gpu_out=out_step)
        result["cpu_baseline"] = cb
        result["max_abs_err"], result["max_rel_err"] = cb["parity"]["max_abs_err"], cb["parity"]["max_rel_err"]
    print(json.dumps(result))


def cpu_baseline_shared(w, q, kc, vc, ks, vs, tables, ctx, budget_s, gpu_out=None):
    """The oracle on whole samples (all heads) over the dequantised E4M3 codes, until the budget is spent;
    with ``gpu_out``, the samples it recomputed are compared with the GPU's rows (``parity``)."""
    import oracle
    import torch
    from threadpoolctl import threadpool_info
    qh = q.cpu().to(torch.float64).numpy()
    done, kv_bytes, spent, refs = 0, 0, 0.0, []
    for s in range(len(ctx)):
        n = int(ctx[s])
        nb = -(-n // w.block_size)
        blocks = torch.from_numpy(tables[s, :nb].astype(np.int64)).to(kc.device)
        kcodes = kc.index_select(0, blocks).cpu().numpy()
        vcodes = vc.index_select(0, blocks).cpu().numpy()
        local = np.arange(nb, dtype=np.int32)[None, :]
        t0 = time.perf_counter()
        kp = oracle.decode_e4m3(kcodes) * np.float64(np.float32(ks))
        vp = oracle.decode_e4m3(vcodes) * np.float64(np.float32(vs))
        refs.append(oracle.attend_ref(qh[s:s + 1], kp, vp, local, ctx[s:s + 1], w.softmax_scale, w.block_size))
        spent += time.perf_counter() - t0
        done += 1
        kv_bytes += n * w.num_kv_heads * w.head_dim * 2
        if spent > budget_s:
            break
    blas_threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    res = {"value": round(kv_bytes / spent / 1e9, 6), "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
           "seq_per_s": round(done / spent, 3),
           "sample": f"first {done} of {len(ctx)} samples of the same decode step, all {w.num_heads} heads "
                     f"({kv_bytes / 1e6:.1f} MB of logical E4M3 KV, dequantised by the oracle), fp64 numpy "
                     f"oracle, {spent:.1f} s wall",
           "host_cores_available": len(os.sched_getaffinity(0))}
    if gpu_out is not None:
        res["parity"] = parity_of(gpu_out[:done].cpu().to(torch.float64).numpy(), np.concatenate(refs), 2e-3, 1e-2)
        res["parity"]["rows"] = f"all (sample, head) rows of the first {done} samples"
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the paged decode path is a "
                                   "single-GPU library (each GPU would hold its own share of the heads and "
                                   "sequences); no multi-GPU mode exists",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    from paged_kv_cache_259_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "stream_probe":
        return main_stream_probe(args)
    w = synth.WORKLOADS[args.workload]
    if isinstance(w, synth.PrefillWorkload):
        return main_prefill(args, w)
    if isinstance(w, synth.PrefixCacheWorkload):
        return main_prefix_cache(args, w)
    if isinstance(w, synth.SharedPrefixWorkload):
        return main_shared_prefix(args, w)
    if not isinstance(w, synth.DecodeWorkload):
        raise SystemExit("unknown workload kind: " + args.workload)
    return main_decode(args, w)


class DecodeState:
    """One decode workload on the GPU: inputs drawn on the device, tables and slots from the host block manager
    (the new token of every sequence gets its slot; the longest-first order is host bookkeeping too), and the
    three ways to run its step."""

    def __init__(self, w, part, dev, stream):
        import torch
        from paged_kv_cache_259_amd import ops, synth
        from paged_kv_cache_259_amd.block_manager import BlockManager
        self.w, self.part, self.stream = w, part, stream
        self.inp = inp = synth.make_decode_inputs(w, device=dev)
        bm = BlockManager(inp.num_blocks, w.block_size, inp.free_list)
        self.seqs = seqs = list(range(w.num_seqs))
        for s in seqs:
            bm.add_sequence(s, int(inp.context_lens[s]) - 1)           # cached before this step
        self.slots = torch.tensor([bm.append_slot(s)[0] for s in seqs], dtype=torch.int64, device=dev)
        self.tables_np = bm.block_table_array(seqs, w.max_blocks_per_seq)
        self.ctx_np = bm.context_lens_array(seqs)
        self.tables = torch.from_numpy(self.tables_np).to(dev)
        self.ctx = torch.from_numpy(self.ctx_np).to(dev)
        self.order = torch.from_numpy(bm.longest_first(seqs)).to(dev)
        self.max_ctx = int(self.ctx_np.max())
        self.qd, self.kvd = ops.dtype_code(inp.q.dtype), ops.dtype_code(inp.k_cache.dtype)
        self.plan = ops.attention_plan(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size,
                                       self.max_ctx, part, self.qd, self.kvd)
        ws_bytes = ops.attention_workspace_bytes(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size,
                                                 self.max_ctx, part, self.qd, self.kvd)
        self.workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.out = torch.empty_like(inp.q)
        self.kvs = dict(k_scale=w.kv_scale, v_scale=w.kv_scale) if w.kv8 else {}
        elt_q, elt_kv = inp.q.element_size(), inp.k_cache.element_size()
        self.kv_bytes, self.alg_bytes = algorithmic_bytes(w, self.ctx_np.astype(np.int64), elt_q, elt_kv)
        self.append_bytes = (2 * w.num_seqs * w.num_kv_heads * w.head_dim * (inp.k_new.element_size() + elt_kv)
                             + 8 * w.num_seqs)
        self.step_bytes = self.alg_bytes + self.append_bytes

    def reshape(self):
        from paged_kv_cache_259_amd import ops
        i = self.inp
        ops.reshape_and_cache(i.k_new, i.v_new, i.k_cache, i.v_cache, self.slots, stream=self.stream, **self.kvs)

    def attend(self, part=None, workspace=None):
        from paged_kv_cache_259_amd import ops
        i = self.inp
        ops.paged_attention_decode(self.out, i.q, i.k_cache, i.v_cache, self.tables, self.ctx, self.w.softmax_scale,
                                   self.max_ctx, partition_size=self.part if part is None else part,
                                   workspace=self.workspace if workspace is None else workspace,
                                   seq_order=self.order, stream=self.stream, **self.kvs)

    def step(self, part=None, workspace=None):
        """The whole step in one launch: write the new tokens, attend."""
        from paged_kv_cache_259_amd import ops
        i = self.inp
        ops.paged_attention_decode_append(self.out, i.q, i.k_cache, i.v_cache, i.k_new, i.v_new, self.slots,
                                          self.tables, self.ctx, self.w.softmax_scale, self.max_ctx,
                                          partition_size=self.part if part is None else part,
                                          workspace=self.workspace if workspace is None else workspace,
                                          seq_order=self.order, stream=self.stream, **self.kvs)

    def plan_json(self, plan=None):
        plan = plan or self.plan
        return {"path": ["vector", "mfma"][plan[0]], "partition_tokens": plan[1], "num_partitions": plan[2],
                "mode": ("one pass" if plan[2] == 1 else "balanced slices" if plan[1] == 0 else "fixed partitions")}

    def pct(self, ms, nbytes=None):
        return 100.0 * (self.step_bytes if nbytes is None else nbytes) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS


def decode_component(name, args, dev, stream, flusher, probe_gbps):
    """Another decode workload timed in the same run (flushed and back to back); its oracle parity on a few
    sequences unless the CPU baseline is off."""
    from paged_kv_cache_259_amd import synth
    w = synth.WORKLOADS[name]
    st = DecodeState(w, w.partition_size, dev, stream)
    warm_up(st.step, args.warmup)
    t_flush = timed_steps(st.step, args.steps, stream, flusher)
    t_hot = timed_steps(st.step, args.steps, stream)
    out_step = st.out.clone()
    ms, ms_hot = float(np.mean(t_flush)), float(np.mean(t_hot))
    achieved = st.step_bytes / (ms * 1e-3) / 1e9
    comp = {"workload": w.name, "plan": st.plan_json(), "step_us": round(ms * 1e3, 2),
            "step_median_us": round(float(np.median(t_flush)) * 1e3, 2),
            "step_us_back_to_back": round(ms_hot * 1e3, 2),
            "kv_gbps": round(st.kv_bytes / (ms * 1e-3) / 1e9, 1),
            "achieved_gbps": round(achieved, 1), "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "frac_back_to_back": round(st.pct(ms_hot) / 100, 4),
            "pct_of_measured_stream_bw": round(100.0 * achieved / probe_gbps, 2) if probe_gbps else None,
            "seq_per_s": round(w.num_seqs / (ms * 1e-3), 1),
            "algorithmic_bytes_per_call": st.step_bytes,
            "slot_utilisation": slot_utilisation(st.ctx_np, w.block_size),
            "traffic": measured_traffic(name)}
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, {"q": st.inp.q, "k": st.inp.k_cache, "v": st.inp.v_cache}, st.tables_np, st.ctx_np,
                          min(args.cpu_seconds, 5.0), gpu_out=out_step)
        comp["parity"] = cb["parity"]
        comp["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "sample")}
    del st
    return comp


def main_stream_probe(args):
    """What HBM delivers to read-only kernels on this machine (the decode roofline's achievable ceiling)."""
    import torch
    stream = torch.cuda.current_stream()
    res = hbm_probe(stream, reps=max(args.steps // 10, 5), flush=Flusher(stream))
    print(json.dumps({
        "metric": "HBM read GB/s of a streaming read kernel and of random-tile reads (% of 8 TB/s)",
        "value": res["stream_read_gbps"], "unit": "GB/s", "n_gpus": 1, "steps": max(args.steps // 10, 5),
        "warmup": 3, "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8", "data": "synthetic (1 GiB of ones)", "config": {"workload": "stream_probe"},
        "pct_of_hbm_peak": round(100.0 * res["stream_read_gbps"] / HBM_PEAK_GBPS, 2), "probe": res,
        "roofline": {"bound": "hbm", "kernel": "stream_read_kernel", "achieved": res["stream_read_gbps"],
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(res["stream_read_gbps"] / HBM_PEAK_GBPS, 4),
                     "traffic": None}}))


def main_decode(args, w):
    import torch
    from paged_kv_cache_259_amd import ops, synth

    dev = torch.device("cuda:0")
    part = w.partition_size if args.partition is None else args.partition
    stream = torch.cuda.current_stream()
    st = DecodeState(w, part, dev, stream)
    inp, tables_np, ctx_np, seqs = st.inp, st.tables_np, st.ctx_np, st.seqs
    flusher = Flusher(stream)

    warm = warm_up(lambda: (st.reshape(), st.attend(), st.step()), args.warmup)
    K = args.steps
    # the timed step: decode with append, caches flushed before every step (the headline), then back to back
    t0 = time.perf_counter()
    t_step = timed_steps(st.step, K, stream, flusher)
    wall = time.perf_counter() - t0
    out_step = st.out.clone()
    t_hot = timed_steps(st.step, K, stream)
    step_ms, hot_ms = float(np.mean(t_step)), float(np.mean(t_hot))
    # the same step as two launches (reshape_and_cache, then decode), for the components
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        flusher()
        ev[i][0].record(stream)
        st.reshape()
        ev[i][1].record(stream)
        st.attend()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    t_reshape = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(K)])
    t_attn = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in range(K)])
    t_split = np.array([ev[i][0].elapsed_time(ev[i][2]) for i in range(K)])

    # ---- with a stated partition size: the same step under the library's automatic plan, for comparison
    # (not in counter runs, which must hold only the timed step's kernels)
    auto = None
    if part and not args.calibrate_copy:
        auto_plan = ops.attention_plan(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size, st.max_ctx,
                                       0, st.qd, st.kvd)
        auto_ws = torch.empty(max(ops.attention_workspace_bytes(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                                                                w.block_size, st.max_ctx, 0, st.qd, st.kvd), 256),
                              dtype=torch.uint8, device=dev)
        warm_up(lambda: st.step(0, auto_ws), 10)
        t_auto = float(np.mean(timed_steps(lambda: st.step(0, auto_ws), K, stream, flusher)))
        auto = {"plan": st.plan_json(auto_plan), "step_us": round(t_auto * 1e3, 2),
                "pct_of_hbm_peak": round(st.pct(t_auto), 2)}

    # ---- copy_blocks on copy-on-write pairs shaped like the shared-prefix workload (timed separately)
    sp = synth.SHARED_PREFIX_FP8
    n_pairs = 3 * sp.num_prompts
    cb_pool_k = torch.zeros((2 * n_pairs + 8, sp.num_heads, sp.block_size, sp.head_dim), dtype=torch.uint8, device=dev)
    cb_pool_v = torch.zeros_like(cb_pool_k)
    perm = np.random.default_rng(sp.seed).permutation(2 * n_pairs)
    pairs = torch.from_numpy(np.stack([perm[:n_pairs], perm[n_pairs:]], 1).astype(np.int64)).to(dev)
    for _ in range(3):
        ops.copy_blocks(cb_pool_k, cb_pool_v, pairs, stream=stream)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(20):
        ops.copy_blocks(cb_pool_k, cb_pool_v, pairs, stream=stream)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_us = c0.elapsed_time(c1) / 20 * 1e3
    block_bytes = sp.num_heads * sp.block_size * sp.head_dim

    # ---- swap_blocks: the 16 most recent sequences preempted whole (device -> pinned host) and back
    n_sw = min(16, w.num_seqs)
    sw_blocks = np.unique(np.concatenate([tables_np[s, : -(-int(ctx_np[s]) // w.block_size)]
                                          for s in seqs[-n_sw:]])).astype(np.int64)
    host_k = torch.empty((len(sw_blocks),) + tuple(inp.k_cache.shape[1:]), dtype=inp.k_cache.dtype, pin_memory=True)
    host_v = torch.empty((len(sw_blocks),) + tuple(inp.k_cache.shape[1:]), dtype=inp.k_cache.dtype, pin_memory=True)
    out_map = torch.from_numpy(np.stack([sw_blocks, np.arange(len(sw_blocks))], 1)).to(dev)
    in_map = torch.from_numpy(np.stack([np.arange(len(sw_blocks)), sw_blocks], 1)).to(dev)   # back in place
    sw_bytes = 2 * len(sw_blocks) * inp.k_cache[0].numel() * inp.k_cache.element_size()
    ops.swap_blocks(inp.k_cache, inp.v_cache, host_k, host_v, out_map, stream=stream)
    ops.swap_blocks(host_k, host_v, inp.k_cache, inp.v_cache, in_map, stream=stream)
    sw_ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    t_out, t_in = [], []
    for _ in range(5):
        sw_ev[0].record(stream)
        ops.swap_blocks(inp.k_cache, inp.v_cache, host_k, host_v, out_map, stream=stream)
        sw_ev[1].record(stream)
        ops.swap_blocks(host_k, host_v, inp.k_cache, inp.v_cache, in_map, stream=stream)
        sw_ev[2].record(stream)
        torch.cuda.synchronize()
        t_out.append(sw_ev[0].elapsed_time(sw_ev[1]))
        t_in.append(sw_ev[1].elapsed_time(sw_ev[2]))
    swap_out_ms, swap_in_ms = float(np.median(t_out)), float(np.median(t_in))

    if args.calibrate_copy:
        calibration_copy(w, inp.k_cache.dtype, args.calibrate_copy, stream)

    # ---- what HBM delivers to a read-only kernel here, and the GQA step beside the headline workload
    probe = None if args.calibrate_copy else hbm_probe(stream, flush=flusher)
    probe_gbps = probe["stream_read_gbps"] if probe else None
    gqa = None
    if args.workload == "llama13b_f16" and not args.calibrate_copy and not args.no_components:
        gqa = decode_component("gqa_bf16", args, dev, stream, flusher, probe_gbps)

    kv_bytes, alg_bytes = st.kv_bytes, st.alg_bytes
    attn_ms = float(np.mean(t_attn))
    achieved = st.step_bytes / (step_ms * 1e-3) / 1e9
    traffic = measured_traffic(args.workload)
    result = {
        "metric": "paged decode KV-read GB/s (% of HBM peak) + sequences/sec per decode step",
        "value": round(kv_bytes / (step_ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warm,
        "warmup_requested": args.warmup,
        "warmup_note": f"warm-up runs at least --warmup steps and at least {int(WARMUP_MIN_S * 1e3)} ms of GPU work",
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype,
        "data": ("synthetic (seeded N(0,1) q and new K/V, uniform E4M3 pool codes, lognormal context lengths, "
                 "shuffled block tables)" if w.kv8 else
                 "synthetic (seeded N(0,1) q/K/V, lognormal context lengths, shuffled block tables)"),
        "config": {
            "workload": w.name, "num_seqs": w.num_seqs, "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size, "q_dtype": w.q_dtype, "kv_dtype": w.kv_dtype,
            "sum_context": int(ctx_np.sum()), "max_context": st.max_ctx, "num_blocks": inp.num_blocks,
            "plan": st.plan_json(),
        },
        "timing": "mean of K steps, HIP events on the launch stream; before each step 512 MiB are written and "
                  "another 512 MiB read (L2 and Infinity Cache cleared), outside the events",
        "pct_of_hbm_peak": round(100.0 * kv_bytes / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        "pct_of_measured_stream_bw": round(100.0 * achieved / probe_gbps, 2) if probe_gbps else None,
        "seq_per_s": round(w.num_seqs / (step_ms * 1e-3), 1),
        "kv_bytes_per_step": kv_bytes,
        "slot_utilisation": slot_utilisation(ctx_np, w.block_size),
        "max_abs_err": None,
        "max_rel_err": None,
        "components": {
            "paged_attention_decode_append_us": round(step_ms * 1e3, 2),
            "paged_attention_decode_append_median_us": round(float(np.median(t_step)) * 1e3, 2),
            "step_us_back_to_back": round(hot_ms * 1e3, 2),
            "frac_back_to_back": round(st.pct(hot_ms) / 100, 4),
            "two_launch_step_us": round(float(np.mean(t_split)) * 1e3, 2),
            "reshape_and_cache_us": round(float(np.mean(t_reshape)) * 1e3, 2),
            "paged_attention_decode_us": round(attn_ms * 1e3, 2),
            "paged_attention_decode_median_us": round(float(np.median(t_attn)) * 1e3, 2),
            "attention_kv_gbps": round(kv_bytes / (attn_ms * 1e-3) / 1e9, 1),
            "attention_pct_of_hbm_peak": round(100.0 * alg_bytes / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
            "copy_blocks_us": round(copy_us, 2),
            "copy_blocks_pairs": n_pairs,
            "copy_blocks_gbps": round(2 * 2 * n_pairs * block_bytes / (copy_us * 1e-6) / 1e9, 1),
            "wall_ms_per_step": round(wall / K * 1e3, 4),
            "automatic_plan_step": auto,
            "swap_blocks": {"blocks": int(len(sw_blocks)), "sequences": n_sw, "bytes": int(sw_bytes),
                            "out_us": round(swap_out_ms * 1e3, 1), "in_us": round(swap_in_ms * 1e3, 1),
                            "out_gbps": round(sw_bytes / (swap_out_ms * 1e-3) / 1e9, 1),
                            "in_gbps": round(sw_bytes / (swap_in_ms * 1e-3) / 1e9, 1)},
            "hbm_probe": probe,
            "gqa_bf16": gqa,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "paged_attention_decode_append (attention kernel writing the new tokens, + split-context "
                      "reduce when planned)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_call": st.step_bytes,
        },
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, {"q": inp.q, "k": inp.k_cache, "v": inp.v_cache}, tables_np, ctx_np, args.cpu_seconds,
                          gpu_out=out_step)
        result["cpu_baseline"] = cb
        result["max_abs_err"] = cb["parity"]["max_abs_err"]
        result["max_rel_err"] = cb["parity"]["max_rel_err"]
    print(json.dumps(result))


if __name__ == "__main__":
    main()
