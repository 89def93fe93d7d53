"""Parallel sampling over shared prompts with copy-on-write, FP8 cache.

Host driver for the shared-prefix workload: every prompt's KV cache is written
once and shared by its n samples through their block tables (reference count
n); each sample then appends its own continuation one token per step, and the
first write of a sample into the shared, partly filled last block copies that
block first ("KV cache paginado e batching contínuo para LLMs", section "Como
funciona"; "PagedAttention", Ultralytics glossary, section "Chia sẻ block giữa
các chuỗi").  Per step: ``copy_blocks`` for the new copy-on-write pairs, then
``reshape_and_cache`` for the step's tokens.  At the end one
``paged_attention_decode`` runs over every sample.

Within a step samples act in ascending index order; a sample copies when its
last block is shared at that moment, so the last remaining holder writes in
place (reading of the pages: they say a writer of a shared block copies and
decrements the original's count).
"""

import numpy as np
import torch

from . import ops, synth
from .block_manager import BlockManager


def run_shared_prefix(inp: synth.SharedPrefixInputs, device, on_step=None, on_prefill=None):
    """Run the whole workload on ``device``; returns a dict with pools, tables, output and counters.

    ``on_prefill(slots)`` and ``on_step(step, seqs, pairs, k, v)`` let a caller
    observe what was written (tests build their independent model from them).
    """
    w = inp.workload
    P, n, L = w.num_prompts, w.samples_per_prompt, w.prompt_len
    H, d, bs = w.num_heads, w.head_dim, w.block_size
    seqs = list(range(P * n))
    bm = BlockManager(w.num_blocks, bs, inp.free_list)
    k_cache = torch.full((w.num_blocks, H, bs, d), 0x7F, dtype=torch.uint8, device=device)   # NaN codes
    v_cache = torch.full((w.num_blocks, H, bs, d), 0x7F, dtype=torch.uint8, device=device)
    # one fp32 scale per pool: the prompt's largest magnitude maps to the largest E4M3 value
    k_scale = float((inp.prompt_k.abs().max().float() / 448.0).item())
    v_scale = float((inp.prompt_v.abs().max().float() / 448.0).item())

    slots = []
    for p in range(P):
        slots += bm.add_sequence(p * n, L)
    slot_t = torch.tensor(slots, dtype=torch.int64, device=device)
    ops.reshape_and_cache(inp.prompt_k.reshape(P * L, H, d), inp.prompt_v.reshape(P * L, H, d),
                          k_cache, v_cache, slot_t, k_scale=k_scale, v_scale=v_scale)
    if on_prefill:
        on_prefill(slots)
    for p in range(P):
        for c in range(1, n):
            bm.fork(p * n, p * n + c)

    n_pairs = 0
    steps = int(inp.cont_lens.max()) if len(inp.cont_lens) else 0
    for step in range(steps):
        active = [s for s in seqs if inp.cont_lens[s] > step]
        pairs, step_slots = [], []
        for s in active:
            slot, pair = bm.append_slot(s)
            step_slots.append(slot)
            if pair is not None:
                pairs.append(pair)
        k, v = synth.draw_step_kv(inp, len(active), device)
        if pairs:
            ops.copy_blocks(k_cache, v_cache, torch.tensor(pairs, dtype=torch.int64, device=device))
            n_pairs += len(pairs)
        ops.reshape_and_cache(k, v, k_cache, v_cache, torch.tensor(step_slots, dtype=torch.int64, device=device),
                              k_scale=k_scale, v_scale=v_scale)
        if on_step:
            on_step(step, active, pairs, k, v)

    tables = bm.block_table_array(seqs, w.max_blocks_per_seq)
    ctx = bm.context_lens_array(seqs)
    q = synth.draw_query(inp, len(seqs), device)
    out = torch.empty_like(q)
    ops.paged_attention_decode(out, q, k_cache, v_cache, torch.from_numpy(tables).to(device),
                               torch.from_numpy(ctx).to(device), w.softmax_scale, int(ctx.max()),
                               k_scale=k_scale, v_scale=v_scale,
                               seq_order=torch.from_numpy(bm.longest_first(seqs, group_shared=True)).to(device))
    return {
        "block_manager": bm, "k_cache": k_cache, "v_cache": v_cache, "k_scale": k_scale, "v_scale": v_scale,
        "tables": tables, "context_lens": ctx, "q": q, "out": out, "cow_pairs": n_pairs,
        "unique_blocks": int(np.count_nonzero(bm.refcount)), "logical_blocks": int(sum(len(t) for t in bm.tables.values())),
    }
