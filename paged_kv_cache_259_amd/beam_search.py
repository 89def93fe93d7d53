"""Beam-search block accounting on the host block manager.

Beam candidates share their common history's blocks through the block table,
with reference counts, and a beam that writes into a block another beam still
uses copies it first ("KV cache paginado e batching contínuo para LLMs", section
"Como funciona": sharing with reference counts and block-level copy-on-write;
"PagedAttention", Ultralytics glossary, section "Chia sẻ block giữa các chuỗi":
beam search reuses a shared prefix).  One step:

1. every new beam forks the beam it extends (all blocks shared, counts + 1);
2. the previous beams are released (counts - 1), so blocks no survivor uses
   return to the pool and the survivors share the rest;
3. every new beam reserves the slot of its next token; the first writers into a
   shared, partly filled last block get a fresh copy (a copy_blocks pair), the
   last one writes in place.

The kernels see only tables, context lengths, slots and copy pairs.
"""

import numpy as np


def beam_step(bm, beams, parents, next_id):
    """Advance a beam group one token.

    ``beams``: sequence ids of the current beams; ``parents[i]``: index in
    ``beams`` of the beam that new beam ``i`` extends (a beam may be extended by
    several new beams, or by none).  New sequence ids are ``next_id, next_id+1,
    ...``.  Returns ``(new_beams, slots, cow_pairs, next_id)``: ``slots[i]`` is
    where new beam ``i``'s token goes, ``cow_pairs`` the block copies to issue
    before writing.
    """
    new = []
    for p in parents:
        bm.fork(beams[p], next_id)
        new.append(next_id)
        next_id += 1
    for b in beams:
        bm.free_sequence(b)
    slots, pairs = [], []
    for sid in new:
        slot, pair = bm.append_slot(sid)
        slots.append(slot)
        if pair is not None:
            pairs.append(pair)
    return new, slots, pairs, next_id


def blocks_in_use(bm):
    """Distinct physical blocks held by any sequence."""
    return int(np.count_nonzero(bm.refcount))


def blocks_without_sharing(bm, seqs):
    """Blocks the same sequences would hold with private copies of every block."""
    bs = bm.block_size
    return int(sum(-(-bm.lengths[s] // bs) for s in seqs))
