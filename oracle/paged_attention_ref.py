"""Plain CPU definition of the paged-KV decode path.  TEST INFRASTRUCTURE ONLY.

Every function is the definition written out in numpy / float64, slow and
obvious on purpose.  Citation labels are defined in ``oracle/__init__.py``:
[KVpag] "KV cache paginado e batching contínuo para LLMs", "Como funciona";
[PA/paging], [PA/sharing], [PA/related] the "PagedAttention" glossary page's
sections on paging, block sharing and related techniques.

Readings where the pages leave a step open (each is also listed in the design
notes of the repository):

* Pool layout: ``pool[block, kv_head, slot, dim]``.  The worked example on
  [PA/paging] uses ``pool[block, slot, dim]`` for one head; the kv-head axis is
  put right after the block axis so each (block, head) tile is the page's
  ``[slot, dim]`` block.  All indexing goes through ``_tile`` below.
* Query / output layout ``[seq, head, dim]``; head h reads kv head
  ``h // (num_heads // num_kv_heads)`` (contiguous groups, [PA/related] only
  says heads share K/V).
* ``context_lens[s]`` counts every cached token the new query attends to,
  including the new token itself; no causal mask is needed for one query token.
  A sequence with zero context attends to nothing and its output is zero.
* Table entries past ceil(ctx / block_size) and slots past ctx in the last
  block are never read.
* A flat slot number is ``block * block_size + offset`` (from the worked
  example's ``pool[table[pos // bs], pos % bs]`` write); a negative slot means
  "no write" (padding).
* Scale multiplies the dot product; softmax is the max-subtracted definition.
* copy_blocks copies whole blocks, every kv head and every slot; destination
  ids are distinct and disjoint from source ids, so pair order does not matter.
"""

import math

import numpy as np


# ---------------------------------------------------------------------------
# Block bookkeeping ([KVpag]; [PA/paging] worked example)
# ---------------------------------------------------------------------------

def blocks_needed(n_tokens, block_size):
    """Number of blocks a request of ``n_tokens`` occupies: ceil(n / block_size).

    [PA/paging]: a new block is taken only when the last one is full, so a
    request holds exactly ceil(n / block_size) blocks (40 tokens at 16 -> 3).
    """
    if n_tokens < 0 or block_size <= 0:
        raise ValueError("n_tokens must be >= 0 and block_size > 0")
    full, rest = divmod(n_tokens, block_size)
    return full + (1 if rest else 0)            # a partly filled last block still takes a block


def take_blocks(free_list, n):
    """Take ``n`` blocks from the front of ``free_list`` (mutates it), in order.

    [PA/paging] worked example: the table records the blocks in the order they
    were taken from the (scattered) free list.
    """
    if n > len(free_list):
        raise RuntimeError("out of free blocks")
    taken = list(free_list[:n])
    del free_list[:n]
    return taken


def slot_of(block_table, pos, block_size):
    """Flat slot of token ``pos``: table[pos // bs] * bs + pos % bs ([PA/paging] example)."""
    return int(block_table[pos // block_size]) * block_size + pos % block_size


def _tile(pool, block, kv_head):
    """The ``[block_size, head_dim]`` tile of one (block, kv head) -- the only layout-aware line."""
    return pool[block, kv_head]


def gather_tokens(pool, block_table, n_tokens, block_size, kv_head):
    """Rows of one sequence in logical order, read through its block table.

    [PA/paging]: attention reads keys and values back block by block through
    the table; token t lives in block table[t // bs] at offset t % bs.
    Returns an array ``[n_tokens, head_dim]`` with the pool's dtype.
    """
    d = pool.shape[-1]
    out = np.empty((n_tokens, d), dtype=pool.dtype)
    for t in range(n_tokens):
        b = int(block_table[t // block_size])
        out[t] = _tile(pool, b, kv_head)[t % block_size]
    return out


# ---------------------------------------------------------------------------
# Attention for the one new query token (plain definition, float64)
# ---------------------------------------------------------------------------

def attend_one_ref(q_vec, keys, values, scale):
    """softmax(scale * keys @ q) @ values for one head, max-subtracted, float64.

    logits_t = scale * <q, K_t>;  m = max_t logits_t;  w_t = exp(logits_t - m);
    out = sum_t w_t V_t / sum_t w_t.  Zero tokens -> zero vector.
    """
    q_vec = np.asarray(q_vec, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if keys.shape[0] == 0:
        return np.zeros(values.shape[-1], dtype=np.float64)
    logits = float(scale) * (keys @ q_vec)
    m = np.max(logits)
    w = np.exp(logits - m)
    return (w @ values) / np.sum(w)


def attend_ref(q, k_pool, v_pool, block_tables, context_lens, scale, block_size):
    """Decode attention of every (sequence, query head) over its paged context.

    ``q``: ``[S, H, d]``; ``k_pool``/``v_pool``: ``[NB, KVH, bs, d]`` holding the
    stored values already dequantised to float64 (for an FP8 cache use
    ``dequant_e4m3``); ``block_tables``: ``[S, maxblk]``; ``context_lens``: ``[S]``.
    Returns ``[S, H, d]`` float64.
    """
    q = np.asarray(q, dtype=np.float64)
    S, H, d = q.shape
    KVH = k_pool.shape[1]
    if H % KVH != 0:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    group = H // KVH
    out = np.zeros((S, H, d), dtype=np.float64)
    for s in range(S):
        ctx = int(context_lens[s])
        for g in range(KVH):
            keys = gather_tokens(k_pool, block_tables[s], ctx, block_size, g)
            vals = gather_tokens(v_pool, block_tables[s], ctx, block_size, g)
            for h in range(g * group, (g + 1) * group):
                out[s, h] = attend_one_ref(q[s, h], keys, vals, scale)
    return out


# ---------------------------------------------------------------------------
# Split-context identity (the partition-plus-merge form of the same result)
# ---------------------------------------------------------------------------

def partial_state_ref(q_vec, keys, values, scale):
    """(m, l, o) of one context slice: max logit, sum of exp(logit - m), unnormalised sum of weights * V.

    FlashAttention-style tiling ([PA/related]) never forms the full score row;
    a slice is summarised by these three quantities.  An empty slice is
    (-inf, 0, 0).
    """
    q_vec = np.asarray(q_vec, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if keys.shape[0] == 0:
        return -math.inf, 0.0, np.zeros(values.shape[-1])
    logits = float(scale) * (keys @ q_vec)
    m = float(np.max(logits))
    w = np.exp(logits - m)
    return m, float(np.sum(w)), w @ values


def merge_partials_ref(states):
    """Merge slice summaries: M = max m_p; out = sum e^(m_p-M) o_p / sum e^(m_p-M) l_p."""
    finite = [st for st in states if st[0] != -math.inf]
    if not finite:
        return np.zeros_like(states[0][2]) if states else None
    M = max(st[0] for st in finite)
    num = sum(math.exp(m - M) * o for m, _, o in finite)
    den = sum(math.exp(m - M) * l for m, l, _ in finite)
    return num / den


# ---------------------------------------------------------------------------
# Cache writes and block copies (byte-exact definitions)
# ---------------------------------------------------------------------------

def reshape_ref(key, value, k_pool, v_pool, slot_mapping, block_size, encode=None):
    """Scatter each token's K/V into its slot; return new pools (inputs untouched).

    For token i with slot sigma = slot_mapping[i] >= 0:
      pool[sigma // bs, h, sigma % bs, :] = encode(key[i, h, :])  for every kv head h
    (the worked example's ``pool[table[pos // bs], pos % bs] = key`` write).
    ``encode`` is the identity for a same-dtype cache (a bit copy of the
    source's stored bits); for an FP8 cache pass a function mapping a ``[KVH, d]``
    float array to uint8 codes.
    """
    k_new = np.array(k_pool, copy=True)
    v_new = np.array(v_pool, copy=True)
    for i, sigma in enumerate(np.asarray(slot_mapping).tolist()):
        if sigma < 0:
            continue
        b, o = sigma // block_size, sigma % block_size
        kr = key[i] if encode is None else encode(key[i])
        vr = value[i] if encode is None else encode(value[i])
        for h in range(k_new.shape[1]):
            _tile(k_new, b, h)[o] = kr[h]
            _tile(v_new, b, h)[o] = vr[h]
    return k_new, v_new


def copy_ref(k_pool, v_pool, pairs):
    """Copy-on-write block copy: for each (src, dst), block dst becomes a copy of block src.

    [KVpag] / [PA/sharing]: before writing into a block other sequences still
    use, the engine takes a new block and copies the old one into it (all kv
    heads, all slots).  Sources are read from the pools as given.
    """
    k_new = np.array(k_pool, copy=True)
    v_new = np.array(v_pool, copy=True)
    for src, dst in np.asarray(pairs).reshape(-1, 2).tolist():
        k_new[dst] = k_pool[src]
        v_new[dst] = v_pool[src]
    return k_new, v_new


def swap_ref(src_k, src_v, dst_k, dst_v, pairs):
    """Block copies between two pools (swap-out to host memory, swap-in back).

    [KVpag]: when physical blocks run out, the most recent requests are
    preempted whole and their blocks are recovered by swapping them to CPU
    memory (and later back).  For each (src, dst): destination block dst becomes
    a copy of source block src (all kv heads, all slots); the source pools are
    not changed.  Returns the new destination pools.
    """
    k_new = np.array(dst_k, copy=True)
    v_new = np.array(dst_v, copy=True)
    for src, dst in np.asarray(pairs).reshape(-1, 2).tolist():
        k_new[dst] = src_k[src]
        v_new[dst] = src_v[src]
    return k_new, v_new


def prefill_ref(q, k_pool, v_pool, block_tables, context_lens, query_start_loc, scale, block_size):
    """Chunked prefill attention over paged K/V, float64.

    [vLLM-rev] (feature list): the prefill of a long prompt is split into chunks,
    so each chunk's queries attend to the context cached by earlier chunks as
    well as to the chunk itself.  Reading taken: sequence s contributes
    ``n = query_start_loc[s+1] - query_start_loc[s]`` query tokens (rows
    ``query_start_loc[s] ..`` of ``q``), which are its last n positions;
    ``context_lens[s]`` counts every cached token including the chunk (whose K/V
    were written into the pool first).  Query i sits at position
    ``p = context_lens[s] - n + i`` and attends to positions 0..p (causal); a
    negative p (more queries than tokens) gives a zero row.  Grouped heads as in
    ``attend_ref``.  ``q``: ``[T, H, d]``; returns ``[T, H, d]``.
    """
    q = np.asarray(q, dtype=np.float64)
    T, H, d = q.shape
    KVH = k_pool.shape[1]
    if H % KVH != 0:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    group = H // KVH
    qsl = np.asarray(query_start_loc)
    out = np.zeros((T, H, d), dtype=np.float64)
    for s in range(len(context_lens)):
        ctx = int(context_lens[s])
        first, last = int(qsl[s]), int(qsl[s + 1])
        n = last - first
        for g in range(KVH):
            keys = gather_tokens(k_pool, block_tables[s], ctx, block_size, g)
            values = gather_tokens(v_pool, block_tables[s], ctx, block_size, g)
            for i in range(n):
                pos = ctx - n + i
                if pos < 0:
                    continue
                for h in range(g * group, (g + 1) * group):
                    out[first + i, h] = attend_one_ref(q[first + i, h], keys[:pos + 1], values[:pos + 1], scale)
    return out
