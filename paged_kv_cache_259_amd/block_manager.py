"""Host-side block bookkeeping that feeds the paged kernels.

The library's kernels are stateless: they move bytes and attend.  Deciding which
physical block holds which tokens is host work, done here:

* a pool of ``num_blocks`` fixed-size blocks, handed out from a free list in
  list order ("from anywhere free" -- [PA/paging], "PagedAttention" glossary,
  section "Cách phân trang hoạt động");
* one block table per sequence recording its blocks in logical order;
* a new block only when the sequence's last block is full, so unused slots are
  confined to the last block ([KVpag], "KV cache paginado e batching contínuo
  para LLMs", section "Como funciona");
* a reference count per block; forking a sequence shares every block
  (count + 1, no data moves);
* copy-on-write: a sequence about to write into a partly filled last block whose
  count is above 1 takes a fresh block, records the (source, destination) pair
  for ``copy_blocks``, drops the source's count by one and points its table at
  the fresh block ([KVpag]; [PA/sharing], section "Chia sẻ block giữa các
  chuỗi").  Sequences are served in the order the caller asks; the last holder
  of a shared block writes in place because its count has dropped to 1.

With ``prefix_cache=True`` full blocks are also shared across requests: a full
block is identified by its tokens and, through a chained key, by every token
before it ([PA/sharing]: hashing whole blocks extends sharing across requests
-- prompt caching; [vLLM-rev] feature list: prefix caching).  A request whose
prompt starts with cached blocks points its table at them (reference count + 1)
and only the remaining tokens need K/V written.  A cached block whose count
drops to 0 keeps its contents and key until the free list is empty; then the
least recently released one is reused.  A lookup compares the stored parent key
and tokens exactly, so a hash collision can only cause a miss.

Running out of blocks raises ``OutOfBlocks``.  Preemption is the caller's
decision; ``preemption_victims`` gives the order the pages describe (requests
served first come, first served; the most recent ones are preempted first, all
or nothing -- [KVpag]), and ``swap_out`` / ``swap_in`` move a preempted group's
blocks to a second, host-side pool and back, returning the (src, dst) pairs for
``swap_blocks``.
"""

from collections import OrderedDict, deque

import numpy as np


class OutOfBlocks(RuntimeError):
    pass


class BlockManager:
    def __init__(self, num_blocks, block_size, free_list=None, num_host_blocks=0, prefix_cache=False):
        if num_blocks <= 0 or block_size <= 0 or num_host_blocks < 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = range(num_blocks) if free_list is None else free_list
        self._free = deque(int(b) for b in order)
        if len(set(self._free)) != len(self._free) or any(not 0 <= b < num_blocks for b in self._free):
            raise ValueError("free list must hold distinct ids in [0, num_blocks)")
        self.refcount = np.zeros(self.num_blocks, dtype=np.int64)
        self.tables = {}
        self.lengths = {}
        # host-side pool for swapped-out sequences
        self.num_host_blocks = int(num_host_blocks)
        self._host_free = deque(range(self.num_host_blocks))
        self.host_refcount = np.zeros(self.num_host_blocks, dtype=np.int64)
        self.swapped = {}          # seq -> host block table (lengths stay in self.lengths)
        # prefix cache: key -> block, block -> (key, parent key, tokens), released cached blocks (LRU order)
        self.prefix_cache = bool(prefix_cache)
        self._cached = {}
        self._block_key = {}
        self._evictable = OrderedDict()

    # -- allocation ---------------------------------------------------------
    def _take(self):
        if self._free:
            b = self._free.popleft()
        elif self._evictable:                   # reuse the least recently released cached block
            b, _ = self._evictable.popitem(last=False)
            key = self._block_key.pop(b)[0]
            if self._cached.get(key) == b:
                del self._cached[key]
        else:
            raise OutOfBlocks("no free physical block left")
        self.refcount[b] = 1
        return b

    def _release(self, b):
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            if b in self._block_key:            # keep the contents for a later prefix hit
                self._evictable[b] = None
            else:
                self._free.append(b)

    def num_free(self):
        """Blocks available to allocations (free, plus released cached blocks)."""
        return len(self._free) + len(self._evictable)

    def add_sequence(self, seq, n_tokens=0):
        """Register ``seq`` holding ``n_tokens`` tokens; returns the flat slots of those tokens."""
        if seq in self.tables:
            raise KeyError(f"sequence {seq} already exists")
        self.tables[seq] = []
        self.lengths[seq] = 0
        return [self.append_slot(seq)[0] for _ in range(n_tokens)]

    def add_sequence_cached(self, seq, token_ids):
        """Register ``seq`` with its prompt, reusing cached full blocks of a matching prefix.

        Returns ``(slots, cached)``: ``cached`` leading tokens already have their
        K/V in the pool (whole blocks, a multiple of block_size); ``slots`` are
        the flat slots of tokens ``cached ..`` that the caller must write.  The
        new full blocks are registered in the cache (their contents are the
        caller's writes, issued before any later reader runs).
        """
        if not self.prefix_cache:
            raise RuntimeError("prefix cache not enabled")
        if seq in self.tables:
            raise KeyError(f"sequence {seq} already exists")
        tokens = [int(t) for t in token_ids]
        bs = self.block_size
        table, parent, cached, hit = [], None, 0, True
        for j in range(len(tokens) // bs):
            blk_tokens = tuple(tokens[j * bs:(j + 1) * bs])
            key = hash((parent, blk_tokens))
            b = self._cached.get(key) if hit else None
            if b is not None and self._block_key[b] == (key, parent, blk_tokens):
                if self.refcount[b] == 0:
                    del self._evictable[b]
                self.refcount[b] += 1
                cached += bs
            else:
                hit = False                     # the cached part is a prefix: stop at the first miss
                b = self._take()
                old = self._cached.get(key)
                if old is None or self.refcount[old] == 0:
                    self._cached[key] = b
                self._block_key[b] = (key, parent, blk_tokens)
            table.append(b)
            parent = key
        if len(tokens) % bs:
            table.append(self._take())          # the partial last block is private
        self.tables[seq] = table
        self.lengths[seq] = len(tokens)
        return [table[p // bs] * bs + p % bs for p in range(cached, len(tokens))], cached

    def cached_blocks(self):
        """Blocks currently registered in the prefix cache."""
        return len(self._block_key)

    def append_slot(self, seq):
        """Reserve the slot of ``seq``'s next token.

        Returns ``(slot, cow_pair)``: ``slot`` is block * block_size + offset and
        ``cow_pair`` is ``(src, dst)`` when the write needs a block copy first,
        else ``None``.
        """
        table = self.tables[seq]
        pos = self.lengths[seq]
        bs = self.block_size
        pair = None
        if pos % bs == 0:                       # no block yet, or the last one is full
            table.append(self._take())
        else:
            last = table[-1]
            if self.refcount[last] > 1:         # shared partial block -> copy on write
                fresh = self._take()
                self.refcount[last] -= 1
                table[-1] = fresh
                pair = (last, fresh)
        self.lengths[seq] = pos + 1
        return table[pos // bs] * bs + pos % bs, pair

    def fork(self, parent, child):
        """``child`` shares every block of ``parent`` (reference counts + 1)."""
        if child in self.tables:
            raise KeyError(f"sequence {child} already exists")
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for b in self.tables[child]:
            self.refcount[b] += 1

    def free_sequence(self, seq):
        if seq in self.swapped:
            for h in self.swapped.pop(seq):
                self.host_refcount[h] -= 1
                if self.host_refcount[h] == 0:
                    self._host_free.append(h)
        else:
            for b in self.tables.pop(seq):
                self._release(b)
        del self.lengths[seq]

    # -- preemption by swapping -----------------------------------------------
    @staticmethod
    def preemption_victims(groups_by_arrival, blocks_needed, blocks_held, num_free):
        """Groups to preempt, most recent arrival first, until ``blocks_needed`` blocks are free.

        ``groups_by_arrival``: running groups in arrival order (each a tuple of
        sequences that share blocks, e.g. the samples of one prompt);
        ``blocks_held(group)``: GPU blocks freed by preempting that group.  A
        group is preempted whole or not at all.  Raises ``OutOfBlocks`` when even
        preempting every group would not free enough.
        """
        victims, free = [], num_free
        for g in reversed(list(groups_by_arrival)):
            if free >= blocks_needed:
                break
            victims.append(g)
            free += blocks_held(g)
        if free < blocks_needed:
            raise OutOfBlocks(f"{blocks_needed} blocks needed, at most {free} can be freed")
        return victims

    def group_blocks(self, seqs):
        """Distinct GPU blocks held by ``seqs``; raises if one is shared with a sequence outside."""
        seqs = list(seqs)
        holders = {}
        for s in seqs:
            for b in self.tables[s]:
                holders[b] = holders.get(b, 0) + 1
        for b, n in holders.items():
            if self.refcount[b] != n:
                raise ValueError(f"block {b} is shared with a sequence outside the group")
        return holders

    def swap_out(self, seqs):
        """Move every block of the group ``seqs`` to the host pool.

        Returns ``(gpu_block, host_block)`` pairs, one per distinct block (a block
        shared inside the group is copied once and stays shared on the host).
        The GPU blocks return to the free list.
        """
        seqs = list(seqs)
        holders = self.group_blocks(seqs)
        if len(holders) > len(self._host_free):
            raise OutOfBlocks("no room in the host pool")
        to_host = {}
        for b in holders:                       # first-use order of the group's tables
            h = self._host_free.popleft()
            to_host[b] = h
            self.host_refcount[h] = holders[b]
        for s in seqs:
            self.swapped[s] = [to_host[b] for b in self.tables.pop(s)]
        for b in holders:
            self.refcount[b] = 1
            self._release(b)                    # cached blocks stay reusable until overwritten
        return list(to_host.items())

    def swap_in(self, seqs):
        """Bring the swapped-out group ``seqs`` back; returns ``(host_block, gpu_block)`` pairs."""
        seqs = list(seqs)
        holders = {}
        for s in seqs:
            for h in self.swapped[s]:
                holders[h] = holders.get(h, 0) + 1
        for h, n in holders.items():
            if self.host_refcount[h] != n:
                raise ValueError(f"host block {h} is shared with a sequence outside the group")
        if len(holders) > len(self._free):
            raise OutOfBlocks("not enough free GPU blocks to swap in")
        to_gpu = {}
        for h in holders:
            b = self._take()
            self.refcount[b] = holders[h]
            to_gpu[h] = b
        for s in seqs:
            self.tables[s] = [to_gpu[h] for h in self.swapped.pop(s)]
        for h in holders:
            self.host_refcount[h] = 0
            self._host_free.append(h)
        return list(to_gpu.items())

    # -- views for the kernels ---------------------------------------------
    def block_table_array(self, seqs, max_blocks_per_seq):
        """int32 ``[len(seqs), max_blocks_per_seq]``; unused entries are -1."""
        out = np.full((len(seqs), max_blocks_per_seq), -1, dtype=np.int32)
        for i, s in enumerate(seqs):
            t = self.tables[s]
            if len(t) > max_blocks_per_seq:
                raise ValueError(f"sequence {s} holds {len(t)} blocks > {max_blocks_per_seq}")
            out[i, :len(t)] = t
        return out

    def context_lens_array(self, seqs):
        return np.array([self.lengths[s] for s in seqs], dtype=np.int32)

    def longest_first(self, seqs, group_shared=False):
        """Positions 0..len(seqs)-1 ordered by decreasing context length (ties by position).

        A scheduling hint for the one-pass attention launch: long contexts start
        first.  Any permutation gives the same attention results.

        With ``group_shared``, sequences whose tables start with the same
        physical block (forks of one prompt) stay adjacent: groups are ordered
        by their longest member, members by length.  Their workgroups then run
        at about the same time and read each shared block close together, so
        the reads after the first can come from the cache instead of HBM.
        """
        lens = self.context_lens_array(seqs)
        if not group_shared:
            return np.argsort(-lens, kind="stable").astype(np.int32)
        first = [self.tables[s][0] if len(self.tables[s]) else -1 - i for i, s in enumerate(seqs)]
        group_len = {}
        for f, n in zip(first, lens):
            group_len[f] = max(group_len.get(f, 0), int(n))
        order = sorted(range(len(seqs)), key=lambda i: (-group_len[first[i]], first[i], -int(lens[i]), i))
        return np.array(order, dtype=np.int32)

    def kv_load_policy(self, seqs, repeat_share=1 / 16):
        """K/V load policy for one plain decode launch over ``seqs``: "cached" when
        at least ``repeat_share`` of the launch's block reads are repeats (a block
        already read by an earlier sequence of the launch: forks of one prompt,
        a cached system prompt), else "stream".

        Non-temporal ("stream") loads make a launch that reads every block once
        about 6 % faster; a repeated read finds the block in the caches only
        under "cached", where it costs no HBM traffic at all.  The policy
        changes no result.
        """
        reads = 0
        seen = set()
        for s in seqs:
            used = self.tables[s][:-(-self.lengths[s] // self.block_size)]
            reads += len(used)
            seen.update(used)
        repeats = reads - len(seen)
        return "cached" if reads and repeats >= repeat_share * reads else "stream"

    def shared_groups(self, seqs, max_group_size):
        """Groups for the shared-block decode: positions of ``seqs`` whose tables
        start with the same physical block, in chunks of at most ``max_group_size``.

        Returns int32 arrays ``(offsets [G+1], members [len(seqs)], shared [G])``:
        group g is ``members[offsets[g]:offsets[g+1]]`` and its first ``shared[g]``
        table entries are the same physical blocks in every member (the longest
        common prefix of their tables, lowered so that no member's newest token
        falls inside it).  A sequence that shares nothing is a group of one with
        0 shared blocks.  Groups are listed by decreasing work (blocks the
        group's workgroups read), longest first, like ``longest_first``.
        """
        if max_group_size < 1:
            raise ValueError("max_group_size must be at least 1")
        bs = self.block_size
        buckets = {}
        for i, s in enumerate(seqs):
            t = self.tables[s]
            key = t[0] if len(t) else ("empty", i)
            buckets.setdefault(key, []).append(i)
        groups = []
        for members in buckets.values():
            # similar lengths together, so a chunk's members finish their own blocks at similar times
            members = sorted(members, key=lambda i: (-self.lengths[seqs[i]], i))
            for c in range(0, len(members), max_group_size):
                chunk = members[c:c + max_group_size]
                tabs = [self.tables[seqs[i]] for i in chunk]
                lcp = min(len(t) for t in tabs)
                for j in range(lcp):
                    if any(t[j] != tabs[0][j] for t in tabs[1:]):
                        lcp = j
                        break
                cap = min(max(self.lengths[seqs[i]] - 1, 0) // bs for i in chunk)
                shared = min(lcp, cap) if len(chunk) > 1 else 0
                work = shared + sum(len(t) - shared for t in tabs)
                groups.append((work, chunk, shared))
        groups.sort(key=lambda g: (-g[0], g[1][0]))
        offsets = np.zeros(len(groups) + 1, dtype=np.int32)
        members = np.zeros(len(seqs), dtype=np.int32)
        shared = np.zeros(len(groups), dtype=np.int32)
        pos = 0
        for g, (_, chunk, sh) in enumerate(groups):
            members[pos:pos + len(chunk)] = chunk
            pos += len(chunk)
            offsets[g + 1] = pos
            shared[g] = sh
        return offsets, members, shared

    def slot(self, seq, pos):
        t = self.tables[seq]
        return t[pos // self.block_size] * self.block_size + pos % self.block_size

    def utilisation(self):
        """Tokens held / slots allocated over all distinct blocks in use."""
        used = int(np.count_nonzero(self.refcount))
        if used == 0:
            return 1.0
        # count each physical slot once even when shared
        filled = {}
        for s, t in self.tables.items():
            n = self.lengths[s]
            for j, b in enumerate(t):
                k = min(self.block_size, n - j * self.block_size)
                filled[b] = max(filled.get(b, 0), k)
        return sum(filled.values()) / (used * self.block_size)
