"""Never-paged model of every sequence's cache.  TEST INFRASTRUCTURE ONLY.

Each sequence keeps its keys and values as one plain array, appended one token
at a time; a fork copies the parent's arrays.  This is the "one contiguous
region per request" layout that [KVpag] ("KV cache paginado e batching
contínuo para LLMs", "Como funciona") describes as the prior design, used here
only as ground truth: the paged pool, read through each sequence's block
table, must hold exactly the same stored bytes, whatever blocks were shared or
copied on write ([PA/sharing], "PagedAttention" glossary, "Chia sẻ block giữa
các chuỗi").
"""

import numpy as np


class ContiguousSequences:
    """Per-sequence contiguous K/V rows; rows are ``[num_kv_heads, head_dim]`` arrays."""

    def __init__(self):
        self._k = {}
        self._v = {}

    def new(self, seq_id):
        if seq_id in self._k:
            raise KeyError(f"sequence {seq_id} exists")
        self._k[seq_id] = []
        self._v[seq_id] = []

    def append(self, seq_id, k_row, v_row):
        self._k[seq_id].append(np.array(k_row, copy=True))
        self._v[seq_id].append(np.array(v_row, copy=True))

    def extend(self, seq_id, k_rows, v_rows):
        for kr, vr in zip(k_rows, v_rows):
            self.append(seq_id, kr, vr)

    def fork(self, parent, child):
        """Child starts as an independent copy of the parent's rows."""
        if child in self._k:
            raise KeyError(f"sequence {child} exists")
        self._k[child] = [r.copy() for r in self._k[parent]]
        self._v[child] = [r.copy() for r in self._v[parent]]

    def length(self, seq_id):
        return len(self._k[seq_id])

    def keys(self, seq_id):
        """``[n, num_kv_heads, head_dim]`` array of the sequence's keys in order."""
        return np.stack(self._k[seq_id]) if self._k[seq_id] else None

    def values(self, seq_id):
        return np.stack(self._v[seq_id]) if self._v[seq_id] else None

    def ids(self):
        return list(self._k.keys())
