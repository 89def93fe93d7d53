"""The byte and flop accounting bench.py reports, against brute-force counts (CPU).

Each figure is recounted by walking the tokens, (query, key) pairs or physical
blocks one by one, so a wrong factor, a dropped term or a ceiling taken the
wrong way fails here before it skews a roofline.
"""

import subprocess
import sys
from types import SimpleNamespace

import numpy as np

import bench


def test_algorithmic_bytes_by_walking_the_tokens():
    w = SimpleNamespace(num_seqs=3, num_heads=6, num_kv_heads=2, head_dim=8, block_size=4)
    ctx = np.array([5, 8, 1], np.int64)
    elt_q, elt_kv = 2, 1
    kv = tables = 0
    for n in ctx:
        for t in range(n):
            kv += w.num_kv_heads * w.head_dim * elt_kv * 2        # K and V of token t, every kv head
            if t % w.block_size == 0:
                tables += 4                                         # one int32 table entry per block
    qo = w.num_seqs * w.num_heads * w.head_dim * elt_q * 2          # q read, out written
    lens = 4 * w.num_seqs
    got_kv, got_total = bench.algorithmic_bytes(w, ctx, elt_q, elt_kv)
    assert got_kv == kv
    assert got_total == kv + qo + tables + lens


def test_prefill_flops_by_walking_the_pairs():
    w = SimpleNamespace(num_heads=3, head_dim=16)
    ctx = np.array([7, 12, 5], np.int64)
    chunk = np.array([3, 12, 1], np.int64)                          # 12 = a whole prompt in one chunk
    pairs = 0
    for c, n in zip(ctx, chunk):
        for i in range(n):
            pos = c - n + i                                         # query i's position
            pairs += sum(1 for k in range(c) if k <= pos)          # causal: keys up to itself
    assert bench.prefill_flops(w, ctx, chunk) == 4 * w.head_dim * w.num_heads * pairs


def test_unique_kv_bytes_counts_each_physical_block_once():
    bs = 4
    # three forks of one prompt: the full blocks 10, 11 are shared, each fork owns the rest
    tables = np.array([[10, 11, 20, -1], [10, 11, 21, -1], [10, 11, 22, 23]], np.int32)
    ctx = np.array([9, 12, 15], np.int64)
    row = 64
    used = {}
    for s in range(3):
        for t in range(ctx[s]):
            b = int(tables[s, t // bs])
            used.setdefault(b, set()).add(t % bs)
    want = sum(len(v) for v in used.values()) * row
    assert bench.unique_kv_bytes(tables, ctx, bs, row) == want
    assert want < int(ctx.sum()) * row                              # sharing: fewer than the logical bytes


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True,
                       cwd=bench.ROOT, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stdout
