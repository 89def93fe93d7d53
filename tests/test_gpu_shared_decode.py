"""Decode over groups of sequences sharing leading blocks (pkv_paged_attention_decode_shared).

Samples forked from one prompt share its blocks; the shared-block decode reads
them once per group.  Its outputs are checked against the fp64 oracle walking
each sequence's own block table (the plain definition), and with append its
pools must come out bit-identical to pkv_paged_attention_decode_append's.
Groups come from BlockManager.shared_groups; edge cases: groups of one, more
samples than a group holds, a prompt ending on a block boundary, a one-token
prompt, a shared count above what the kernel allows.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_259_amd.block_manager import BlockManager
from tests.helpers import TOL, as_f64, check_close

pytestmark = pytest.mark.gpu
DEV = "cuda"
DT = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def ops():
    from paged_kv_cache_259_amd import ops as _ops
    return _ops


def forked_batch(rng, prompt_lens, n, cont_max, bs=16):
    """Prompts forked into n samples, each continued by 0..cont_max tokens, then
    the decode step's slots (copy-on-write pairs applied by the caller)."""
    S = len(prompt_lens) * n
    NB = sum(-(-L // bs) * n + -(-(cont_max + 1) // bs) * n + n for L in prompt_lens) + 8
    bm = BlockManager(NB, bs, free_list=rng.permutation(NB))
    pairs = []
    for p, L in enumerate(prompt_lens):
        bm.add_sequence(p * n, L)
        for c in range(1, n):
            bm.fork(p * n, p * n + c)
    for s in range(S):
        for _ in range(int(rng.integers(0, cont_max + 1))):
            pair = bm.append_slot(s)[1]
            if pair is not None:
                pairs.append(pair)
    slots = []
    for s in range(S):                       # the decode step's new token
        slot, pair = bm.append_slot(s)
        slots.append(slot)
        if pair is not None:
            pairs.append(pair)
    return bm, NB, list(range(S)), slots, pairs


CASES = [
    # name, q dtype, cache format, H, KVH, d, prompt lengths, samples, continuation max, group max
    ("f16 mha", "f16", None, 8, 8, 128, [40, 33, 100, 16, 1], 4, 40, 4),
    ("bf16 gqa2", "bf16", None, 8, 4, 128, [70, 200, 15], 3, 35, 8),
    ("e4m3 mha", "f16", "e4m3", 8, 8, 128, [1000, 64, 250], 4, 60, 4),
    ("e5m2 gqa4 d256 per head", "bf16", "e5m2", 8, 2, 256, [90, 48, 300], 4, 20, 4),
    ("bf16 six samples in chunks of four", "bf16", None, 4, 4, 128, [130, 47], 6, 30, 4),
    ("f16 groups of one", "f16", None, 4, 4, 128, [20, 300, 5, 64], 1, 10, 4),
    ("e4m3 gqa8 d128", "bf16", "e4m3", 16, 2, 128, [500, 31], 2, 100, 2),
]


def make_pools(rng, fmt, qdt, NB, KVH, d, bs):
    if fmt is None:
        k = torch.from_numpy(rng.standard_normal((NB, KVH, bs, d)).astype(np.float32)).to(DT[qdt])
        v = torch.from_numpy(rng.standard_normal((NB, KVH, bs, d)).astype(np.float32)).to(DT[qdt])
        return k, v, {}
    top = 0x7E if fmt == "e4m3" else 0x4B                   # E5M2 below 0x4B: |code| <= 14
    k = torch.from_numpy(rng.integers(0, top, (NB, KVH, bs, d)).astype(np.uint8))
    v = torch.from_numpy(rng.integers(0, top, (NB, KVH, bs, d)).astype(np.uint8))
    k |= torch.from_numpy((rng.integers(0, 2, k.shape) << 7).astype(np.uint8))   # random signs
    v |= torch.from_numpy((rng.integers(0, 2, v.shape) << 7).astype(np.uint8))
    if fmt == "e5m2":
        kw = dict(k_scales=torch.tensor(rng.uniform(0.01, 0.05, KVH), dtype=torch.float32, device=DEV),
                  v_scales=torch.tensor(rng.uniform(0.1, 1.0, KVH), dtype=torch.float32, device=DEV))
        return k.view(torch.float8_e5m2), v.view(torch.float8_e5m2), kw
    return k, v, dict(k_scale=0.04, v_scale=0.25)


def dequant(pool, fmt, kw, which):
    codes = pool.view(torch.uint8).cpu().numpy()
    if fmt == "e4m3":
        return oracle.dequant_e4m3(codes, kw[which + "_scale"])
    if fmt == "e5m2":
        return oracle.dequant_per_head(codes, kw[which + "_scales"].cpu().numpy(), oracle.decode_e5m2)
    return as_f64(pool)


@pytest.mark.parametrize("append", [False, True], ids=["plain", "append"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_shared_decode_matches_oracle(ops, case, append):
    name, qdt, fmt, H, KVH, d, plens, n, cmax, gmax = case
    bs = 16
    rng = np.random.default_rng(sum(ord(c) for c in name) + append)
    bm, NB, seqs, slots, pairs = forked_batch(rng, plens, n, cmax, bs)
    S = len(seqs)
    kc, vc, kw = make_pools(rng, fmt, qdt, NB, KVH, d, bs)
    if pairs:                                             # copy-on-write copies, as copy_blocks would do
        src = torch.tensor([a for a, _ in pairs])
        dst = torch.tensor([b for _, b in pairs])
        kc.view(torch.uint8)[dst] = kc.view(torch.uint8)[src]
        vc.view(torch.uint8)[dst] = vc.view(torch.uint8)[src]
    maxblk = max(len(bm.tables[s]) for s in seqs) + 2
    tables_np = bm.block_table_array(seqs, maxblk)
    ctx_np = bm.context_lens_array(seqs)
    offs, mem, shared = bm.shared_groups(seqs, gmax)
    assert sorted(mem.tolist()) == seqs
    if n > 1:
        assert shared.max() > 0 or max(plens) < bs
    q = torch.from_numpy(rng.standard_normal((S, H, d)).astype(np.float32)).to(DT[qdt]).to(DEV)
    key = torch.from_numpy(rng.standard_normal((S, KVH, d)).astype(np.float32)).to(DT[qdt]).to(DEV)
    val = torch.from_numpy(rng.standard_normal((S, KVH, d)).astype(np.float32)).to(DT[qdt]).to(DEV)
    slot_t = torch.tensor(slots, dtype=torch.int64, device=DEV)
    tables = torch.from_numpy(tables_np).to(DEV)
    ctx = torch.from_numpy(ctx_np).to(DEV)
    g = [torch.from_numpy(a).to(DEV) for a in (offs, mem, shared)]
    kA, vA = kc.to(DEV), vc.to(DEV)
    kB, vB = kA.clone(), vA.clone()
    out = torch.full_like(q, float("nan"))
    extra = dict(key=key, value=val, slot_mapping=slot_t) if append else {}
    ops.paged_attention_decode_shared(out, q, kB, vB, tables, ctx, *g, gmax, d ** -0.5, int(ctx_np.max()), **extra,
                                      **kw)
    if append:                                            # the pools: as the validated one-launch append writes them
        ref_out = torch.empty_like(q)
        ops.paged_attention_decode_append(ref_out, q, kA, vA, key, val, slot_t, tables, ctx, d ** -0.5,
                                          int(ctx_np.max()), **kw)
    torch.cuda.synchronize()
    if append:
        assert torch.equal(kA.view(torch.uint8), kB.view(torch.uint8)), "k_cache bytes differ"
        assert torch.equal(vA.view(torch.uint8), vB.view(torch.uint8)), "v_cache bytes differ"
    else:
        assert torch.equal(kB.view(torch.uint8).cpu(), kc.view(torch.uint8)), "a plain decode wrote the pool"
    ref = oracle.attend_ref(as_f64(q), dequant(kB, fmt, kw, "k"), dequant(vB, fmt, kw, "v"), tables_np, ctx_np,
                            d ** -0.5, bs)
    check_close(as_f64(out), ref, TOL["fp8_e4m3" if fmt else qdt], name)


def test_shared_count_above_the_limit_is_lowered(ops):
    """Sample 0's newest token sits in its second block (it writes there in place),
    so at most one block may be read as shared even if the caller says two."""
    bs, H, d = 16, 4, 128
    rng = np.random.default_rng(11)
    bm = BlockManager(16, bs, free_list=rng.permutation(16))
    bm.add_sequence(0, 31)
    bm.fork(0, 1)
    bm.append_slot(1)                                     # sample 1 copies block 1 (shared, partly filled)
    s0 = bm.append_slot(0)[0]                             # sample 0 now holds block 1 alone: writes in place
    s1 = bm.append_slot(1)[0]
    seqs = [0, 1]
    tables_np = bm.block_table_array(seqs, 4)
    ctx_np = bm.context_lens_array(seqs)
    assert ctx_np.tolist() == [32, 33]
    kc = torch.randn((16, H, bs, d)).half()
    vc = torch.randn((16, H, bs, d)).half()
    kc[tables_np[1, 1]] = kc[tables_np[0, 1]]             # the copy-on-write copy
    vc[tables_np[1, 1]] = vc[tables_np[0, 1]]
    q = torch.randn((2, H, d), device=DEV).half()
    key = torch.randn((2, H, d), device=DEV).half()
    val = torch.randn((2, H, d), device=DEV).half()
    k, v = kc.to(DEV), vc.to(DEV)
    out = torch.empty_like(q)
    g = [torch.tensor(a, dtype=torch.int32, device=DEV) for a in ([0, 2], [0, 1], [2])]   # 2: too many
    ops.paged_attention_decode_shared(out, q, k, v, torch.from_numpy(tables_np).to(DEV),
                                      torch.from_numpy(ctx_np).to(DEV), *g, 2, d ** -0.5, 33, key=key, value=val,
                                      slot_mapping=torch.tensor([s0, s1], device=DEV))
    torch.cuda.synchronize()
    assert bm.shared_groups(seqs, 2)[2].tolist() == [1]
    ref = oracle.attend_ref(as_f64(q), as_f64(k), as_f64(v), tables_np, ctx_np, d ** -0.5, bs)
    check_close(as_f64(out), ref, TOL["f16"], "lowered shared count")


def test_shared_decode_rejects_too_many_columns(ops):
    q = torch.zeros((4, 8, 128), device=DEV).half()
    pool = torch.zeros((4, 2, 16, 128), device=DEV).half()
    t = torch.zeros((4, 1), dtype=torch.int32, device=DEV)
    c = torch.ones(4, dtype=torch.int32, device=DEV)
    g = [torch.tensor(a, dtype=torch.int32, device=DEV) for a in ([0, 4], [0, 1, 2, 3], [0])]
    with pytest.raises(ops.PkvError):
        ops.paged_attention_decode_shared(torch.empty_like(q), q, pool, pool, t, c, *g, 5, 0.1, 1)   # 5 x 4 > 16


def test_shared_decode_xcd_orders_only_schedule(ops, monkeypatch):
    """16 heads: the shared-block decode takes the head-runs order; the hardware order
    and runs of n work ids give identical bits."""
    H, d, bs = 16, 128, 16
    rng = np.random.default_rng(21)
    bm, NB, seqs, slots, pairs = forked_batch(rng, [90, 33, 260], 4, 30, bs)
    kc, vc, _ = make_pools(rng, None, "f16", NB, H, d, bs)
    tables_np = bm.block_table_array(seqs, 32)
    ctx_np = bm.context_lens_array(seqs)
    g = [torch.from_numpy(a).to(DEV) for a in bm.shared_groups(seqs, 4)]
    q = torch.from_numpy(rng.standard_normal((len(seqs), H, d)).astype(np.float32)).half().to(DEV)
    k, v = kc.to(DEV), vc.to(DEV)
    tables, ctx = torch.from_numpy(tables_np).to(DEV), torch.from_numpy(ctx_np).to(DEV)

    def run():
        out = torch.empty_like(q)
        ops.paged_attention_decode_shared(out, q, k, v, tables, ctx, *g, 4, d ** -0.5, int(ctx_np.max()))
        torch.cuda.synchronize()
        return out

    base = run()
    ref = oracle.attend_ref(as_f64(q), as_f64(k), as_f64(v), tables_np, ctx_np, d ** -0.5, bs)
    check_close(as_f64(base), ref, TOL["f16"], "shared-block decode, head runs")
    for chunk in ("0", "8", "5"):
        monkeypatch.setenv("PKV_XCD_CHUNK", chunk)
        assert torch.equal(run().view(torch.int16), base.view(torch.int16)), f"PKV_XCD_CHUNK={chunk}"
