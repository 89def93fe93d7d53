"""Pins of the CPU oracle to facts fixed outside the oracle itself (CPU only).

Each test names what it pins and where the fact comes from: a value the pages
print (fixtures under tests/golden/), a library routine that computes the same
definition by another route, a closed form, or brute force on tiny inputs.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3_ref
from oracle.paged_attention_ref import (
    swap_ref, prefill_ref,
    attend_one_ref, attend_ref, blocks_needed, copy_ref, gather_tokens,
    merge_partials_ref, partial_state_ref, reshape_ref, slot_of, take_blocks,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Worked example of the glossary page (paging section): values it prints
# ---------------------------------------------------------------------------

def test_worked_example_table_gather_and_waste():
    g = _golden("worked_example.json")
    bs, d, nb, n = g["block_size"], g["head_dim"], g["pool_blocks"], g["request_tokens"]
    free = list(g["free_blocks"])
    keys = torch.randn(n, d, generator=torch.Generator().manual_seed(0)).numpy()
    pool = np.zeros((nb, 1, bs, d), dtype=np.float32)          # one kv head
    table = take_blocks(free, blocks_needed(n, bs))
    assert table == g["expected_block_table"]
    assert free == [2, 33]
    slots = [slot_of(table, pos, bs) for pos in range(n)]
    pool_k, _ = reshape_ref(keys[:, None, :], keys[:, None, :], pool, pool, np.array(slots), bs)
    gathered = gather_tokens(pool_k, table, n, bs, 0)
    assert np.array_equal(gathered, keys) == g["expected_keys_intact"]
    assert len(table) * bs - n == g["expected_unused_slots_paged"]
    assert g["reservation_tokens"] - n == g["expected_unused_slots_reserved"]


def test_tiny_workload_block_count():
    # 40, 17, 1 and 64 tokens at block size 16 take 3 + 2 + 1 + 4 blocks
    assert [blocks_needed(c, 16) for c in (40, 17, 1, 64)] == [3, 2, 1, 4]
    assert sum(blocks_needed(c, 16) for c in (40, 17, 1, 64)) == 10


@pytest.mark.parametrize("bs", [1, 8, 16, 32])
def test_waste_confined_to_last_block(bs):
    for n in range(0, 300):
        nb = blocks_needed(n, bs)
        waste = nb * bs - n
        assert 0 <= waste < bs                       # less than one block
        assert waste == (-n) % bs
        if nb:
            assert (nb - 1) * bs < n <= nb * bs       # every block but the last is full


def test_llama13b_bytes_per_sequence():
    g = _golden("llama13b_kv_bytes.json")
    s = g["model_shape_reading"]
    per_token = 2 * s["layers"] * s["heads"] * s["head_dim"] * s["bytes_per_element"]
    total = per_token * g["tokens"]
    assert abs(total - g["approx_bytes_per_sequence"]) <= g["rounding"]


def test_fp8_pool_is_half_of_fp16_pool():
    shape = (10, 4, 16, 128)
    assert np.zeros(shape, np.uint8).nbytes * 2 == np.zeros(shape, np.float16).nbytes


# ---------------------------------------------------------------------------
# Attention: library routine, closed forms, special cases, brute force
# ---------------------------------------------------------------------------

def _rand_case(seed, S, H, KVH, d, bs, lens, nb):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((S, H, d))
    kp = rng.standard_normal((nb, KVH, bs, d))
    vp = rng.standard_normal((nb, KVH, bs, d))
    perm = rng.permutation(nb).tolist()
    maxblk = max(blocks_needed(c, bs) for c in lens)
    tables = np.full((S, maxblk), -1, np.int64)
    for s, c in enumerate(lens):
        t = take_blocks(perm, blocks_needed(c, bs))
        tables[s, :len(t)] = t
    return q, kp, vp, tables, np.array(lens)


def _sdpa(q_vec, keys, values, scale):
    """torch's scaled_dot_product_attention on CPU float64, one query row."""
    qq = torch.from_numpy(np.asarray(q_vec, np.float64))[None, None, None, :]
    kk = torch.from_numpy(np.asarray(keys, np.float64))[None, None]
    vv = torch.from_numpy(np.asarray(values, np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)[0, 0, 0].numpy()


@pytest.mark.parametrize("seed,H,KVH,d,bs,lens", [
    (1, 2, 2, 8, 4, [5, 1, 9]),
    (2, 4, 1, 16, 16, [40, 17, 33]),
    (3, 8, 2, 4, 2, [3, 7]),
])
def test_attend_matches_torch_sdpa(seed, H, KVH, d, bs, lens):
    nb = sum(blocks_needed(c, bs) for c in lens) + 3
    q, kp, vp, tables, ctx = _rand_case(seed, len(lens), H, KVH, d, bs, lens, nb)
    scale = 1.0 / math.sqrt(d)
    out = attend_ref(q, kp, vp, tables, ctx, scale, bs)
    G = H // KVH
    for s in range(len(lens)):
        for h in range(H):
            K = gather_tokens(kp, tables[s], ctx[s], bs, h // G)
            V = gather_tokens(vp, tables[s], ctx[s], bs, h // G)
            np.testing.assert_allclose(out[s, h], _sdpa(q[s, h], K, V, scale), rtol=1e-12, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv_heads():
    S, H, KVH, d, bs, lens = 3, 8, 2, 8, 4, [6, 11, 1]
    nb = 12
    q, kp, vp, tables, ctx = _rand_case(7, S, H, KVH, d, bs, lens, nb)
    out_gqa = attend_ref(q, kp, vp, tables, ctx, 0.3, bs)
    kp_rep = torch.from_numpy(kp).repeat_interleave(H // KVH, dim=1).numpy()
    vp_rep = torch.from_numpy(vp).repeat_interleave(H // KVH, dim=1).numpy()
    out_mha = attend_ref(q, kp_rep, vp_rep, tables, ctx, 0.3, bs)
    np.testing.assert_array_equal(out_gqa, out_mha)


def test_any_block_permutation_gives_the_same_output():
    """Paged output equals contiguous attention for every placement of the blocks."""
    bs, d, ctx, nb = 2, 3, 7, 5          # 4 blocks used out of a 5-block pool
    rng = np.random.default_rng(11)
    K = rng.standard_normal((ctx, d))
    V = rng.standard_normal((ctx, d))
    q = rng.standard_normal((1, 1, d))
    ref = _sdpa(q[0, 0], K, V, 0.7)
    outs = []
    for perm in itertools.permutations(range(nb), blocks_needed(ctx, bs)):
        kp = np.full((nb, 1, bs, d), np.nan)
        vp = np.full((nb, 1, bs, d), np.nan)      # unused blocks and tail slots poisoned
        table = list(perm)
        for t in range(ctx):
            kp[table[t // bs], 0, t % bs] = K[t]
            vp[table[t // bs], 0, t % bs] = V[t]
        out = attend_ref(q, kp, vp, np.array([table]), np.array([ctx]), 0.7, bs)
        outs.append(out[0, 0])
        np.testing.assert_allclose(out[0, 0], ref, rtol=1e-12, atol=1e-13)
    assert len(outs) == 120
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(3)
    K = rng.standard_normal((1, 8))
    V = rng.standard_normal((1, 8))
    np.testing.assert_array_equal(attend_one_ref(rng.standard_normal(8), K, V, 0.5), V[0])


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(4)
    K = rng.standard_normal((13, 8))
    V = rng.standard_normal((13, 8))
    np.testing.assert_allclose(attend_one_ref(np.zeros(8), K, V, 0.5), V.mean(axis=0), rtol=1e-13, atol=1e-14)


def test_one_hot_logit_selects_its_value_even_when_huge():
    rng = np.random.default_rng(5)
    d = 8
    K = rng.standard_normal((9, d)) * 0.01
    q = np.zeros(d); q[2] = 1000.0
    K[6, 2] = 5.0                               # logit 5000 for token 6, |others| < ~30
    V = rng.standard_normal((9, d))
    out = attend_one_ref(q, K, V, 1.0)
    assert np.all(np.isfinite(out))            # max subtraction keeps exp finite
    np.testing.assert_allclose(out, V[6], rtol=0, atol=1e-12)


def test_two_tokens_closed_form_logistic():
    rng = np.random.default_rng(6)
    for _ in range(20):
        q = rng.standard_normal(4); K = rng.standard_normal((2, 4)); V = rng.standard_normal((2, 4))
        sc = 0.37
        a = sc * K[0] @ q; b = sc * K[1] @ q
        w0 = 1.0 / (1.0 + math.exp(b - a))      # logistic form of a 2-way softmax
        np.testing.assert_allclose(attend_one_ref(q, K, V, sc), w0 * V[0] + (1 - w0) * V[1], rtol=1e-12, atol=1e-13)


def test_brute_force_tiny_with_fractions():
    """ctx <= 3, d <= 2 with small integers: exact rational weights via math.exp of integers."""
    K = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    V = np.array([[2.0, -1.0], [0.5, 4.0], [-3.0, 1.0]])
    q = np.array([1.0, 2.0])
    # logits 1, 2, 3 (scale 1): weights e^1 : e^2 : e^3
    e = [math.e, math.e ** 2, math.e ** 3]
    expect = sum(w * v for w, v in zip(e, V)) / sum(e)
    np.testing.assert_allclose(attend_one_ref(q, K, V, 1.0), expect, rtol=1e-14)


def test_zero_context_gives_zero_output():
    q, kp, vp, tables, _ = _rand_case(8, 2, 2, 2, 4, 4, [4, 4], 4)
    out = attend_ref(q, kp, vp, tables, np.array([0, 4]), 0.5, 4)
    assert np.all(out[0] == 0.0)
    assert np.any(out[1] != 0.0)


@pytest.mark.parametrize("part", [1, 2, 3, 5, 16, 100])
def test_partition_merge_equals_single_pass(part):
    rng = np.random.default_rng(part)
    n, d = 37, 6
    q = rng.standard_normal(d) * 30.0           # logits ~ N(0, 30^2): needs the max shift
    K = rng.standard_normal((n, d)); V = rng.standard_normal((n, d))
    states = [partial_state_ref(q, K[a:a + part], V[a:a + part], 0.5) for a in range(0, n, part)]
    states.append(partial_state_ref(q, K[:0], V[:0], 0.5))      # an empty slice merges as nothing
    np.testing.assert_allclose(merge_partials_ref(states), _sdpa(q, K, V, 0.5), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# Cache writes and block copies: another formulation through torch indexing
# ---------------------------------------------------------------------------

def test_reshape_matches_flat_slot_indexing_and_touches_nothing_else():
    rng = np.random.default_rng(9)
    NB, KVH, bs, d, T = 7, 3, 4, 5, 9
    kp = rng.integers(-1000, 1000, (NB, KVH, bs, d)).astype(np.int16)
    vp = rng.integers(-1000, 1000, (NB, KVH, bs, d)).astype(np.int16)
    key = rng.integers(-1000, 1000, (T, KVH, d)).astype(np.int16)
    val = rng.integers(-1000, 1000, (T, KVH, d)).astype(np.int16)
    slots = rng.choice(NB * bs, T, replace=False).astype(np.int64)
    slots[[2, 5]] = -1                                       # padding tokens write nothing
    k2, v2 = reshape_ref(key, val, kp, vp, slots, bs)
    # same write via a [NB*bs, KVH, d] view of a [NB, bs, KVH, d] permutation
    for pool, src, got in ((kp, key, k2), (vp, val, v2)):
        t = torch.from_numpy(pool.copy()).permute(0, 2, 1, 3).contiguous().view(NB * bs, KVH, d)
        keep = slots >= 0
        t[torch.from_numpy(slots[keep])] = torch.from_numpy(src[keep])
        expect = t.view(NB, bs, KVH, d).permute(0, 2, 1, 3).numpy()
        np.testing.assert_array_equal(got, expect)
        changed = np.argwhere(np.any(got != pool, axis=-1))
        allowed = {(s // bs, h, s % bs) for s in slots[keep] for h in range(KVH)}
        assert {tuple(c) for c in changed} <= allowed


def test_copy_blocks_matches_index_copy():
    rng = np.random.default_rng(10)
    NB, KVH, bs, d = 9, 2, 4, 3
    kp = rng.integers(0, 255, (NB, KVH, bs, d)).astype(np.uint8)
    vp = rng.integers(0, 255, (NB, KVH, bs, d)).astype(np.uint8)
    pairs = np.array([[1, 5], [1, 6], [3, 8]])
    k2, v2 = copy_ref(kp, vp, pairs)
    for pool, got in ((kp, k2), (vp, v2)):
        t = torch.from_numpy(pool.copy())
        t.index_copy_(0, torch.tensor(pairs[:, 1]), torch.from_numpy(pool)[torch.tensor(pairs[:, 0])])
        np.testing.assert_array_equal(got, t.numpy())
        for b in range(NB):
            if b not in pairs[:, 1]:
                np.testing.assert_array_equal(got[b], pool[b])


def test_swap_matches_index_copy_across_pools_and_leaves_source():
    rng = np.random.default_rng(11)
    KVH, bs, d = 2, 4, 3
    gk = rng.integers(0, 255, (9, KVH, bs, d)).astype(np.uint8)
    gv = rng.integers(0, 255, (9, KVH, bs, d)).astype(np.uint8)
    hk = rng.integers(0, 255, (5, KVH, bs, d)).astype(np.uint8)       # a smaller host pool
    hv = rng.integers(0, 255, (5, KVH, bs, d)).astype(np.uint8)
    pairs = np.array([[7, 0], [2, 4], [8, 1]])
    gk0, gv0 = gk.copy(), gv.copy()
    k2, v2 = swap_ref(gk, gv, hk, hv, pairs)
    np.testing.assert_array_equal(gk, gk0)
    np.testing.assert_array_equal(gv, gv0)
    for src, dst, got in ((gk, hk, k2), (gv, hv, v2)):
        t = torch.from_numpy(dst.copy())
        t.index_copy_(0, torch.tensor(pairs[:, 1]), torch.from_numpy(src)[torch.tensor(pairs[:, 0])])
        np.testing.assert_array_equal(got, t.numpy())
        assert got.shape == dst.shape
        for b in range(5):
            if b not in pairs[:, 1]:
                np.testing.assert_array_equal(got[b], dst[b])


def test_swap_out_then_in_restores_every_sequence_through_new_tables():
    """A round trip through a host pool into different GPU blocks gathers the same tokens."""
    rng = np.random.default_rng(12)
    NB, KVH, bs, d = 12, 2, 4, 3
    gk = rng.standard_normal((NB, KVH, bs, d))
    gv = rng.standard_normal((NB, KVH, bs, d))
    table, n = [3, 9, 5], 10
    before = [oracle.gather_tokens(p, table, n, bs, h) for p in (gk, gv) for h in range(KVH)]
    hk, hv = swap_ref(gk, gv, np.zeros((4, KVH, bs, d)), np.zeros((4, KVH, bs, d)), [[3, 2], [9, 0], [5, 3]])
    gk2, gv2 = gk.copy(), gv.copy()
    gk2[[3, 9, 5]] = np.nan                                   # the freed blocks are reused by others
    gk2, gv2 = swap_ref(hk, hv, gk2, gv2, [[2, 7], [0, 1], [3, 11]])
    after = [oracle.gather_tokens(p, [7, 1, 11], n, bs, h) for p in (gk2, gv2) for h in range(KVH)]
    for a, b in zip(before, after):
        np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------------------
# Chunked prefill: decode, causal SDPA, chunking, causality, GQA
# ---------------------------------------------------------------------------

def _paged_problem(rng, lens, H, KVH, d, bs, extra_blocks=3):
    nblk = [-(-n // bs) for n in lens]
    NB = sum(nblk) + extra_blocks
    perm = rng.permutation(NB)
    tables = np.full((len(lens), max(nblk)), -1, dtype=np.int64)
    k = 0
    for s, m in enumerate(nblk):
        tables[s, :m] = perm[k:k + m]
        k += m
    kp = np.full((NB, KVH, bs, d), np.nan)
    vp = np.full((NB, KVH, bs, d), np.nan)
    for s, n in enumerate(lens):
        for t in range(n):
            kp[tables[s, t // bs], :, t % bs] = rng.standard_normal((KVH, d))
            vp[tables[s, t // bs], :, t % bs] = rng.standard_normal((KVH, d))
    return kp, vp, tables


def test_prefill_chunk_of_one_is_decode():
    rng = np.random.default_rng(30)
    lens, H, KVH, d, bs = [5, 17, 1, 33], 4, 2, 8, 4
    kp, vp, tables = _paged_problem(rng, lens, H, KVH, d, bs)
    q = rng.standard_normal((len(lens), H, d))
    got = prefill_ref(q, kp, vp, tables, lens, np.arange(len(lens) + 1), 0.3, bs)
    np.testing.assert_array_equal(got, attend_ref(q, kp, vp, tables, lens, 0.3, bs))


def test_prefill_whole_prompt_is_causal_sdpa():
    rng = np.random.default_rng(31)
    lens, H, KVH, d, bs = [13, 7, 20], 6, 3, 8, 4
    kp, vp, tables = _paged_problem(rng, lens, H, KVH, d, bs)
    qsl = np.concatenate([[0], np.cumsum(lens)])
    q = rng.standard_normal((int(qsl[-1]), H, d))
    got = prefill_ref(q, kp, vp, tables, lens, qsl, 0.25, bs)
    for s, n in enumerate(lens):
        K = np.stack([gather_tokens(kp, tables[s], n, bs, g) for g in range(KVH)])      # [KVH, n, d]
        V = np.stack([gather_tokens(vp, tables[s], n, bs, g) for g in range(KVH)])
        K = torch.from_numpy(np.repeat(K, H // KVH, axis=0))
        V = torch.from_numpy(np.repeat(V, H // KVH, axis=0))
        Q = torch.from_numpy(q[qsl[s]:qsl[s + 1]].transpose(1, 0, 2).copy())            # [H, n, d]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=0.25)
        np.testing.assert_allclose(got[qsl[s]:qsl[s + 1]], ref.numpy().transpose(1, 0, 2), rtol=1e-12, atol=1e-12)


def test_prefill_in_chunks_equals_one_chunk():
    """Chunks [0,4), [4,11), [11,19) of one prompt, each with the context cached so far."""
    rng = np.random.default_rng(32)
    n, H, KVH, d, bs = 19, 2, 1, 8, 4
    kp, vp, tables = _paged_problem(rng, [n], H, KVH, d, bs)
    q = rng.standard_normal((n, H, d))
    whole = prefill_ref(q, kp, vp, tables, [n], [0, n], 0.5, bs)
    parts = [prefill_ref(q[a:b], kp, vp, tables, [b], [0, b - a], 0.5, bs) for a, b in ((0, 4), (4, 11), (11, 19))]
    np.testing.assert_array_equal(np.concatenate(parts), whole)
    # two sequences' chunks packed in one call: rows land at their query offsets
    both = prefill_ref(np.concatenate([q[4:11], q[11:19]]), kp, vp, np.concatenate([tables, tables]), [11, 19],
                       [0, 7, 15], 0.5, bs)
    np.testing.assert_array_equal(both, whole[4:19])


def test_prefill_is_causal_and_short_contexts_give_zero_rows():
    rng = np.random.default_rng(33)
    n, H, KVH, d, bs = 9, 2, 2, 4, 4
    kp, vp, tables = _paged_problem(rng, [n], H, KVH, d, bs)
    q = rng.standard_normal((n, H, d))
    base = prefill_ref(q, kp, vp, tables, [n], [0, n], 1.0, bs)
    kp2, vp2 = kp.copy(), vp.copy()
    t = 6                                             # change the token at position 6
    kp2[tables[0, t // bs], :, t % bs] += 5.0
    vp2[tables[0, t // bs], :, t % bs] -= 3.0
    moved = prefill_ref(q, kp2, vp2, tables, [n], [0, n], 1.0, bs)
    np.testing.assert_array_equal(moved[:t], base[:t])
    assert np.all(np.abs(moved[t:] - base[t:]).max(axis=(1, 2)) > 0)
    np.testing.assert_array_equal(base[0], np.stack([vp[tables[0, 0], h // (H // KVH), 0] for h in range(H)]))
    # 3 queries over a 2-token context: the first has no position and stays zero
    short = prefill_ref(q[:3], kp, vp, tables, [2], [0, 3], 1.0, bs)
    assert not short[0].any()
    np.testing.assert_array_equal(short[1:], prefill_ref(q[1:3], kp, vp, tables, [2], [0, 2], 1.0, bs))


# ---------------------------------------------------------------------------
# E4M3 codec: OCP definition, torch's float8_e4m3fn cast, closed forms
# ---------------------------------------------------------------------------

def test_e4m3_decode_all_codes_match_torch_float8():
    ours = e4m3_ref.decode_e4m3(np.arange(256))
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], lib[~nan])
    assert np.flatnonzero(nan).tolist() == [0x7F, 0xFF]


def test_e4m3_closed_form_values():
    dec = e4m3_ref.decode_e4m3
    assert dec(0x7E) == 448.0                   # largest finite: 2^8 * 1.75
    assert dec(0x01) == 2.0 ** -9               # smallest subnormal
    assert dec(0x07) == 7 * 2.0 ** -9           # largest subnormal
    assert dec(0x08) == 2.0 ** -6               # smallest normal
    assert dec(0x38) == 1.0                     # exponent field = bias
    assert dec(0xB8) == -1.0
    assert dec(0x80) == 0.0 and np.signbit(dec(0x80))
    assert np.isnan(dec(0x7F)) and np.isnan(dec(0xFF))


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -5, 3.7 / 448.0])
def test_e4m3_encode_every_fp16_pattern_matches_torch_in_range(scale):
    x = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.float16).to(torch.float32)
    xs = x.numpy()
    codes = e4m3_ref.encode_e4m3(xs, scale)
    quot = torch.from_numpy((xs / np.float32(scale)).astype(np.float32))
    lib = quot.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    in_range = np.abs(quot.numpy()) <= 448.0
    assert in_range.sum() > 10000
    np.testing.assert_array_equal(codes[in_range], lib[in_range])
    big = np.isfinite(quot.numpy()) & ~in_range
    assert np.all((codes[big] & 0x7F) == 0x7E)                  # saturate to +-448
    assert np.array_equal(codes[big] >> 7, np.signbit(quot.numpy()[big]).astype(np.uint8))


def test_e4m3_special_inputs():
    enc = e4m3_ref.encode_e4m3
    v = np.array([np.inf, -np.inf, np.nan, -np.nan, 0.0, -0.0, 1e30, -1e30], np.float32)
    v[3] = -np.float32(np.nan)
    got = enc(v, 1.0).tolist()
    assert got[0] == 0x7E and got[1] == 0xFE
    assert got[2] == 0x7F and got[3] == 0xFF
    assert got[4] == 0x00 and got[5] == 0x80
    assert got[6] == 0x7E and got[7] == 0xFE


def test_e4m3_roundtrip_ties_and_error_bound():
    enc, dec = e4m3_ref.encode_e4m3, e4m3_ref.decode_e4m3
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    vals = dec(np.array(finite))
    assert enc(vals.astype(np.float32), 1.0).tolist() == finite        # exact values round-trip
    pos = dec(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2                                     # exact in float32
    got = enc(mids.astype(np.float32), 1.0)
    lo_codes = np.arange(0x7E)
    expect = np.where(lo_codes % 2 == 0, lo_codes, lo_codes + 1)       # tie -> even mantissa
    np.testing.assert_array_equal(got, expect)
    rng = np.random.default_rng(12)
    x = (rng.standard_normal(20000) * 50).astype(np.float32)
    err = np.abs(dec(enc(x, 1.0)) - np.clip(x, -448, 448))
    gap = np.diff(pos)
    idx = np.clip(np.searchsorted(pos, np.minimum(np.abs(x), 448)) - 1, 0, len(gap) - 1)
    assert np.all(err <= gap[idx] / 2 + 1e-12)                          # at most half a step


# ---------------------------------------------------------------------------
# Contiguous model
# ---------------------------------------------------------------------------

def test_contiguous_model_fork_is_independent():
    m = oracle.ContiguousSequences()
    m.new(0)
    rows = np.arange(12, dtype=np.float32).reshape(3, 1, 4)
    m.extend(0, rows, -rows)
    m.fork(0, 1)
    m.append(1, np.full((1, 4), 7, np.float32), np.full((1, 4), 8, np.float32))
    assert m.length(0) == 3 and m.length(1) == 4
    np.testing.assert_array_equal(m.keys(0), rows)
    np.testing.assert_array_equal(m.keys(1)[:3], rows)
    np.testing.assert_array_equal(m.values(1)[3], np.full((1, 4), 8))


# ---------------------------------------------------------------------------
# E5M2 codec: OCP definition, torch's float8_e5m2 cast, the fp16 prefix property
# ---------------------------------------------------------------------------
from oracle import e5m2_ref  # noqa: E402


def test_e5m2_decode_all_codes_match_torch_float8():
    ours = e5m2_ref.decode_e5m2(np.arange(256))
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 6
    np.testing.assert_array_equal(ours[~nan], lib[~nan])


def test_e5m2_codes_are_the_top_byte_of_fp16():
    """E5M2 shares fp16's sign and exponent fields: code << 8 is the fp16 bit pattern of the same value."""
    codes = np.arange(256, dtype=np.uint16)
    as_f16 = (codes << 8).astype(np.uint16).view(np.float16).astype(np.float64)
    ours = e5m2_ref.decode_e5m2(codes.astype(np.uint8))
    nan = np.isnan(ours)
    assert np.array_equal(np.isnan(as_f16), nan)
    np.testing.assert_array_equal(as_f16[~nan], ours[~nan])


def test_e5m2_closed_forms():
    d = e5m2_ref.decode_e5m2
    assert d(0x7B) == 57344.0 and d(0xFB) == -57344.0
    assert d(0x01) == 2.0 ** -16 and d(0x04) == 2.0 ** -14 and d(0x3C) == 1.0
    assert d(0x7C) == np.inf and d(0xFC) == -np.inf and np.isnan(d(0x7D))
    assert e5m2_ref.encode_e5m2(np.float32(np.nan), 1.0) == 0x7F
    assert e5m2_ref.encode_e5m2(np.array([-np.nan], np.float32), 1.0)[0] == 0xFF
    assert e5m2_ref.encode_e5m2(np.array([np.inf, -np.inf, 1e9], np.float32), 1.0).tolist() == [0x7B, 0xFB, 0x7B]
    assert e5m2_ref.encode_e5m2(np.array([-0.0], np.float32), 1.0)[0] == 0x80
    # 1.125 lies halfway between 1.0 (m=0) and 1.25 (m=1): ties to the even mantissa
    assert e5m2_ref.encode_e5m2(np.array([1.125, 1.375], np.float32), 1.0).tolist() == [0x3C, 0x3E]


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -5, 3.7 / 57344.0])
def test_e5m2_encode_every_fp16_pattern_matches_torch(scale):
    x = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.float16).to(torch.float32)
    q = (x / torch.tensor(scale, dtype=torch.float32))
    ours = e5m2_ref.encode_e5m2(x.numpy(), scale)
    lib = q.to(torch.float8_e5m2).view(torch.uint8).numpy()
    finite = torch.isfinite(q).numpy() & (np.abs(q.numpy()) <= 57344.0)
    np.testing.assert_array_equal(ours[finite], lib[finite])
    big = ~finite & ~np.isnan(q.numpy())
    assert np.all((ours[big] & 0x7F) == 0x7B)                  # saturated, sign kept
    assert np.all(np.isnan(e5m2_ref.decode_e5m2(ours[np.isnan(q.numpy())])))


def test_dequant_per_head_scales_each_head():
    codes = np.random.default_rng(3).integers(0, 0x7B, (5, 3, 4, 8)).astype(np.uint8)
    scales = np.array([0.5, 2.0, 0.125], np.float32)
    got = e5m2_ref.dequant_per_head(codes, scales, e5m2_ref.decode_e5m2)
    for h in range(3):
        np.testing.assert_array_equal(got[:, h], e5m2_ref.dequant_e5m2(codes[:, h], scales[h]))


# ---------------------------------------------------------------------------
# 8-bit dequantisation at scales other than 1: stored value = code's value x the
# fp32 scale ("PagedAttention", Ultralytics glossary, section "Các kỹ thuật
# liên quan": the FP8 cache; one fp32 scale per pool or per kv head).  Pinned to
# closed forms (the code of 1.0 reads back as the fp32 scale itself), to torch's
# float8 decode times the fp32 scale, and to a half-step error bound whose step
# is written from the formats' exponent ranges, not read off the oracle's table.
# ---------------------------------------------------------------------------

# 0.05 and 3.7/448 are not binary fractions, so their fp32 rounding differs from
# the float64 value (a scale taken in float64 fails the exact checks); 2^-5 is
# exact; 7.3 is above 1.
DEQUANT_SCALES = [0.05, 2.0 ** -5, 3.7 / 448.0, 7.3]


@pytest.mark.parametrize("scale", DEQUANT_SCALES)
def test_e4m3_dequant_closed_forms_at_scale(scale):
    s32 = float(np.float32(scale))
    dq = lambda c: float(e4m3_ref.dequant_e4m3(np.uint8(c), scale))
    assert dq(0x38) == s32                          # code of 1.0 reads back as the fp32 scale
    assert dq(0xB8) == -s32
    assert dq(0x40) == 2.0 * s32                    # 0 1000 000 = 2
    assert dq(0x7E) == 448.0 * s32                  # largest finite code
    assert dq(0x01) == 2.0 ** -9 * s32              # smallest subnormal
    assert dq(0x00) == 0.0
    if s32 != scale:
        assert dq(0x38) != scale                    # the scale is the fp32 one, not the float64 argument


@pytest.mark.parametrize("scale", DEQUANT_SCALES)
def test_e5m2_dequant_closed_forms_at_scale(scale):
    s32 = float(np.float32(scale))
    dq = lambda c: float(e5m2_ref.dequant_e5m2(np.uint8(c), scale))
    assert dq(0x3C) == s32                          # code of 1.0 reads back as the fp32 scale
    assert dq(0xBC) == -s32
    assert dq(0x40) == 2.0 * s32                    # 0 10000 00 = 2
    assert dq(0x7B) == 57344.0 * s32                # largest finite code
    assert dq(0x01) == 2.0 ** -16 * s32             # smallest subnormal
    if s32 != scale:
        assert dq(0x3C) != scale


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("scale", DEQUANT_SCALES)
def test_dequant_all_codes_equal_torch_decode_times_fp32_scale(fmt, scale):
    codes = np.arange(256, dtype=np.uint8)
    tdt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    lib = torch.from_numpy(codes).view(tdt).to(torch.float64) * torch.tensor(scale, dtype=torch.float32).double()
    lib = lib.numpy()
    ours = (e4m3_ref.dequant_e4m3 if fmt == "e4m3" else e5m2_ref.dequant_e5m2)(codes, scale)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], lib[~nan])


def _fp8_step(a, fmt):
    """Spacing of the 8-bit values around magnitude a (in code units): 2^(e - mantissa bits), with the
    exponent e = floor(log2 a) held at the smallest normal exponent below it (subnormals share that step)."""
    mbits, emin = (3, -6) if fmt == "e4m3" else (2, -14)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** emin)))
    return 2.0 ** (np.maximum(e, emin) - mbits)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("scale", [2.0 ** -5, 3.7 / 448.0, 0.05])
def test_fp8_roundtrip_every_fp16_pattern_within_half_step(fmt, scale):
    """|dequant(encode(x, s), s) - clip(x, +-max*s)| <= half a step (times s), plus the fp32 rounding of x / s."""
    x = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.float16).to(torch.float64).numpy()
    x = x[np.isfinite(x)]
    s32 = float(np.float32(scale))
    if fmt == "e4m3":
        enc, dq, vmax = e4m3_ref.encode_e4m3, e4m3_ref.dequant_e4m3, 448.0
    else:
        enc, dq, vmax = e5m2_ref.encode_e5m2, e5m2_ref.dequant_e5m2, 57344.0
    back = dq(enc(x, scale), scale)
    target = np.clip(x, -vmax * s32, vmax * s32)
    a = np.minimum(np.abs(x) / s32, vmax)
    bound = _fp8_step(a, fmt) / 2 * s32 + 2.0 ** -23 * np.abs(x)
    err = np.abs(back - target)
    assert np.all(err <= bound), (x[np.argmax(err - bound)], float(np.max(err - bound)))
    assert np.array_equal(np.signbit(back[x != 0]), np.signbit(x[x != 0]))


def test_dequant_per_head_closed_form():
    """Every code 1.0 under per-head scales reads back as each head's own fp32 scale."""
    scales = np.array([0.05, 7.3, 3.7 / 448.0], np.float64)
    for codes, dec in ((np.full((2, 3, 4, 8), 0x3C, np.uint8), e5m2_ref.decode_e5m2),
                       (np.full((2, 3, 4, 8), 0x38, np.uint8), e4m3_ref.decode_e4m3)):
        got = e5m2_ref.dequant_per_head(codes, scales, dec)
        for h in range(3):
            assert np.all(got[:, h] == float(np.float32(scales[h])))
