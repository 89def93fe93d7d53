"""Seeded synthetic inputs for the paged decode workloads.

This module only draws random numbers and sizes buffers: it holds none of the
method's arithmetic (no addressing, allocation, attention or encoding).  Both
the GPU path's tests/bench and the CPU oracle consume what it produces.

Draw order for a decode workload (one ``numpy.random.Generator`` seeded with the
workload's seed, then one ``torch.Generator`` with the same seed for the
tensors):  context lengths -> free-list permutation -> q -> K pool -> V pool ->
new-token K -> new-token V.  Values are fp32 N(0, 1) cast to the storage dtype
by round-to-nearest-even (torch's ``.to``).

Length recipes:
* ``("fixed", [..])``                     exact lengths;
* ``("lognormal", median, sigma, lo, hi)`` ``clip(round(exp(N(ln median, sigma))), lo, hi)``;
* ``("uniform", lo, hi)``                  integers uniform in [lo, hi].
The lognormal sigma (0.6) is a reading: the workloads name only median and range.
The pages measure on ShareGPT / Alpaca request traces; those are not used --
these lognormal / uniform mixes of the stated sizes stand in for them.
"""

from dataclasses import dataclass, field, replace
import math

import numpy as np
import torch

DTYPES = {
    "f32": torch.float32,
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "fp8_e4m3": torch.uint8,   # stored codes; written by reshape_and_cache
}


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    seed: int
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q_dtype: str
    kv_dtype: str
    lengths: tuple
    max_blocks_per_seq: int
    num_blocks: int = 0          # 0 -> sized from the drawn lengths (pool_slack x need, upper bound)
    pool_slack: float = 1.2
    partition_size: int = 0      # 0 -> library's automatic choice
    scale: float = 0.0           # 0 -> 1/sqrt(head_dim)
    kv_scale: float = 1.0        # 8-bit caches: the pool-wide k_scale and v_scale
    code_max: int = 0x5F         # 8-bit caches: largest magnitude code drawn for the pools

    @property
    def softmax_scale(self):
        return self.scale if self.scale > 0 else 1.0 / math.sqrt(self.head_dim)

    @property
    def kv8(self):
        return DTYPES[self.kv_dtype] == torch.uint8

    @property
    def src_dtype(self):         # type of the new tokens' K/V (an 8-bit cache encodes them)
        return self.q_dtype if self.kv8 else self.kv_dtype


@dataclass(frozen=True)
class SharedPrefixWorkload:
    """Parallel sampling over shared prompts, FP8 cache (copy-on-write workload)."""
    name: str
    seed: int
    num_prompts: int
    prompt_len: int
    samples_per_prompt: int
    cont_lo: int
    cont_hi: int
    num_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    q_dtype: str = "f16"
    src_dtype: str = "f16"
    kv_dtype: str = "fp8_e4m3"

    @property
    def softmax_scale(self):
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def num_kv_heads(self):          # multi-head attention: one kv head per query head
        return self.num_heads

    @property
    def num_seqs(self):              # every sample is a sequence
        return self.num_prompts * self.samples_per_prompt


@dataclass(frozen=True)
class PrefillWorkload:
    """Chunked prefill: each sequence has ``prior`` cached tokens and a chunk of new query tokens."""
    name: str
    seed: int
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str
    chunk: tuple                 # length recipe of the chunks (query tokens per sequence)
    prior: tuple                 # length recipe of the context cached before the chunk
    max_blocks_per_seq: int
    pool_slack: float = 1.2
    kv_dtype: str = ""           # "" -> the cache has ``dtype``; "fp8_e4m3": an 8-bit cache
    kv_scale: float = 1.0        # 8-bit caches: the pool-wide k_scale and v_scale
    code_max: int = 0x5F         # 8-bit caches: largest magnitude code drawn for the pools

    @property
    def softmax_scale(self):
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def kv8(self):
        return bool(self.kv_dtype) and DTYPES[self.kv_dtype] == torch.uint8


# The five named workloads.
TINY_F32 = DecodeWorkload(
    name="tiny fp32 paged decode: 4 seqs ctx {40,17,1,64}, 8 heads MHA, d64, bs16, 64-block pool",
    seed=25901, num_seqs=4, num_heads=8, num_kv_heads=8, head_dim=64, block_size=16,
    q_dtype="f32", kv_dtype="f32", lengths=("fixed", (40, 17, 1, 64)),
    max_blocks_per_seq=4, num_blocks=64, scale=1.0 / 8.0)

LLAMA13B_F16 = DecodeWorkload(
    name="LLaMA-13B-shaped decode, one layer: 64 seqs, 40/40 heads, d128, fp16, bs16, "
         "lognormal ctx median 600 in [16,2048]",
    seed=25902, num_seqs=64, num_heads=40, num_kv_heads=40, head_dim=128, block_size=16,
    q_dtype="f16", kv_dtype="f16", lengths=("lognormal", 600, 0.6, 16, 2048),
    max_blocks_per_seq=128)

GQA_BF16 = DecodeWorkload(
    name="GQA decode, one layer: 256 seqs, 64 q heads over 8 kv heads, d128, bf16, bs16, "
         "lognormal ctx median 1000 in [32,4096]",
    seed=25903, num_seqs=256, num_heads=64, num_kv_heads=8, head_dim=128, block_size=16,
    q_dtype="bf16", kv_dtype="bf16", lengths=("lognormal", 1000, 0.6, 32, 4096),
    max_blocks_per_seq=256)

# The GQA shape over an E4M3 cache: pool codes drawn uniformly over magnitudes
# 0 .. 0x5F (|value| <= 30 before the scale) with random signs.
GQA_FP8 = DecodeWorkload(
    name="GQA decode over an E4M3 cache, one layer: 256 seqs, 64 q heads over 8 kv heads, d128, bf16 q, "
         "fp8 E4M3 K/V (scale 0.05), bs16, lognormal ctx median 1000 in [32,4096]",
    seed=25909, num_seqs=256, num_heads=64, num_kv_heads=8, head_dim=128, block_size=16,
    q_dtype="bf16", kv_dtype="fp8_e4m3", lengths=("lognormal", 1000, 0.6, 32, 4096),
    max_blocks_per_seq=256, kv_scale=0.05)

LONG_SPLITK_BF16 = DecodeWorkload(
    name="long-context split-K decode: 8 seqs ctx uniform [32768,131072], 32 q / 8 kv heads, "
         "d128, bf16, bs16, partitions of 512 tokens, 70000-block pool",
    seed=25904, num_seqs=8, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
    q_dtype="bf16", kv_dtype="bf16", lengths=("uniform", 32768, 131072),
    max_blocks_per_seq=8192, num_blocks=70000, partition_size=512)

SHARED_PREFIX_FP8 = SharedPrefixWorkload(
    name="shared-prefix parallel sampling with copy-on-write: 32 prompts x 1000 tokens, n=4, "
         "continuations 0-512, 40 heads MHA, d128, fp16 q, fp8 e4m3 K/V with per-tensor scale",
    seed=25905, num_prompts=32, prompt_len=1000, samples_per_prompt=4, cont_lo=0, cont_hi=512,
    num_heads=40, head_dim=128, block_size=16, num_blocks=6400, max_blocks_per_seq=95)

# Chunked prefill (the next workload after decode: compute-bound, MFMA-dense).
PREFILL_LLAMA13B_F16 = PrefillWorkload(
    name="chunked prefill, LLaMA-13B-shaped layer: 8 seqs x 512-token chunks over 0-3584 cached tokens, "
         "40/40 heads, d128, fp16, bs16",
    seed=25906, num_seqs=8, num_heads=40, num_kv_heads=40, head_dim=128, block_size=16, dtype="f16",
    chunk=("fixed", (512,) * 8), prior=("uniform", 0, 3584), max_blocks_per_seq=256)

PREFILL_GQA_BF16 = PrefillWorkload(
    name="chunked prefill, GQA layer: 16 seqs x 512-token chunks over 0-7680 cached tokens, "
         "64 q / 8 kv heads, d128, bf16, bs16",
    seed=25907, num_seqs=16, num_heads=64, num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16",
    chunk=("fixed", (512,) * 16), prior=("uniform", 0, 7680), max_blocks_per_seq=512)

# The GQA prefill over an E4M3 cache: the prior context's codes drawn like the
# GQA E4M3 decode pool's, the chunk's K/V (bf16) encoded by reshape_and_cache.
PREFILL_GQA_FP8 = PrefillWorkload(
    name="chunked prefill, GQA layer over an E4M3 cache: 16 seqs x 512-token chunks over 0-7680 cached tokens, "
         "64 q / 8 kv heads, d128, bf16 q, fp8 E4M3 K/V (scale 0.05), bs16",
    seed=25910, num_seqs=16, num_heads=64, num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16",
    chunk=("fixed", (512,) * 16), prior=("uniform", 0, 7680), max_blocks_per_seq=512, kv_dtype="fp8_e4m3",
    kv_scale=0.05)

@dataclass(frozen=True)
class PrefixCacheWorkload:
    """Requests that share a system prompt, prefilled with and without the prefix cache."""
    name: str
    seed: int
    num_requests: int
    shared_len: int
    unique_len: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str
    max_blocks_per_seq: int

    @property
    def softmax_scale(self):
        return 1.0 / math.sqrt(self.head_dim)


PREFIX_CACHE_LLAMA13B_F16 = PrefixCacheWorkload(
    name="prefix caching, LLaMA-13B-shaped layer: 16 requests = a shared 2048-token system prompt + 512 own "
         "tokens each, 40/40 heads, d128, fp16, bs16",
    seed=25908, num_requests=16, shared_len=2048, unique_len=512, num_heads=40, num_kv_heads=40, head_dim=128,
    block_size=16, dtype="f16", max_blocks_per_seq=160)

WORKLOADS = {
    "tiny_f32": TINY_F32,
    "llama13b_f16": LLAMA13B_F16,
    "gqa_bf16": GQA_BF16,
    "long_splitk_bf16": LONG_SPLITK_BF16,
    "gqa_fp8": GQA_FP8,
    "shared_prefix_fp8": SHARED_PREFIX_FP8,
    "prefill_llama13b_f16": PREFILL_LLAMA13B_F16,
    "prefill_gqa_bf16": PREFILL_GQA_BF16,
    "prefill_gqa_fp8": PREFILL_GQA_FP8,
    "prefix_cache_llama13b_f16": PREFIX_CACHE_LLAMA13B_F16,
}


def draw_lengths(rng, recipe, n):
    kind = recipe[0]
    if kind == "fixed":
        vals = np.asarray(recipe[1], dtype=np.int64)
        if len(vals) != n:
            raise ValueError("fixed length list does not match num_seqs")
        return vals
    if kind == "lognormal":
        _, median, sigma, lo, hi = recipe
        x = np.exp(rng.normal(np.log(median), sigma, size=n))
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    if kind == "uniform":
        _, lo, hi = recipe
        return rng.integers(lo, hi + 1, size=n).astype(np.int64)
    raise ValueError(f"unknown length recipe {kind}")


def pool_blocks_upper_bound(lengths, block_size, slack):
    """Pool size: slack x an upper bound on the blocks the lengths can occupy (sizing only)."""
    bound = int(np.sum(lengths)) // block_size + len(lengths)
    return int(math.ceil(slack * bound))


def randn(gen, shape, dtype, device):
    """fp32 N(0,1) drawn with ``gen`` on ``device``, cast by round-to-nearest-even."""
    x = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    return x.to(dtype)


def codes8(gen, shape, code_max, device):
    """uint8 codes: magnitude uniform in 0 .. code_max, random sign bit."""
    mag = torch.randint(0, code_max + 1, shape, generator=gen, dtype=torch.int32, device=device)
    sign = torch.randint(0, 2, shape, generator=gen, dtype=torch.int32, device=device)
    return (mag | (sign << 7)).to(torch.uint8)


def make_generator(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


@dataclass
class DecodeInputs:
    workload: DecodeWorkload
    context_lens: np.ndarray       # int64 [S]
    free_list: list                # seeded permutation of the pool's block ids
    num_blocks: int
    q: torch.Tensor                # [S, H, d]
    k_cache: torch.Tensor          # [NB, KVH, bs, d]
    v_cache: torch.Tensor
    k_new: torch.Tensor            # [S, KVH, d]   the new token's key per sequence
    v_new: torch.Tensor
    extra: dict = field(default_factory=dict)


def make_decode_inputs(w: DecodeWorkload, device="cpu", lengths=None):
    """Draw every input of one decode step of workload ``w`` on ``device``."""
    rng = np.random.default_rng(w.seed)
    ctx = draw_lengths(rng, w.lengths, w.num_seqs) if lengths is None else np.asarray(lengths, np.int64)
    nb = w.num_blocks or pool_blocks_upper_bound(ctx, w.block_size, w.pool_slack)
    free_list = rng.permutation(nb).tolist()
    gen = make_generator(w.seed, device)
    qdt, kvdt = DTYPES[w.q_dtype], DTYPES[w.kv_dtype]
    S, H, KVH, d, bs = w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size
    q = randn(gen, (S, H, d), qdt, device)
    if w.kv8:
        k_cache = codes8(gen, (nb, KVH, bs, d), w.code_max, device)
        v_cache = codes8(gen, (nb, KVH, bs, d), w.code_max, device)
    else:
        k_cache = randn(gen, (nb, KVH, bs, d), kvdt, device)
        v_cache = randn(gen, (nb, KVH, bs, d), kvdt, device)
    srcdt = DTYPES[w.src_dtype]
    k_new = randn(gen, (S, KVH, d), srcdt, device)
    v_new = randn(gen, (S, KVH, d), srcdt, device)
    return DecodeInputs(w, ctx, free_list, nb, q, k_cache, v_cache, k_new, v_new)


def scaled(w: DecodeWorkload, **kw):
    """A copy of workload ``w`` with some fields replaced (smaller parity-test variants)."""
    return replace(w, **kw)


@dataclass
class SharedPrefixInputs:
    workload: SharedPrefixWorkload
    cont_lens: np.ndarray          # int64 [num_prompts * samples]
    free_list: list
    prompt_k: torch.Tensor         # [num_prompts, prompt_len, H, d] src dtype
    prompt_v: torch.Tensor
    gen: torch.Generator           # continues the stream: per-step K/V, then q


def make_shared_prefix_inputs(w: SharedPrefixWorkload, device="cpu"):
    rng = np.random.default_rng(w.seed)
    n_seq = w.num_prompts * w.samples_per_prompt
    cont = rng.integers(w.cont_lo, w.cont_hi + 1, size=n_seq).astype(np.int64)
    free_list = rng.permutation(w.num_blocks).tolist()
    gen = make_generator(w.seed, device)
    sdt = DTYPES[w.src_dtype]
    pk = randn(gen, (w.num_prompts, w.prompt_len, w.num_heads, w.head_dim), sdt, device)
    pv = randn(gen, (w.num_prompts, w.prompt_len, w.num_heads, w.head_dim), sdt, device)
    return SharedPrefixInputs(w, cont, free_list, pk, pv, gen)


def draw_step_kv(inp: SharedPrefixInputs, n_tokens, device):
    """Keys and values of the next ``n_tokens`` continuation tokens (draw order continues)."""
    w = inp.workload
    sdt = DTYPES[w.src_dtype]
    k = randn(inp.gen, (n_tokens, w.num_heads, w.head_dim), sdt, device)
    v = randn(inp.gen, (n_tokens, w.num_heads, w.head_dim), sdt, device)
    return k, v


def draw_query(inp: SharedPrefixInputs, n_seqs, device):
    w = inp.workload
    return randn(inp.gen, (n_seqs, w.num_heads, w.head_dim), DTYPES[w.q_dtype], device)


@dataclass
class PrefillInputs:
    workload: PrefillWorkload
    chunk_lens: np.ndarray         # int64 [S] query tokens per sequence
    context_lens: np.ndarray       # int64 [S] prior + chunk
    query_start_loc: np.ndarray    # int64 [S + 1]
    free_list: list
    num_blocks: int
    q: torch.Tensor                # [T, H, d]
    k_cache: torch.Tensor          # [NB, KVH, bs, d]
    v_cache: torch.Tensor
    k_new: torch.Tensor            # [T, KVH, d] the chunk's keys, in query order
    v_new: torch.Tensor


def make_prefill_inputs(w: PrefillWorkload, device="cpu", chunk=None, prior=None):
    """Draw one chunked-prefill step: chunk lengths -> prior lengths -> free-list permutation
    -> q -> K pool -> V pool -> chunk K -> chunk V."""
    rng = np.random.default_rng(w.seed)
    n = draw_lengths(rng, w.chunk, w.num_seqs) if chunk is None else np.asarray(chunk, np.int64)
    pre = draw_lengths(rng, w.prior, w.num_seqs) if prior is None else np.asarray(prior, np.int64)
    ctx = pre + n
    nb = pool_blocks_upper_bound(ctx, w.block_size, w.pool_slack)
    free_list = rng.permutation(nb).tolist()
    qsl = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
    T = int(qsl[-1])
    gen = make_generator(w.seed, device)
    dt = DTYPES[w.dtype]
    H, KVH, d, bs = w.num_heads, w.num_kv_heads, w.head_dim, w.block_size
    q = randn(gen, (T, H, d), dt, device)
    if w.kv8:
        k_cache = codes8(gen, (nb, KVH, bs, d), w.code_max, device)
        v_cache = codes8(gen, (nb, KVH, bs, d), w.code_max, device)
    else:
        k_cache = randn(gen, (nb, KVH, bs, d), dt, device)
        v_cache = randn(gen, (nb, KVH, bs, d), dt, device)
    k_new = randn(gen, (T, KVH, d), dt, device)
    v_new = randn(gen, (T, KVH, d), dt, device)
    return PrefillInputs(w, n, ctx, qsl, free_list, nb, q, k_cache, v_cache, k_new, v_new)


@dataclass
class PrefixCacheInputs:
    workload: PrefixCacheWorkload
    prompts: list                  # token ids per request (shared prefix + own tokens)
    free_list: list
    num_blocks: int
    q: torch.Tensor                # [requests * prompt_len, H, d] queries of every prompt token
    k: torch.Tensor                # [requests * prompt_len, KVH, d] K of every prompt token
    v: torch.Tensor


def make_prefix_cache_inputs(w: PrefixCacheWorkload, device="cpu"):
    """Token ids (shared prefix, then each request's own) -> free-list permutation -> q -> K -> V.
    K/V of a shared-prefix token are the same in every request."""
    rng = np.random.default_rng(w.seed)
    shared = rng.integers(0, 32000, w.shared_len).tolist()
    prompts = [shared + rng.integers(0, 32000, w.unique_len).tolist() for _ in range(w.num_requests)]
    L = w.shared_len + w.unique_len
    nb = int(math.ceil(1.1 * w.num_requests * (-(-L // w.block_size))))
    free_list = rng.permutation(nb).tolist()
    gen = make_generator(w.seed, device)
    dt = DTYPES[w.dtype]
    R, H, KVH, d = w.num_requests, w.num_heads, w.num_kv_heads, w.head_dim
    q = randn(gen, (R * L, H, d), dt, device)
    k_sh = randn(gen, (w.shared_len, KVH, d), dt, device)
    v_sh = randn(gen, (w.shared_len, KVH, d), dt, device)
    k_own = randn(gen, (R, w.unique_len, KVH, d), dt, device)
    v_own = randn(gen, (R, w.unique_len, KVH, d), dt, device)
    k = torch.cat([torch.cat([k_sh, k_own[r]]) for r in range(R)])
    v = torch.cat([torch.cat([v_sh, v_own[r]]) for r in range(R)])
    return PrefixCacheInputs(w, prompts, free_list, nb, q, k, v)
