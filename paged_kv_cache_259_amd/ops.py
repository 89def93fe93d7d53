"""Thin Python binding over ``libpkv.so`` (C ABI in include/pkv.h).

Argument marshalling only: shapes and dtypes are read off torch tensors,
``data_ptr()``s and torch's current HIP stream are passed to the C calls, and a
negative status becomes a ``PkvError``.  Every step of the path runs in the HIP
kernels; there is no CPU fallback -- importing this module raises ImportError
when the library has not been built.
"""

import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PKV_LIB", os.path.join(_HERE, "libpkv.so"))

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"paged_kv_cache_259_amd: HIP library not found at {LIB_PATH}; "
        "build it with `python -m paged_kv_cache_259_amd.build` (there is no CPU fallback)")

_lib = ctypes.CDLL(LIB_PATH)

F32, F16, BF16, FP8_E4M3, FP8_E5M2 = 0, 1, 2, 3, 4
PATH_VECTOR, PATH_MFMA = 0, 1

_c_int, _c_float, _c_size, _vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

_lib.pkv_status_string.restype = ctypes.c_char_p
_lib.pkv_status_string.argtypes = [_c_int]
_lib.pkv_version.restype = _c_int
_lib.pkv_version.argtypes = []
_lib.pkv_attention_plan.restype = _c_int
_lib.pkv_attention_plan.argtypes = [_c_int] * 9 + [ctypes.POINTER(_c_int)] * 3
_lib.pkv_attention_workspace_bytes.restype = _c_size
_lib.pkv_attention_workspace_bytes.argtypes = [_c_int] * 9
_lib.pkv_paged_attention_decode.restype = _c_int
_lib.pkv_paged_attention_decode.argtypes = (
    [_vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp]
    + [_c_int] * 7
    + [_c_float] * 3
    + [_vp, _vp]
    + [_c_int] * 3
    + [_vp, _c_size, _vp])
_lib.pkv_paged_attention_decode_noalloc.restype = _c_int
_lib.pkv_paged_attention_decode_noalloc.argtypes = (
    [_vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp]
    + [_c_int] * 7
    + [_c_float] * 3
    + [_vp, _vp]
    + [_c_int] * 3
    + [_vp])
_lib.pkv_paged_attention_decode_append.restype = _c_int
_lib.pkv_paged_attention_decode_append.argtypes = (
    [_vp] * 7 + [_vp, _c_int, _vp, _vp] + [_c_int] * 7 + [_c_float] * 3 + [_vp, _vp] + [_c_int] * 3
    + [_vp, _c_size, _vp])
_lib.pkv_paged_attention_decode_shared.restype = _c_int
_lib.pkv_paged_attention_decode_shared.argtypes = (
    [_vp] * 7 + [_vp, _c_int, _vp] + [_vp] * 3 + [_c_int] * 2 + [_c_int] * 7 + [_c_float] * 3 + [_vp, _vp]
    + [_c_int] * 2 + [_vp])
_lib.pkv_reshape_and_cache.restype = _c_int
_lib.pkv_reshape_and_cache.argtypes = [_vp] * 5 + [_c_int] * 7 + [_c_float] * 2 + [_vp, _vp, _vp]
_lib.pkv_copy_blocks.restype = _c_int
_lib.pkv_copy_blocks.argtypes = [_vp, _vp, _vp] + [_c_int] * 6 + [_vp]
_lib.pkv_paged_prefill_attention.restype = _c_int
_lib.pkv_paged_prefill_attention.argtypes = ([_vp] * 5 + [_c_int] + [_vp, _vp] + [_c_int] * 9 + [_c_float] * 3
                                              + [_vp, _vp] + [_c_int] * 2 + [_vp])
_lib.pkv_swap_blocks.restype = _c_int
_lib.pkv_swap_blocks.argtypes = [_vp, _vp, _c_int, _vp, _vp, _c_int, _vp] + [_c_int] * 5 + [_vp]
_lib.pkv_set_debug_checks.restype = _c_int
_lib.pkv_set_debug_checks.argtypes = [_c_int]
_lib.pkv_debug_report.restype = _c_int
_lib.pkv_debug_report.argtypes = [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(_c_int),
                                  ctypes.POINTER(ctypes.c_int64)]
_lib.pkv_set_kv_load_policy.restype = _c_int
_lib.pkv_set_kv_load_policy.argtypes = [_c_int]

EXPORTED_SYMBOLS = (
    "pkv_status_string", "pkv_version", "pkv_attention_plan", "pkv_attention_workspace_bytes",
    "pkv_paged_attention_decode", "pkv_reshape_and_cache", "pkv_copy_blocks", "pkv_swap_blocks",
    "pkv_paged_prefill_attention", "pkv_paged_attention_decode_append", "pkv_paged_attention_decode_shared",
    "pkv_paged_attention_decode_noalloc", "pkv_set_debug_checks", "pkv_debug_report", "pkv_set_kv_load_policy",
)

ERR_PRECONDITION = -11              # PKV_ERR_PRECONDITION
# PKV_CHECK_* violation kinds of the debug checks
CHECK_KINDS = {
    1: "context_len", 2: "block_id", 3: "slot", 4: "duplicate_slot", 5: "append_slot", 6: "pair_id",
    7: "duplicate_dst", 8: "dst_is_src", 9: "seq_order", 10: "group", 11: "group_member", 12: "shared_block",
    13: "query_start", 14: "scale",
}

STATIC_SCRATCH_BYTES = 48 << 20     # PKV_STATIC_SCRATCH_BYTES
KV_LOAD_POLICIES = {"stream": 0, "cached": 1}   # PKV_KV_LOADS_STREAM, PKV_KV_LOADS_CACHED


class PkvError(RuntimeError):
    def __init__(self, status, call):
        self.status = status
        self.report = debug_report() if status == ERR_PRECONDITION else None
        msg = f"{call}: {_lib.pkv_status_string(status).decode()} (status {status})"
        if self.report:
            n, kind, index = self.report
            msg += f"; {n} violation(s), first: {CHECK_KINDS.get(kind, kind)} at index {index}"
        super().__init__(msg)


def set_debug_checks(mode):
    """Debug checks of the device-resident values: 1 on, 0 off, -1 follow PKV_DEBUG. Returns the previous mode."""
    return _lib.pkv_set_debug_checks(int(mode))


def set_kv_load_policy(policy):
    """K/V load policy of this thread's later decode calls: "stream" (non-temporal, the default: each block
    read once per launch) or "cached" (shared blocks stay in the caches between their readers).  Returns the
    previous policy's name."""
    prev = _lib.pkv_set_kv_load_policy(KV_LOAD_POLICIES[policy])
    _check(prev if prev < 0 else 0, "pkv_set_kv_load_policy")
    return {v: k for k, v in KV_LOAD_POLICIES.items()}[prev]


@contextlib.contextmanager
def kv_load_policy(policy):
    """Run the enclosed decode calls of this thread under `policy` (see set_kv_load_policy)."""
    prev = set_kv_load_policy(policy)
    try:
        yield
    finally:
        set_kv_load_policy(prev)


def debug_report():
    """(violations, kind, index) of the calling thread's most recent checked call (kind 0 / index -1: none)."""
    n, kind, index = ctypes.c_int64(0), ctypes.c_int(0), ctypes.c_int64(-1)
    _check(_lib.pkv_debug_report(ctypes.byref(n), ctypes.byref(kind), ctypes.byref(index)), "pkv_debug_report")
    return n.value, kind.value, index.value


def _check(status, call):
    if status != 0:
        raise PkvError(status, call)


def dtype_code(t: torch.dtype):
    if t == torch.float32:
        return F32
    if t == torch.float16:
        return F16
    if t == torch.bfloat16:
        return BF16
    if t in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    if t == torch.float8_e5m2:
        return FP8_E5M2
    raise TypeError(f"unsupported dtype {t}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _on_device(device, *tensors):
    """Every tensor argument on the pools' GPU: the kernels dereference them all."""
    if device.type != "cuda":
        raise ValueError("the KV pools must be GPU tensors")
    for t in tensors:
        if t is not None and t.device != device:
            raise ValueError(f"all tensor arguments must be on {device}; one is on {t.device}")


def _head_scales(t, kvh, device):
    """Optional per-kv-head scale array: fp32 [kvh], contiguous, on the pools' device."""
    if t is None:
        return None
    if t.dtype != torch.float32 or t.shape != (kvh,) or not t.is_contiguous() or t.device != device:
        raise ValueError("per-head scales must be a contiguous float32 [num_kv_heads] tensor on the pools' device")
    return t


def library_version():
    return _lib.pkv_version()


def attention_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len,
                   partition_size=0, q_dtype=F16, kv_dtype=F16):
    """(path, partition_tokens, num_partitions) the decode call would use."""
    path, ptoks, nparts = _c_int(), _c_int(), _c_int()
    _check(_lib.pkv_attention_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len,
                                   partition_size, q_dtype, kv_dtype,
                                   ctypes.byref(path), ctypes.byref(ptoks), ctypes.byref(nparts)),
           "pkv_attention_plan")
    return path.value, ptoks.value, nparts.value


def attention_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len,
                              partition_size=0, q_dtype=F16, kv_dtype=F16):
    return _lib.pkv_attention_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                              max_context_len, partition_size, q_dtype, kv_dtype)


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                           k_scale=1.0, v_scale=1.0, partition_size=0, workspace=None, num_blocks=None,
                           seq_order=None, k_scales=None, v_scales=None, stream=None):
    """out[s, h] = softmax(scale * K_s q[s, h]) V_s over each sequence's paged context.

    out, q: [S, H, d]; k_cache, v_cache: [NB, KVH, bs, d]; block_tables: int32
    [S, maxblk]; context_lens: int32 [S].  ``workspace``: a device uint8 tensor
    of at least ``attention_workspace_bytes(...)`` bytes (allocated here if None).
    ``seq_order``: optional int32 [S] device tensor, the sequences longest first
    (scheduling only; see ``BlockManager.longest_first``).  8-bit caches: uint8 /
    float8_e4m3fn pools are E4M3, float8_e5m2 pools E5M2; ``k_scales`` /
    ``v_scales`` (float32 [KVH]) replace the pool-wide scales per kv head.
    """
    S, H, d = q.shape
    NB, KVH, bs, d2 = k_cache.shape
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q/out and the pools")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S, maxblk] and context_lens [S]")
    for t in (out, q, k_cache, v_cache, block_tables, context_lens):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    qd, kvd = dtype_code(q.dtype), dtype_code(k_cache.dtype)
    if out.dtype != q.dtype:
        raise TypeError("out must have q's dtype")
    need = attention_workspace_bytes(S, H, KVH, d, bs, max_context_len, partition_size, qd, kvd)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if seq_order is not None and (seq_order.dtype != torch.int32 or seq_order.shape != (S,)
                                  or not seq_order.is_contiguous()):
        raise ValueError("seq_order must be a contiguous int32 [S] tensor")
    _on_device(k_cache.device, out, q, v_cache, block_tables, context_lens, workspace, seq_order)
    _check(_lib.pkv_paged_attention_decode(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), _ptr(seq_order), S, H, KVH, d, bs, NB if num_blocks is None else num_blocks, max_context_len,
        float(scale), float(k_scale), float(v_scale), _ptr(_head_scales(k_scales, KVH, k_cache.device)),
        _ptr(_head_scales(v_scales, KVH, k_cache.device)), qd, kvd, partition_size, ws_ptr, ws_bytes,
        _stream(stream)), "pkv_paged_attention_decode")
    return out


def paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                                   k_scale=1.0, v_scale=1.0, partition_size=0, num_blocks=None, seq_order=None,
                                   k_scales=None, v_scales=None, stream=None):
    """paged_attention_decode without a workspace: the library's static per-GPU scratch holds the
    split-context summaries, and nothing is allocated (for HIP graph capture and callers that cannot
    allocate).  Raises PkvError (PKV_ERR_SCRATCH_LIMIT) when the plan needs more than
    STATIC_SCRATCH_BYTES.  Calls that overlap on one GPU race on the scratch."""
    S, H, d = q.shape
    NB, KVH, bs, d2 = k_cache.shape
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q/out and the pools")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S, maxblk] and context_lens [S]")
    for t in (out, q, k_cache, v_cache, block_tables, context_lens):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if out.dtype != q.dtype:
        raise TypeError("out must have q's dtype")
    if seq_order is not None and (seq_order.dtype != torch.int32 or seq_order.shape != (S,)
                                  or not seq_order.is_contiguous()):
        raise ValueError("seq_order must be a contiguous int32 [S] tensor")
    _on_device(k_cache.device, out, q, v_cache, block_tables, context_lens, seq_order)
    _check(_lib.pkv_paged_attention_decode_noalloc(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), _ptr(seq_order), S, H, KVH, d, bs, NB if num_blocks is None else num_blocks,
        max_context_len, float(scale), float(k_scale), float(v_scale),
        _ptr(_head_scales(k_scales, KVH, k_cache.device)), _ptr(_head_scales(v_scales, KVH, k_cache.device)),
        dtype_code(q.dtype), dtype_code(k_cache.dtype), partition_size, _stream(stream)),
        "pkv_paged_attention_decode_noalloc")
    return out


def paged_prefill_attention(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale,
                            max_query_len, max_context_len, num_blocks=None, k_scale=1.0, v_scale=1.0,
                            k_scales=None, v_scales=None, stream=None):
    """Chunked prefill: query row i of sequence s (rows query_start_loc[s]..) sits at
    position context_lens[s] - n_s + i and attends causally over the paged cache.

    out, q: [num_tokens, H, d]; pools [NB, KVH, bs, d] of q's type or an 8-bit
    format (uint8 / float8_e4m3fn: E4M3, float8_e5m2: E5M2, values code * scale);
    block_tables int32 [S, maxblk]; context_lens int32 [S]; query_start_loc int32 [S + 1].
    """
    T, H, d = q.shape
    NB, KVH, bs, d2 = k_cache.shape
    S = context_lens.shape[0]
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q/out and the pools")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32 or query_start_loc.dtype != torch.int32:
        raise TypeError("block_tables, context_lens and query_start_loc must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or query_start_loc.shape != (S + 1,):
        raise ValueError("block_tables must be [S, maxblk] and query_start_loc [S + 1]")
    for t in (out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if out.dtype != q.dtype:
        raise TypeError("out must have q's dtype")
    if v_cache.dtype != k_cache.dtype:
        raise TypeError("k_cache and v_cache differ in dtype")
    _on_device(k_cache.device, out, q, v_cache, block_tables, context_lens, query_start_loc)
    _check(_lib.pkv_paged_prefill_attention(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), _ptr(query_start_loc), S, T, H, KVH, d, bs, NB if num_blocks is None else num_blocks,
        int(max_query_len), int(max_context_len), float(scale), float(k_scale), float(v_scale),
        _ptr(_head_scales(k_scales, KVH, k_cache.device)), _ptr(_head_scales(v_scales, KVH, k_cache.device)),
        dtype_code(q.dtype), dtype_code(k_cache.dtype), _stream(stream)), "pkv_paged_prefill_attention")
    return out


def paged_attention_decode_append(out, q, k_cache, v_cache, key, value, slot_mapping, block_tables, context_lens,
                                  scale, max_context_len, k_scale=1.0, v_scale=1.0, partition_size=0,
                                  workspace=None, num_blocks=None, seq_order=None, k_scales=None, v_scales=None,
                                  stream=None):
    """reshape_and_cache of each sequence's new token (key/value [S, KVH, d] in q's dtype, slot_mapping int64 [S])
    followed by paged_attention_decode, in one launch."""
    S, H, d = q.shape
    NB, KVH, bs, d2 = k_cache.shape
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q/out and the pools")
    if tuple(key.shape) != (S, KVH, d) or tuple(value.shape) != (S, KVH, d):
        raise ValueError("key/value must be [num_seqs, num_kv_heads, head_dim]")
    if key.dtype != q.dtype or value.dtype != q.dtype:
        raise TypeError("key/value must have q's dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (S,):
        raise TypeError("slot_mapping must be int64 [num_seqs]")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S, maxblk] and context_lens [S]")
    for t in (out, q, k_cache, v_cache, key, value, slot_mapping, block_tables, context_lens):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if out.dtype != q.dtype:
        raise TypeError("out must have q's dtype")
    if seq_order is not None and (seq_order.dtype != torch.int32 or seq_order.shape != (S,)
                                  or not seq_order.is_contiguous()):
        raise ValueError("seq_order must be a contiguous int32 [S] tensor")
    qd, kvd = dtype_code(q.dtype), dtype_code(k_cache.dtype)
    need = attention_workspace_bytes(S, H, KVH, d, bs, max_context_len, partition_size, qd, kvd)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _on_device(k_cache.device, out, q, v_cache, key, value, slot_mapping, block_tables, context_lens, workspace,
               seq_order)
    _check(_lib.pkv_paged_attention_decode_append(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(key), _ptr(value), _ptr(slot_mapping),
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), _ptr(seq_order), S, H, KVH, d, bs,
        NB if num_blocks is None else num_blocks, max_context_len, float(scale), float(k_scale), float(v_scale),
        _ptr(_head_scales(k_scales, KVH, k_cache.device)), _ptr(_head_scales(v_scales, KVH, k_cache.device)),
        qd, kvd, partition_size, ws_ptr, ws_bytes, _stream(stream)), "pkv_paged_attention_decode_append")
    return out


def paged_attention_decode_shared(out, q, k_cache, v_cache, block_tables, context_lens, group_offsets,
                                  group_members, group_shared_blocks, max_group_size, scale, max_context_len,
                                  key=None, value=None, slot_mapping=None, k_scale=1.0, v_scale=1.0, num_blocks=None,
                                  k_scales=None, v_scales=None, stream=None):
    """Decode (with append when key/value/slot_mapping are given) over groups of sequences whose tables start
    with the same physical blocks; a shared block is read once per group.  group_offsets int32 [G+1],
    group_members int32 [S], group_shared_blocks int32 [G] (see BlockManager.shared_groups)."""
    S, H, d = q.shape
    NB, KVH, bs, d2 = k_cache.shape
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q/out and the pools")
    if out.dtype != q.dtype:
        raise TypeError("out must have q's dtype")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S, maxblk] and context_lens [S]")
    G = group_shared_blocks.shape[0]
    for name, t, n in (("group_offsets", group_offsets, G + 1), ("group_members", group_members, S),
                       ("group_shared_blocks", group_shared_blocks, G)):
        if t.dtype != torch.int32 or t.shape != (n,) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 [{n}] tensor")
    append = key is not None
    if append:
        if tuple(key.shape) != (S, KVH, d) or tuple(value.shape) != (S, KVH, d):
            raise ValueError("key/value must be [num_seqs, num_kv_heads, head_dim]")
        if key.dtype != q.dtype or value.dtype != q.dtype:
            raise TypeError("key/value must have q's dtype")
        if slot_mapping is None or slot_mapping.dtype != torch.int64 or slot_mapping.shape != (S,):
            raise TypeError("slot_mapping must be int64 [num_seqs]")
    for t in (out, q, k_cache, v_cache, block_tables, context_lens) + ((key, value, slot_mapping) if append else ()):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    _on_device(k_cache.device, out, q, v_cache, block_tables, context_lens, group_offsets, group_members,
               group_shared_blocks, key, value, slot_mapping)
    _check(_lib.pkv_paged_attention_decode_shared(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(key), _ptr(value), _ptr(slot_mapping),
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), _ptr(group_offsets), _ptr(group_members),
        _ptr(group_shared_blocks), G, int(max_group_size), S, H, KVH, d, bs,
        NB if num_blocks is None else num_blocks, int(max_context_len), float(scale), float(k_scale), float(v_scale),
        _ptr(_head_scales(k_scales, KVH, k_cache.device)), _ptr(_head_scales(v_scales, KVH, k_cache.device)),
        dtype_code(q.dtype), dtype_code(k_cache.dtype), _stream(stream)), "pkv_paged_attention_decode_shared")
    return out


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, k_scale=1.0, v_scale=1.0, k_scales=None,
                      v_scales=None, stream=None):
    """k_cache[slot // bs, h, slot % bs] = enc(key[i, h]) for every token i (slot < 0 skipped)."""
    T, KVH, d = key.shape
    NB, KVH2, bs, d2 = k_cache.shape
    if (KVH2, d2) != (KVH, d) or tuple(value.shape) != tuple(key.shape) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch between key/value and the pools")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
        raise TypeError("slot_mapping must be int64 [num_tokens]")
    for t in (key, value, k_cache, v_cache, slot_mapping):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    _on_device(k_cache.device, key, value, v_cache, slot_mapping)
    _check(_lib.pkv_reshape_and_cache(
        _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), T, KVH, d, bs, NB,
        dtype_code(key.dtype), dtype_code(k_cache.dtype), float(k_scale), float(v_scale),
        _ptr(_head_scales(k_scales, KVH, k_cache.device)), _ptr(_head_scales(v_scales, KVH, k_cache.device)),
        _stream(stream)),
        "pkv_reshape_and_cache")


def copy_blocks(k_cache, v_cache, block_mapping, stream=None):
    """Whole-block copies k_cache[dst] = k_cache[src] (and V) for each (src, dst) row of block_mapping."""
    NB, KVH, bs, d = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache differ in shape")
    if block_mapping.dtype != torch.int64 or block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise TypeError("block_mapping must be int64 [num_pairs, 2]")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous() and block_mapping.is_contiguous()):
        raise ValueError("all tensors must be contiguous")
    _on_device(k_cache.device, v_cache, block_mapping)
    _check(_lib.pkv_copy_blocks(
        _ptr(k_cache), _ptr(v_cache), _ptr(block_mapping), block_mapping.shape[0], KVH, d, bs, NB,
        dtype_code(k_cache.dtype), _stream(stream)), "pkv_copy_blocks")


def swap_blocks(src_k, src_v, dst_k, dst_v, block_mapping, stream=None):
    """dst_k[dst] = src_k[src] (and V) for each (src, dst) row of block_mapping, between two pools.

    One pool is typically on the GPU and the other a pinned CPU tensor
    (``pin_memory=True``): swap-out is GPU -> CPU, swap-in CPU -> GPU.
    ``block_mapping`` (int64 [num_pairs, 2]) may be on the GPU or pinned.  The
    copy is enqueued on the stream: keep pinned tensors alive, and do not read a
    CPU pool, until the stream has passed the call.
    """
    NB_s, KVH, bs, d = src_k.shape
    NB_d = dst_k.shape[0]
    if tuple(src_v.shape) != tuple(src_k.shape) or tuple(dst_v.shape) != tuple(dst_k.shape) \
            or tuple(dst_k.shape[1:]) != (KVH, bs, d):
        raise ValueError("pools differ in block shape")
    if not (src_k.dtype == src_v.dtype == dst_k.dtype == dst_v.dtype):
        raise TypeError("pools differ in dtype")
    if block_mapping.dtype != torch.int64 or block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise TypeError("block_mapping must be int64 [num_pairs, 2]")
    for t in (src_k, src_v, dst_k, dst_v, block_mapping):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if t.device.type == "cpu" and not t.is_pinned():
            raise ValueError("CPU tensors must be pinned (pin_memory=True)")
    _check(_lib.pkv_swap_blocks(
        _ptr(src_k), _ptr(src_v), NB_s, _ptr(dst_k), _ptr(dst_v), NB_d, _ptr(block_mapping),
        block_mapping.shape[0], KVH, d, bs, dtype_code(src_k.dtype), _stream(stream)), "pkv_swap_blocks")


def raw_lib():
    """The ctypes handle (tests call the C ABI directly through it)."""
    return _lib
