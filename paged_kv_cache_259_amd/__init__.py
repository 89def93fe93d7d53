"""Paged-KV decode for AMD MI355X (gfx950): PagedAttention decode, reshape_and_cache, copy_blocks.

The compute lives in the HIP library ``libpkv.so`` (C ABI, declared in
``include/pkv.h``).  ``paged_kv_cache_259_amd.ops`` is the thin Python binding
over it (argument marshalling only); it raises ImportError if the library has
not been built -- there is no CPU fallback.  ``block_manager`` holds the host
block bookkeeping and ``synth`` the seeded synthetic inputs.
"""

__all__ = [
    "paged_attention_decode",
    "reshape_and_cache",
    "copy_blocks",
    "attention_workspace_bytes",
    "attention_plan",
    "BlockManager",
]


def __getattr__(name):
    if name == "BlockManager":
        from .block_manager import BlockManager
        return BlockManager
    if name in __all__:
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
