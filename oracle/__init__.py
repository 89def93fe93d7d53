"""CPU oracle for the paged-KV decode path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the
``paged_kv_cache_259_amd`` package and its HIP library) never imports it, and
this package never imports the product: the two share no code.  The only thing
both sides consume is the seeded input generator
``paged_kv_cache_259_amd.synth``, which holds none of the method's arithmetic.

Everything here is plain numpy in float64 (or exact integer / byte work), written
from the definitions on the source pages, one small function per step, with no
blocking, fusion or reordering beyond what the definition states.

Sources cited in this package (page title, then section):

* [KVpag]  "KV cache paginado e batching contínuo para LLMs" (system-design
  concept page), section "Como funciona": per-request block table mapping
  logical to physical blocks; a block is allocated only when the previous ones
  are full; reference-counted shared blocks; block-level copy-on-write.
* [PA/paging]  "PagedAttention" (Ultralytics glossary), section
  "Cách phân trang hoạt động" (how paging works): 16-token default block, new
  block only when the last is full, taken from anywhere free, the table keeps the
  order, attention gathers keys and values block by block; the PyTorch worked
  example and its printed result.
* [PA/sharing]  same page, section "Chia sẻ block giữa các chuỗi" (sharing
  blocks between sequences): per-block reference counts, copy before writing a
  block another sequence still uses.
* [PA/related]  same page, section "Các kỹ thuật liên quan" (related
  techniques): FlashAttention-style tiling never writes the score matrix; GQA
  shares K/V heads between query heads; FP8 cache stores 8-bit keys/values.
* [vLLM-rev]  "vLLM PagedAttention: uma revolução no throughput de inferência
  de LLMs", feature list: chunked prefill (a long prompt's prefill split into
  chunks), prefix caching, prefill compute-bound vs decode bandwidth-bound.
* [OFP8]  the OCP 8-bit floating point specification (E4M3 "FN" and E5M2
  encodings) -- not on the pages; the pages only say "8-bit".  It fixes the codecs.

Readings where the pages are silent are listed in each function's docstring.
"""

from .e4m3_ref import decode_e4m3, encode_e4m3, dequant_e4m3, E4M3_MAX  # noqa: F401
from .e5m2_ref import decode_e5m2, encode_e5m2, dequant_e5m2, dequant_per_head, E5M2_MAX  # noqa: F401
from .paged_attention_ref import (  # noqa: F401
    blocks_needed,
    take_blocks,
    slot_of,
    gather_tokens,
    attend_ref,
    attend_one_ref,
    reshape_ref,
    copy_ref,
    swap_ref,
    prefill_ref,
    partial_state_ref,
    merge_partials_ref,
)
from .contiguous_model import ContiguousSequences  # noqa: F401
