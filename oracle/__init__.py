"""Float64 CPU oracle for the paged decode path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct numpy code that states what the PagedAttention decode path
computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it.  The product (``paged_kv_cache_306_amd``) never imports it and
shares no code with it: every step of the product path runs in the HIP library.

Modules:
  storage        exact decoding of f32 / f16 / bf16 storage bits to float64
  attention      gather through the block table, then textbook softmax(q K^T * scale) V
  multi_query    several new tokens of a sequence at once (prefix-cache hits, prompt chunks,
                 draft tokens): each attends to the cached tokens up to its own position
  cache_ops      reshape_and_cache (append a token's K/V into its slot), copy_blocks and
                 swap_blocks (block copies within a pool or between HBM and host pools)
  block_manager  block allocation with reference counts and copy-on-write

Every function is pinned by ``tests/test_oracle_pins.py`` (closed forms, a library
reduction, invariances, the pages' worked examples); none is "parity unpinned".
"""
from .storage import decode, decode_bits_f16, decode_bits_bf16
from .attention import gather_sequence, attend, paged_attention_decode, decode_unit
from .multi_query import paged_attention_multi_query, multi_query_unit, query_position
from .cache_ops import reshape_and_cache, copy_blocks, swap_blocks
from .block_manager import BlockManager, OutOfBlocks

__all__ = [
    "decode", "decode_bits_f16", "decode_bits_bf16",
    "gather_sequence", "attend", "paged_attention_decode", "decode_unit",
    "paged_attention_multi_query", "multi_query_unit", "query_position",
    "reshape_and_cache", "copy_blocks", "swap_blocks",
    "BlockManager", "OutOfBlocks",
]
