"""Plain CPU oracle of the paged-attention hot path -- TEST INFRASTRUCTURE.

This package is the checker, not the product.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP library (no kernels, headers,
helpers, tables or constants) and imports nothing from it; both sides are fed
the same seeded arrays from ``paged_attention_kv_block_amd.inputs``, which
holds none of the method's arithmetic.

Everything here is written from the pages' description, in float64, as slow
and obvious code:

  kv_block_bytes, num_blocks_for_budget   closed forms (block size formula)
  OracleAllocator                         FIFO free_block_queue + refcounts
  slot_mapping, build_*_block_tables      logical token -> physical slot
  reshape_and_cache                       scatter of new K/V into the pool
  gather_kv                               pool + block table -> logical K/V
  attention                               softmax(scale * q K^T) V, and lse
  decode, prefill_chunk                   the two attention entry points
  fp8: e4m3_encode/decode, quantize      the FP8 (E4M3) KV-cache codec

Pins (tests/test_oracle_*.py) tie each function to something other than
itself: hand-worked fixtures under tests/golden/, closed forms, torch's
scaled_dot_product_attention in float64, coordinate-encoded pools, and the
invariants the pages fix.  No function here is "parity unpinned".
"""
from .paged_attention import (  # noqa: F401
    kv_block_bytes,
    num_blocks_for_budget,
    slot_mapping,
    reshape_and_cache,
    gather_kv,
    attention,
    decode,
    prefill_chunk,
    to_f64,
    empty_pool,
)
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    e4m3_decode,
    e4m3_encode,
    e4m3_decode_array,
    e4m3_encode_array,
    quantize,
)
from .allocator import (  # noqa: F401
    OracleAllocator,
    NoFreeBlocks,
    InvalidArgument,
    build_decode_block_tables,
    build_prefill_block_tables,
)
