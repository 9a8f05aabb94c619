"""Host-side step metadata built on libpa's allocator and slot mapping.

The CPU side of a step prepares the block tables ("Inside vLLM", section
"LLM Engine constructor": the CPU-side input batch holds the block tables for
KV-cache indexing) and the slot of every new token; the device kernels only
read them.  These helpers arrange the allocator's block ids into the int32
[B, max_blocks] tables the kernels take (-1 marks an unused entry).
"""
from __future__ import annotations

import numpy as np

from . import ops


def blocks_for(tokens: int, block_size: int) -> int:
    return (int(tokens) + block_size - 1) // block_size


def decode_block_tables(alloc: "ops.Allocator", seq_lens, block_size: int,
                        max_blocks: int | None = None) -> np.ndarray:
    """Sequences 0..B-1 in order each take the blocks their tokens need (one
    native call, pa_allocator_build_tables)."""
    need = [blocks_for(L, block_size) for L in seq_lens]
    width = max(need + [1]) if max_blocks is None else int(max_blocks)
    return alloc.build_tables(seq_lens, block_size, width)


def prefill_block_tables(alloc: "ops.Allocator", num_seqs: int, prefix_tokens: int,
                         own_tokens: int, block_size: int, share_prefix: bool = True) -> np.ndarray:
    """Prefix caching ("Im Inneren von vLLM", "Fortgeschrittene Funktionen"):
    sequence 0 takes the prefix blocks and the others share them by reference
    count (or take their own copies when share_prefix is False); then each
    sequence takes the blocks of its private suffix and chunk."""
    if prefix_tokens % block_size:
        raise ValueError("the shared prefix must fill whole blocks")
    npre = prefix_tokens // block_size
    nown = blocks_for(own_tokens, block_size)
    bt = np.full((num_seqs, npre + nown), -1, dtype=np.int32)
    if npre:
        first = alloc.allocate(npre)
        bt[0, :npre] = first
        for b in range(1, num_seqs):
            if share_prefix:
                alloc.share(first)
                bt[b, :npre] = first
            else:
                bt[b, :npre] = alloc.allocate(npre)
    for b in range(num_seqs):
        bt[b, npre:] = alloc.allocate(nown)
    return bt
