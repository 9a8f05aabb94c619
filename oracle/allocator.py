"""Oracle of the KV-cache block allocator -- test infrastructure.

[IV] "Inside vLLM: Anatomy of a High-Throughput LLM Inference System",
section "LLM Engine & Engine Core": the scheduler's KV-cache manager keeps a
free_block_queue, a pool of free KV-cache blocks (often hundreds of
thousands).  [IM] "Im Inneren von vLLM ...", section "Fortgeschrittene
Funktionen", and [TE] "Tiefenanalyse": prefix caching reuses the KV cache of
shared prompt prefixes.

The pages name the queue but not its policy.  Readings:
  * FIFO: allocate pops from the head, a block whose last user frees it is
    pushed to the tail; a sequence frees its blocks in logical order;
  * the initial queue order is given by the caller (a seeded permutation);
  * allocation is all-or-nothing: too few free blocks raises NoFreeBlocks
    and leaves the state untouched;
  * sharing a block (prefix reuse) raises its reference count; sharing a free
    block, or freeing more references than a block holds, is an invalid
    argument, detected for the whole request before anything changes.
"""
from __future__ import annotations

from collections import deque


class NoFreeBlocks(Exception):
    pass


class InvalidArgument(Exception):
    pass


class OracleAllocator:
    def __init__(self, num_blocks: int, initial_order=None):
        if num_blocks < 0:
            raise InvalidArgument("num_blocks < 0")
        order = list(range(num_blocks)) if initial_order is None else [int(x) for x in initial_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidArgument("initial_order must be a permutation of 0..N-1")
        self.num_blocks = num_blocks
        self.free_block_queue = deque(order)
        self.refcount = [0] * num_blocks

    @property
    def num_free(self) -> int:
        return len(self.free_block_queue)

    def allocate(self, n: int) -> list:
        if n < 0:
            raise InvalidArgument("n < 0")
        if n > len(self.free_block_queue):
            raise NoFreeBlocks(f"need {n}, have {len(self.free_block_queue)}")
        ids = [self.free_block_queue.popleft() for _ in range(n)]
        for i in ids:
            self.refcount[i] = 1
        return ids

    def share(self, ids) -> None:
        ids = [int(i) for i in ids]
        for i in ids:
            if not (0 <= i < self.num_blocks) or self.refcount[i] == 0:
                raise InvalidArgument(f"block {i} is not allocated")
        for i in ids:
            self.refcount[i] += 1

    def free(self, ids) -> None:
        ids = [int(i) for i in ids]
        want = {}
        for i in ids:
            if not (0 <= i < self.num_blocks):
                raise InvalidArgument(f"block {i} out of range")
            want[i] = want.get(i, 0) + 1
        for i, k in want.items():
            if k > self.refcount[i]:
                raise InvalidArgument(f"block {i} freed {k} times, holds {self.refcount[i]}")
        for i in ids:
            self.refcount[i] -= 1
            if self.refcount[i] == 0:
                self.free_block_queue.append(i)

    def export(self):
        """(queue head..tail, refcounts) -- the whole allocator state."""
        return list(self.free_block_queue), list(self.refcount)

    def stats(self, seq_lens, block_size: int):
        """(blocks in use, tail waste in tokens): the last block of a sequence
        of L tokens leaves ceil(L/bs)*bs - L slots unused (paging removes
        external, not internal, fragmentation)."""
        used = self.num_blocks - len(self.free_block_queue)
        waste = sum(-(-int(L) // block_size) * block_size - int(L) for L in seq_lens)
        return used, waste


def build_decode_block_tables(alloc, seq_lens, block_size: int, max_blocks=None):
    """Decode recipe: sequences 0..B-1 in order each take ceil(L/bs) blocks.
    Returns int32 [B, max_blocks] with -1 padding."""
    import numpy as np
    need = [-(-int(L) // block_size) for L in seq_lens]
    width = max(need + [1]) if max_blocks is None else max_blocks
    bt = np.full((len(seq_lens), width), -1, dtype=np.int32)
    for b, n in enumerate(need):
        bt[b, :n] = alloc.allocate(n)
    return bt


def build_prefill_block_tables(alloc, num_seqs: int, prefix_tokens: int,
                               own_tokens: int, block_size: int, share_prefix=True):
    """Prefix-sharing recipe: sequence 0 takes the prefix blocks; every other
    sequence shares them (share_prefix=True) or takes its own copy
    (share_prefix=False, sequence by sequence); then each sequence in order
    takes ceil(own_tokens/bs) blocks for its private suffix and chunk."""
    import numpy as np
    assert prefix_tokens % block_size == 0
    npre = prefix_tokens // block_size
    nown = -(-own_tokens // block_size)
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
