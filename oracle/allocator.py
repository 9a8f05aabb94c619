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

Prefix cache ([IM] "Fortgeschrittene Funktionen", [TE] "Tiefenanalyse": the
KV cache of common prompt prefixes is stored and reused).  The pages give no
mechanism.  Readings, written here as plainly as possible:
  * only full blocks are cached; block j of a token list holds the keys and
    values of tokens [j*bs, (j+1)*bs), which depend on every token before
    them, so the cache key of that block is the whole prefix
    tokens[0 : (j+1)*bs] (a tuple; Python's dict compares it exactly);
  * a freed block keeps its cached contents while it waits in the queue;
    allocate() popping it means new contents, so its key is dropped;
  * acquire(tokens) walks j = 0, 1, ... and stops at the first uncached key;
    each hit gains a reference, and a hit on a free block takes it out of
    the queue;
  * insert(tokens, ids) caches block ids[j] under key j unless that key is
    cached already; an id that is free, repeated or caching another key is
    an invalid argument, detected before anything changes.
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
        self.cache_block_size = 0          # prefix cache off
        self.cached = {}                   # prefix tuple -> block id
        self.block_key = [None] * num_blocks
        self.hits = 0
        self.evictions = 0

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
            if self.block_key[i] is not None:   # cached free block: evicted
                del self.cached[self.block_key[i]]
                self.block_key[i] = None
                self.evictions += 1
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

    # prefix cache -----------------------------------------------------------
    def enable_prefix_cache(self, block_size: int) -> None:
        if block_size <= 0:
            raise InvalidArgument("block_size <= 0")
        if self.cache_block_size not in (0, block_size):
            raise InvalidArgument("prefix cache enabled with another block size")
        self.cache_block_size = block_size

    def _key(self, tokens, j):
        bs = self.cache_block_size
        return tuple(int(t) for t in tokens[:(j + 1) * bs])

    def acquire(self, tokens) -> list:
        if not self.cache_block_size:
            raise InvalidArgument("prefix cache not enabled")
        hit = []
        for j in range(len(tokens) // self.cache_block_size):
            key = self._key(tokens, j)
            if key not in self.cached:
                break
            b = self.cached[key]
            if self.refcount[b] == 0:
                self.free_block_queue.remove(b)
            self.refcount[b] += 1
            hit.append(b)
        self.hits += len(hit)
        return hit

    def insert(self, tokens, ids) -> None:
        if not self.cache_block_size:
            raise InvalidArgument("prefix cache not enabled")
        full = len(tokens) // self.cache_block_size
        ids = [int(i) for i in ids]
        if len(ids) < full:
            raise InvalidArgument("fewer block ids than full blocks")
        ids = ids[:full]
        if len(set(ids)) != len(ids):
            raise InvalidArgument("block listed twice")
        for j, b in enumerate(ids):
            if not (0 <= b < self.num_blocks) or self.refcount[b] == 0:
                raise InvalidArgument(f"block {b} is not allocated")
            if self.block_key[b] is not None and self.block_key[b] != self._key(tokens, j):
                raise InvalidArgument(f"block {b} caches another prefix")
        for j, b in enumerate(ids):
            key = self._key(tokens, j)
            if key not in self.cached:
                self.cached[key] = b
                self.block_key[b] = key

    def export_prefix_cache(self):
        """(cached flag per block, (cached blocks, hit blocks, evictions))."""
        flags = [0 if k is None else 1 for k in self.block_key]
        return flags, (len(self.cached), self.hits, self.evictions)

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
