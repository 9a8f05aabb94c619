"""Builds the oracle side of a workload from the seeded draws (test harness).

Everything here goes through ``oracle`` only: its allocator, its slot mapping
and its reshape_and_cache fill the pool that the oracle then reads."""
from __future__ import annotations

import numpy as np

import oracle

NAN_BF16 = np.uint16(0x7FC0)
NAN_F32 = np.float32(np.nan)


def stored_dtype(wl):
    return np.float32 if wl.dtype == "f32" else np.uint16


def poison(wl):
    return NAN_F32 if wl.dtype == "f32" else NAN_BF16


class OracleSide:
    """Allocator state, block tables, slot mapping and the filled pool."""

    def __init__(self, d, share_prefix=True, seqs=None, fill_pool=True):
        wl = d.wl
        self.d, self.wl = d, wl
        bs = wl.block_size
        self.alloc = oracle.OracleAllocator(d.num_blocks, d.pool_order)
        if wl.kind == "prefill" and wl.prefix_tokens:
            own = int(d.seq_lens[0]) - wl.prefix_tokens
            self.block_tables = oracle.build_prefill_block_tables(
                self.alloc, wl.num_seqs, wl.prefix_tokens, own, bs, share_prefix)
        else:
            self.block_tables = oracle.build_decode_block_tables(self.alloc, d.seq_lens, bs)
        self.pool = None
        if fill_pool:
            self.fill(seqs)

    def slots_for(self, b, start, n):
        return oracle.slot_mapping(self.block_tables[b], start, n, self.wl.block_size)

    def fill(self, seqs=None):
        """Write every cached token of the selected sequences (all by default)
        through the oracle's reshape_and_cache; unwritten slots hold NaN."""
        wl, d = self.wl, self.d
        self.pool = oracle.empty_pool(d.num_blocks, wl.num_kv_heads, wl.block_size,
                                      wl.head_size, stored_dtype(wl), fill=poison(wl))
        written = set()
        for b in (range(wl.num_seqs) if seqs is None else seqs):
            L = int(d.seq_lens[b])
            k, v = d.kv(b)
            slots = self.slots_for(b, 0, L)
            # a shared prefix block is written once (the first sequence that owns it)
            keep = np.array([int(s) not in written for s in slots])
            slots = np.where(keep, slots, -1)
            written.update(int(s) for s in slots if s >= 0)
            oracle.reshape_and_cache(self.pool, k, v, slots)
        return self.pool

    def decode(self, scale=None, seqs=None):
        wl = self.wl
        return oracle.decode(self.d.query(), self.pool, self.block_tables, self.d.seq_lens,
                             wl.scale if scale is None else scale, seqs=seqs)

    def query_start_loc(self):
        return np.concatenate([[0], np.cumsum(self.wl.chunk_lens())]).astype(np.int32)

    def prefill(self, scale=None, seqs=None):
        wl = self.wl
        return oracle.prefill_chunk(self.d.query(), self.query_start_loc(), self.pool,
                                    self.block_tables, self.d.seq_lens,
                                    wl.scale if scale is None else scale, seqs=seqs)
