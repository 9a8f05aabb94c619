"""Builds the HIP side of a workload from the seeded draws (test harness).

Allocation, block tables and slot mapping go through libpa's host API; the
pool is filled on the GPU by pa_reshape_and_cache; attention runs through
pa_decode / pa_prefill_chunk.  Nothing here touches the oracle."""
from __future__ import annotations

import numpy as np
import torch

from paged_attention_kv_block_amd import host, ops

NAN_BF16_BITS = 0x7FC0


def torch_dtype(wl):
    return torch.float32 if wl.dtype == "f32" else torch.bfloat16


def to_device(arr: np.ndarray, wl, device="cuda"):
    """Seeded values (float32 or bf16 bit patterns) -> GPU tensor."""
    if wl.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr)).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.bfloat16)


def from_device(t) -> np.ndarray:
    """GPU tensor -> float32 (f32) or bf16 bit patterns (uint16) on the host."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def empty_pool(d, device="cuda", poison=True):
    wl = d.wl
    shape = (d.num_blocks, 2, wl.num_kv_heads, wl.block_size, wl.head_size)
    if wl.dtype == "f32":
        pool = torch.full(shape, float("nan") if poison else 0.0, dtype=torch.float32, device=device)
    else:
        pool = torch.full(shape, NAN_BF16_BITS if poison else 0, dtype=torch.int16, device=device)
        pool = pool.view(torch.bfloat16)
    return pool


class GpuSide:
    def __init__(self, d, share_prefix=True, fill=True, device="cuda"):
        wl = d.wl
        self.d, self.wl, self.device = d, wl, device
        bs = wl.block_size
        self.alloc = ops.Allocator(d.num_blocks, d.pool_order)
        if wl.kind == "prefill" and wl.prefix_tokens:
            own = int(d.seq_lens[0]) - wl.prefix_tokens
            self.block_tables = host.prefill_block_tables(self.alloc, wl.num_seqs, wl.prefix_tokens,
                                                          own, bs, share_prefix)
        else:
            self.block_tables = host.decode_block_tables(self.alloc, d.seq_lens, bs)
        self.bt_dev = torch.from_numpy(self.block_tables).to(device)
        self.seq_lens_dev = torch.from_numpy(np.ascontiguousarray(d.seq_lens, dtype=np.int32)).to(device)
        self.pool = None
        if fill:
            self.fill()

    def fill(self, seqs=None):
        """Writes every cached token of the selected sequences through
        pa_reshape_and_cache (shared prefix blocks once)."""
        wl, d = self.wl, self.d
        self.pool = empty_pool(d, self.device)
        written = set()
        ks, vs, slots = [], [], []
        for b in (range(wl.num_seqs) if seqs is None else seqs):
            L = int(d.seq_lens[b])
            k, v = d.kv(b)
            s = ops.slot_mapping(self.block_tables[b], 0, L, wl.block_size)
            keep = np.array([int(x) not in written for x in s], dtype=bool)
            s = np.where(keep, s, -1)
            written.update(int(x) for x in s if x >= 0)
            ks.append(k)
            vs.append(v)
            slots.append(s)
        if not ks:
            return self.pool
        key = to_device(np.concatenate(ks), wl, self.device)
        val = to_device(np.concatenate(vs), wl, self.device)
        sm = torch.from_numpy(np.concatenate(slots).astype(np.int64)).to(self.device)
        ops.reshape_and_cache(key, val, sm, self.pool)
        return self.pool

    def decode(self, partition_size=None, scale=None, with_lse=True, max_seq_len=None,
               use_plan=False):
        wl, d = self.wl, self.d
        q = to_device(d.query(), wl, self.device)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=self.device) if with_lse else None
        P = wl.partition_size if partition_size is None else partition_size
        msl = int(max(d.seq_lens)) if max_seq_len is None else max_seq_len
        ws = ops.decode_workspace(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_size, msl,
                                  P, self.device)
        plan = None
        if use_plan:
            plan = torch.from_numpy(ops.decode_plan(d.seq_lens, msl, P)).to(self.device)
        ops.decode(out, q, self.pool, self.bt_dev, self.seq_lens_dev, msl,
                   float(wl.scale if scale is None else scale), P, ws, lse, plan)
        torch.cuda.synchronize()
        return out, lse

    def query_start_loc(self):
        return np.concatenate([[0], np.cumsum(self.wl.chunk_lens())]).astype(np.int32)

    def prefill(self, scale=None, with_lse=True):
        wl, d = self.wl, self.d
        q = to_device(d.query(), wl, self.device)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=self.device) if with_lse else None
        qsl = self.query_start_loc()
        ops.prefill_chunk(out, q, torch.from_numpy(qsl).to(self.device), int(max(wl.chunk_lens())),
                          self.pool, self.bt_dev, self.seq_lens_dev, int(max(d.seq_lens)),
                          float(wl.scale if scale is None else scale), lse)
        torch.cuda.synchronize()
        return out, lse

    def varlen(self, partition_size=0, scale=None, with_lse=True, max_seq_len=None, out=None,
               workspace=None):
        """pa_attention_varlen over the packed rows (chunk lengths of the
        workload; a length of 1 makes a decode row)."""
        wl, d = self.wl, self.d
        q = to_device(d.query(), wl, self.device)
        if out is None:
            out = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=self.device) if with_lse else None
        qsl = self.query_start_loc()
        msl = int(max(d.seq_lens)) if max_seq_len is None else max_seq_len
        plan, npre = ops.varlen_plan(qsl, d.seq_lens, msl, wl.num_q_heads, wl.num_kv_heads,
                                     partition_size)
        ws = workspace
        if ws is None:
            ws = ops.decode_workspace(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_size,
                                      msl, partition_size, self.device)
        ops.attention_varlen(out, q, torch.from_numpy(qsl).to(self.device), self.pool, self.bt_dev,
                             self.seq_lens_dev, msl, float(wl.scale if scale is None else scale),
                             torch.from_numpy(plan).to(self.device), partition_size, ws, lse)
        torch.cuda.synchronize()
        return out, lse
