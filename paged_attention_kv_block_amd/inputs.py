"""Seeded synthetic inputs for the paged-attention workloads.

This module only draws numbers: sequence lengths, the initial order of the
free-block pool, queries and the per-token keys/values that the cache will
hold.  It contains none of the method's arithmetic (no slot computation, no
block tables, no attention) so that the oracle and the HIP path can both be
fed from it without sharing any computation.

Workloads (one layer of attention, shapes only; no weights are involved):

  0  tiny fp32 decode: 2 sequences of 7 and 19 tokens, 4 query / 2 KV heads,
     head size 64, an 8-block pool in a seeded random order.
  1  TinyLlama-1.1B-shaped decode, bf16: 64 sequences, 32 query / 4 KV heads,
     head size 64, lengths uniform in [128, 2048], pool = 110 % of need.
  2  Llama-3-8B-shaped decode, bf16: 256 sequences, 32 / 8 heads, head size
     128, lengths log-normal (median 1024, sigma 1.0) clipped to [64, 8192],
     512-token split-K partitions.
  3  chunked prefill with a shared prefix, bf16: 16 sequences share a
     2048-token prefix, each has a private 512-token suffix and runs a
     256-token causal chunk; 32 / 8 heads, head size 128.
  4  long-context decode, bf16: 16 sequences, 64 / 8 heads, head size 128,
     lengths uniform in [32768, 131072], 1024-token partitions.

Every value is drawn from numpy's PCG64 under SeedSequence(1000 + index);
children are spawned in a fixed order (lengths, pool order, queries, keys and
values) and every sequence has its own key/value stream, so any subset of
sequences can be regenerated alone.  Floating values are N(0, 1) float32;
bf16 workloads round them to bf16 with round-to-nearest-even, and both sides
receive the rounded values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BLOCK_SIZE = 16


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    kind: str                 # "decode" or "prefill"
    dtype: str                # "f32" or "bf16"
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int = BLOCK_SIZE
    partition_size: int = 0   # 0: no split-K requested by the workload
    # decode: length distribution
    len_dist: str = "fixed"   # "fixed", "uniform", "lognormal"
    len_lo: int = 0
    len_hi: int = 0
    fixed_lens: tuple = ()
    # prefill: prefix sharing geometry (tokens)
    prefix_tokens: int = 0
    private_tokens: int = 0
    chunk_tokens: int = 0
    fixed_chunks: tuple = ()  # prefill: per-sequence chunk lengths (ragged)
    # pool
    fixed_num_blocks: int = 0  # 0: ceil(1.1 * blocks needed)

    def chunk_lens(self) -> tuple:
        if self.fixed_chunks:
            return tuple(self.fixed_chunks)
        return (self.chunk_tokens,) * self.num_seqs

    @property
    def dtype_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def scale(self) -> np.float32:
        """Softmax scale as the float32 value both sides use: 1/sqrt(D)."""
        return np.float32(1.0 / math.sqrt(self.head_size))


WORKLOADS = {
    0: Workload(0, "tiny-fp32-decode", "decode", "f32", 2, 4, 2, 64,
                len_dist="fixed", fixed_lens=(7, 19), fixed_num_blocks=8),
    1: Workload(1, "tinyllama-1.1b-decode-b64", "decode", "bf16", 64, 32, 4, 64,
                len_dist="uniform", len_lo=128, len_hi=2048),
    2: Workload(2, "llama3-8b-decode-b256-splitk512", "decode", "bf16", 256, 32, 8, 128,
                partition_size=512, len_dist="lognormal", len_lo=64, len_hi=8192),
    3: Workload(3, "chunked-prefill-shared-prefix-b16", "prefill", "bf16", 16, 32, 8, 128,
                prefix_tokens=2048, private_tokens=512, chunk_tokens=256),
    4: Workload(4, "long-context-decode-b16-splitk1024", "decode", "bf16", 16, 64, 8, 128,
                partition_size=1024, len_dist="uniform", len_lo=32768, len_hi=131072),
}


def workload(index: int) -> Workload:
    return WORKLOADS[index]


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.

    Inputs here are finite normal draws, so no NaN handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


class Draw:
    """All seeded inputs of one workload.

    Attributes
      seq_lens     int32 [B]   tokens in each sequence's cache after this step
                               (decode: includes the query token itself)
      pool_order   int32 [N]   initial order of the free-block pool
      num_blocks   int         N
    Methods
      query()      decode: [B, H_q, D]; prefill: [B*C, H_q, D] (packed)
      kv(b)        (K, V), each [L_b, H_kv, D]: keys/values of sequence b's
                   tokens 0..L_b-1 in logical order (prefill: the shared prefix
                   positions hold the shared prefix values)
    Values are float32 for f32 workloads and uint16 bf16 bit patterns for bf16.
    """

    def __init__(self, wl: Workload, seed_offset: int = 1000):
        self.wl = wl
        ss = np.random.SeedSequence(seed_offset + wl.index)
        self._ss_len, self._ss_order, self._ss_q, self._ss_kv = ss.spawn(4)
        self._kv_children = self._ss_kv.spawn(wl.num_seqs + 1)
        self.seq_lens = self._draw_lengths()
        need = self.blocks_needed()
        if wl.fixed_num_blocks:
            self.num_blocks = wl.fixed_num_blocks
        else:
            self.num_blocks = int(math.ceil(1.1 * need))
        rng = np.random.Generator(np.random.PCG64(self._ss_order))
        self.pool_order = rng.permutation(self.num_blocks).astype(np.int32)

    # -- lengths -----------------------------------------------------------
    def _draw_lengths(self) -> np.ndarray:
        wl = self.wl
        rng = np.random.Generator(np.random.PCG64(self._ss_len))
        if wl.kind == "prefill":
            L = wl.prefix_tokens + wl.private_tokens + wl.chunk_tokens
            return np.full(wl.num_seqs, L, dtype=np.int32)
        if wl.len_dist == "fixed":
            return np.asarray(wl.fixed_lens, dtype=np.int32)
        if wl.len_dist == "uniform":
            return rng.integers(wl.len_lo, wl.len_hi, size=wl.num_seqs,
                                endpoint=True).astype(np.int32)
        if wl.len_dist == "lognormal":
            x = rng.lognormal(mean=math.log(1024.0), sigma=1.0, size=wl.num_seqs)
            return np.clip(np.rint(x), wl.len_lo, wl.len_hi).astype(np.int32)
        raise ValueError(wl.len_dist)

    def blocks_needed(self) -> int:
        """Distinct blocks the workload occupies (shared prefix counted once)."""
        wl, bs = self.wl, self.wl.block_size
        if wl.kind == "prefill":
            own = -(-(wl.private_tokens + wl.chunk_tokens) // bs)
            return -(-wl.prefix_tokens // bs) + wl.num_seqs * own
        return int(sum(-(-int(L) // bs) for L in self.seq_lens))

    # -- tensors -----------------------------------------------------------
    def _normal(self, rng: np.random.Generator, shape) -> np.ndarray:
        x = rng.standard_normal(size=shape, dtype=np.float32)
        return x if self.wl.dtype == "f32" else round_to_bf16_bits(x)

    def query(self) -> np.ndarray:
        wl = self.wl
        rng = np.random.Generator(np.random.PCG64(self._ss_q))
        rows = wl.num_seqs if wl.kind == "decode" else sum(wl.chunk_lens())
        return self._normal(rng, (rows, wl.num_q_heads, wl.head_size))

    def prefix_kv(self):
        """Prefill workload only: keys/values of the shared prefix tokens."""
        wl = self.wl
        rng = np.random.Generator(np.random.PCG64(self._kv_children[wl.num_seqs]))
        shp = (wl.prefix_tokens, wl.num_kv_heads, wl.head_size)
        return self._normal(rng, shp), self._normal(rng, shp)

    def own_kv(self, b: int):
        """Keys/values of sequence b's own (unshared) tokens."""
        wl = self.wl
        rng = np.random.Generator(np.random.PCG64(self._kv_children[b]))
        n = int(self.seq_lens[b]) - wl.prefix_tokens
        shp = (n, wl.num_kv_heads, wl.head_size)
        return self._normal(rng, shp), self._normal(rng, shp)

    def kv(self, b: int):
        k, v = self.own_kv(b)
        if self.wl.prefix_tokens:
            pk, pv = self.prefix_kv()
            k = np.concatenate([pk, k], axis=0)
            v = np.concatenate([pv, v], axis=0)
        return k, v


def draw(index: int, seed_offset: int = 1000) -> Draw:
    return Draw(workload(index), seed_offset)


def custom(name: str = "custom", *, kind: str = "decode", dtype: str = "bf16",
           seq_lens=(1,), num_q_heads: int = 4, num_kv_heads: int = 2,
           head_size: int = 64, num_blocks: Optional[int] = None,
           chunk_lens=(), seed: int = 7, index: int = 100) -> Draw:
    """A small ad-hoc workload for edge cases: fixed lengths, a chosen pool
    size and (prefill) per-sequence chunk lengths; no shared prefix."""
    wl = Workload(index, name, kind, dtype, len(seq_lens), num_q_heads, num_kv_heads,
                  head_size, len_dist="fixed", fixed_lens=tuple(seq_lens),
                  fixed_chunks=tuple(chunk_lens), fixed_num_blocks=num_blocks or 0)
    d = Draw.__new__(Draw)
    d.wl = wl
    ss = np.random.SeedSequence(seed)
    d._ss_len, d._ss_order, d._ss_q, d._ss_kv = ss.spawn(4)
    d._kv_children = d._ss_kv.spawn(wl.num_seqs + 1)
    d.seq_lens = np.asarray(seq_lens, dtype=np.int32)
    need = int(sum(-(-int(L) // wl.block_size) for L in d.seq_lens))
    d.num_blocks = num_blocks if num_blocks else max(1, int(math.ceil(1.1 * need)))
    rng = np.random.Generator(np.random.PCG64(d._ss_order))
    d.pool_order = rng.permutation(d.num_blocks).astype(np.int32)
    return d


def mixed_step(num_prefill: int = 16, prefill_context: int = 2560, chunk: int = 256,
               num_decode: int = 240, num_q_heads: int = 32, num_kv_heads: int = 8,
               head_size: int = 128, seed: int = 11, index: int = 105,
               decode_rows: int = 1) -> Draw:
    """One flattened step of continuous batching, Llama-3-8B-shaped heads:
    `num_prefill` sequences each run a `chunk`-token causal prefill chunk
    after `prefill_context` cached tokens (the chunked-prefill workload's
    geometry: 2048 + 512 tokens before a 256-token chunk, here without the
    shared prefix), followed by `num_decode` sequences with one query row
    each, lengths log-normal (median 1024, sigma 1.0) clipped to [64, 8192]
    like the Llama-3-8B-shaped decode batch.  Packed query rows: the chunks
    in sequence order, then the decode rows.  decode_rows > 1 gives each
    decode sequence that many rows (its last tokens, as a speculative step
    checks them); the lengths stay the same draws."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    x = rng.lognormal(mean=math.log(1024.0), sigma=1.0, size=num_decode)
    dec = np.clip(np.rint(x), 64, 8192).astype(np.int32)
    seq_lens = [prefill_context + chunk] * num_prefill + [int(v) for v in dec]
    chunks = [chunk] * num_prefill + [int(decode_rows)] * num_decode
    return custom("mixed-step", kind="prefill", seq_lens=seq_lens, chunk_lens=chunks,
                  num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_size=head_size,
                  seed=seed, index=index)


def token_stream_rows(tokens, num_heads: int, head_size: int, dtype: str = "bf16",
                      stream: int = 0, salt: int = 77) -> np.ndarray:
    """Rows [len(tokens), num_heads, head_size] drawn N(0,1) where row t depends
    only on tokens[0..t] (and the stream number): the seed of position t is
    SeedSequence([seed word of position t-1, tokens[t], stream]).  Two token
    lists with a common prefix get identical rows over that prefix, as keys
    and values computed by a causal model would; prefix-cache tests draw
    keys (stream 0), values (stream 1) and queries (stream 2) this way.
    float32 for "f32", bf16 bit patterns (uint16) otherwise."""
    out = np.empty((len(tokens), num_heads, head_size),
                   dtype=np.float32 if dtype == "f32" else np.uint16)
    word = salt
    for t, tok in enumerate(tokens):
        word = int(np.random.SeedSequence([word, int(tok)]).generate_state(1, np.uint64)[0])
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([word, stream])))
        x = rng.standard_normal(size=(num_heads, head_size), dtype=np.float32)
        out[t] = x if dtype == "f32" else round_to_bf16_bits(x)
    return out
