"""Oracle arithmetic of paged attention (float64, CPU) -- test infrastructure.

Sources (page titles and sections; the pages are the authority on what is
computed, and where they are silent the reading used is stated inline):

  [IV]  "Inside vLLM: Anatomy of a High-Throughput LLM Inference System",
        sections "LLM Engine & Engine Core" and "LLM Engine constructor".
  [IM]  "Im Inneren von vLLM: Anatomie eines Hochdurchsatz-LLM-Inferenz-
        systems", section "Paged Attention & KV-Cache".
  [TE]  "vLLM: Ein tiefer Einblick in die hochdurchsatzfähige LLM-Inferenz-
        und Serving-Engine auf Basis von PagedAttention", section
        "Tiefenanalyse".

What the pages fix: a KV-cache block holds keys and values of block_size
tokens for every KV head, so its size is 2 * block_size * num_kv_heads *
head_size * dtype_bytes ([IV] "LLM Engine constructor", [IM]); blocks are the
indexing structure from a sequence's tokens to where their keys/values live
([IV] "LLM Engine & Engine Core"); storage is non-contiguous, in the manner of
OS paging, and changes where K/V live but not what attention computes ([TE]).
The attention itself is only cited as the standard transformer's ([IV] "LLM
Engine & Engine Core"); the reading is scaled-dot-product softmax attention.

Readings taken where the pages are silent:
  * pool layout [num_blocks][2 (0=key, 1=value)][H_kv][block_size][D]: one
    block is exactly the formula's bytes and contiguous;
  * token p of a sequence lives at slot bt[p // bs] * bs + p % bs;
    a negative slot means "do not write";
  * query head h reads KV head h // (H_q / H_kv) (contiguous GQA groups);
  * a decode query is the last token of the sequence and sees all seq_len
    tokens, itself included; a prefill chunk of C queries is the last C
    tokens, query i at position seq_len - C + i sees tokens 0..that position;
  * softmax subtracts the row maximum; lse = m + ln(sum exp(s - m));
  * a sequence with seq_len 0 yields O = 0 and lse = -inf.
"""
from __future__ import annotations

import numpy as np

from .fp8 import e4m3_decode_array


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
def kv_block_bytes(block_size: int, num_kv_heads: int, head_size: int,
                   dtype_bytes: int) -> int:
    """Bytes of one KV-cache block of a standard (non-MLA) layer: keys and
    values (the factor 2) for block_size tokens of every KV head.
    [IV] "LLM Engine constructor"; [IM] "Paged Attention & KV-Cache"."""
    return 2 * block_size * num_kv_heads * head_size * dtype_bytes


def num_blocks_for_budget(budget_bytes: int, block_bytes: int, num_layers: int) -> int:
    """How many blocks fit in a memory budget when every layer needs one block
    per block id ([IV] "LLM Engine constructor": count how many KV-cache blocks
    fit in the VRAM left after the profiling pass).  Reading: round down."""
    if block_bytes <= 0 or num_layers <= 0:
        raise ValueError("block_bytes and num_layers must be positive")
    return budget_bytes // (block_bytes * num_layers)


# ---------------------------------------------------------------------------
# dtype handling: the oracle decodes stored values itself
# ---------------------------------------------------------------------------
def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact float64 value of stored elements: float32 arrays are widened;
    uint16 arrays are bf16 bit patterns (the top half of a float32); uint8
    arrays are FP8 E4M3 codes (oracle/fp8.py), before any scale."""
    x = np.asarray(x)
    if x.dtype == np.uint8:
        return e4m3_decode_array(x)
    if x.dtype == np.uint16:
        wide = x.astype(np.uint32) * np.uint32(65536)
        return wide.view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported element type {x.dtype}")


def empty_pool(num_blocks: int, num_kv_heads: int, block_size: int, head_size: int,
               dtype, fill=None) -> np.ndarray:
    """A pool [N][2][H_kv][bs][D] of the stored element type.  ``fill`` is a
    stored value (e.g. a NaN bit pattern) for slots nobody writes."""
    pool = np.zeros((num_blocks, 2, num_kv_heads, block_size, head_size), dtype=dtype)
    if fill is not None:
        pool[...] = fill
    return pool


# ---------------------------------------------------------------------------
# token -> slot
# ---------------------------------------------------------------------------
def slot_mapping(block_table_row, start_pos: int, num_tokens: int,
                 block_size: int) -> np.ndarray:
    """Physical slots of logical positions start_pos .. start_pos+num_tokens-1
    of one sequence: the block table maps logical block p // bs to a physical
    block, and the token sits at offset p % bs in it ([IV] "LLM Engine & Engine
    Core": blocks map tokens to their KV-cache blocks)."""
    out = np.empty(num_tokens, dtype=np.int64)
    for i in range(num_tokens):
        p = start_pos + i
        phys = int(block_table_row[p // block_size])
        if phys < 0:
            raise ValueError(f"position {p} has no block in the table")
        out[i] = phys * block_size + p % block_size
    return out


def reshape_and_cache(pool: np.ndarray, key: np.ndarray, value: np.ndarray,
                      slots: np.ndarray) -> np.ndarray:
    """Write token t's key/value rows [H_kv, D] into the pool at slot slots[t];
    a negative slot is skipped.  Values are copied unchanged (no arithmetic).
    Two tokens writing one slot would race, so distinct slots are required."""
    n_blocks, two, n_kv, bs, d = pool.shape
    assert two == 2 and key.shape == value.shape and key.shape[1:] == (n_kv, d)
    live = [int(s) for s in slots if s >= 0]
    assert len(live) == len(set(live)), "slot_mapping must not repeat a slot"
    for t, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        blk, off = divmod(s, bs)
        assert blk < n_blocks
        pool[blk, 0, :, off, :] = key[t]
        pool[blk, 1, :, off, :] = value[t]
    return pool


def gather_kv(pool: np.ndarray, block_table_row, seq_len: int):
    """Logical keys/values [seq_len, H_kv, D] of one sequence, read through its
    block table, as float64."""
    n_blocks, _, n_kv, bs, d = pool.shape
    K = np.empty((seq_len, n_kv, d), dtype=np.float64)
    V = np.empty((seq_len, n_kv, d), dtype=np.float64)
    for j in range(-(-seq_len // bs)):
        phys = int(block_table_row[j])
        assert 0 <= phys < n_blocks, "block table entry out of range"
        lo, hi = j * bs, min((j + 1) * bs, seq_len)
        rows = hi - lo
        # pool[phys, 0] is [H_kv, bs, D]; tokens run along the bs axis
        K[lo:hi] = to_f64(pool[phys, 0, :, :rows, :]).transpose(1, 0, 2)
        V[lo:hi] = to_f64(pool[phys, 1, :, :rows, :]).transpose(1, 0, 2)
    return K, V


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Scaled-dot-product softmax attention of query rows q [R, D] over keys
    K [L, D] and values V [L, D] (float64).  Returns (O [R, D], lse [R]) with
    lse the natural-log normaliser.  L == 0 gives O = 0 and lse = -inf."""
    q = np.asarray(q, dtype=np.float64)
    R, D = q.shape
    L = K.shape[0]
    if L == 0:
        return np.zeros((R, D)), np.full(R, -np.inf)
    s = float(scale) * (q @ K.T)                     # [R, L]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    denom = e.sum(axis=1, keepdims=True)
    p = e / denom
    assert np.all(np.abs(p.sum(axis=1) - 1.0) <= 1e-12), "softmax rows must sum to 1"
    return p @ V, m[:, 0] + np.log(denom[:, 0])


def decode(query: np.ndarray, pool: np.ndarray, block_tables: np.ndarray,
           seq_lens, scale: float, seqs=None, k_scale: float = 1.0,
           v_scale: float = 1.0):
    """One query token per sequence (the sequence's last token, already in the
    cache) attending to all seq_len[b] cached tokens through its block table.

    query [B, H_q, D] (stored dtype), pool [N][2][H_kv][bs][D],
    block_tables int32 [B, max_blocks] (padding entries are never read).
    Returns (out [B, H_q, D] float64, lse [B, H_q] float64); ``seqs`` limits
    the work to a subset of sequences (other rows stay NaN).  An FP8 pool
    holds codes: keys and values are their values times k_scale / v_scale."""
    B, Hq, D = query.shape
    Hkv = pool.shape[2]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    out = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_lens[b])
        K, V = gather_kv(pool, block_tables[b], L)
        K, V = K * float(k_scale), V * float(v_scale)
        qb = to_f64(query[b])
        for g in range(Hkv):
            heads = slice(g * G, (g + 1) * G)          # query heads of KV head g
            o, l = attention(qb[heads], K[:, g, :], V[:, g, :], scale)
            out[b, heads] = o
            lse[b, heads] = l
    return out, lse


def prefill_chunk(query: np.ndarray, query_start_loc, pool: np.ndarray,
                  block_tables: np.ndarray, seq_lens, scale: float, seqs=None,
                  k_scale: float = 1.0, v_scale: float = 1.0):
    """A causal chunk per sequence: the C_b = qsl[b+1] - qsl[b] query tokens of
    sequence b are its last C_b tokens (their keys/values already written);
    query i sits at position seq_len[b] - C_b + i and sees tokens 0..position.

    query is packed [sum C_b, H_q, D].  Returns out [sum C_b, H_q, D] and
    lse [sum C_b, H_q] in float64.  An FP8 pool holds codes: keys and values
    are their values times k_scale / v_scale, as in decode()."""
    T, Hq, D = query.shape
    Hkv = pool.shape[2]
    G = Hq // Hkv
    out = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    B = len(seq_lens)
    for b in (range(B) if seqs is None else seqs):
        lo, hi = int(query_start_loc[b]), int(query_start_loc[b + 1])
        C, L = hi - lo, int(seq_lens[b])
        assert 0 <= C <= L
        K, V = gather_kv(pool, block_tables[b], L)
        K, V = K * float(k_scale), V * float(v_scale)
        for i in range(C):
            pos = L - C + i
            qi = to_f64(query[lo + i])
            for g in range(Hkv):
                heads = slice(g * G, (g + 1) * G)
                o, l = attention(qi[heads], K[:pos + 1, g, :], V[:pos + 1, g, :], scale)
                out[lo + i, heads] = o
                lse[lo + i, heads] = l
    return out, lse
