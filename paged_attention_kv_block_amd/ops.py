"""ctypes binding of libpa.so: argument marshalling only.

Every computation runs in the library: the host entry points (allocator, slot
mapping, closed forms) in its C++ part and the device entry points in its HIP
kernels.  Device arguments are torch tensors on the GPU; their data pointers
and the current torch stream are handed to the C ABI unchanged.  There is no
CPU fallback: if libpa.so is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa.so")

PA_OK, PA_EINVAL, PA_ENOBLOCKS, PA_ENOTSUP, PA_EHIP = 0, 1, 2, 3, 4
PA_F32, PA_BF16, PA_FP8 = 0, 1, 2
_STATUS = {PA_EINVAL: "EINVAL", PA_ENOBLOCKS: "ENOBLOCKS", PA_ENOTSUP: "ENOTSUP", PA_EHIP: "EHIP"}

# name -> (restype, argtypes); mirrors include/pa.h
_c_int, _c_i32, _c_i64, _c_u64, _c_sz = ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t
_vp, _f = ctypes.c_void_p, ctypes.c_float
SIGNATURES = {
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_version": (_c_int, []),
    "pa_kv_block_bytes": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32]),
    "pa_num_blocks_for_budget": (_c_i64, [_c_u64, _c_sz, _c_i32]),
    "pa_allocator_create": (_c_int, [_c_i32, _vp, ctypes.POINTER(_vp)]),
    "pa_allocator_destroy": (None, [_vp]),
    "pa_allocator_allocate": (_c_int, [_vp, _c_i32, _vp]),
    "pa_allocator_share": (_c_int, [_vp, _vp, _c_i32]),
    "pa_allocator_build_tables": (_c_int, [_vp, _vp, _c_i32, _c_i32, _c_i32, _vp]),
    "pa_allocator_free": (_c_int, [_vp, _vp, _c_i32]),
    "pa_allocator_num_free": (_c_i32, [_vp]),
    "pa_allocator_num_blocks": (_c_i32, [_vp]),
    "pa_allocator_export": (_c_int, [_vp, _vp, _vp]),
    "pa_allocator_stats": (_c_int, [_vp, _vp, _c_i32, _c_i32, _vp, _vp]),
    "pa_prefix_cache_enable": (_c_int, [_vp, _c_i32]),
    "pa_prefix_cache_acquire": (_c_int, [_vp, _vp, _c_i32, _vp, _vp]),
    "pa_prefix_cache_insert": (_c_int, [_vp, _vp, _c_i32, _vp, _c_i32]),
    "pa_prefix_cache_export": (_c_int, [_vp, _vp, _vp]),
    "pa_slot_mapping": (_c_int, [_vp, _c_i32, _vp, _vp, _c_i32, _c_i32, _vp, _vp]),
    "pa_reshape_and_cache": (_c_int, [_vp, _vp, _vp, _c_i32, _vp, _c_i32, _c_i32, _c_i32,
                                      _c_i32, _c_i32, _vp]),
    "pa_reshape_and_cache_fp8": (_c_int, [_vp, _vp, _vp, _c_i32, _vp, _c_i32, _c_i32, _c_i32,
                                          _c_i32, _f, _f, _vp]),
    "pa_decode_workspace_bytes": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "pa_decode_workspace_init": (_c_int, [_vp, _c_sz, _vp]),
    "pa_decode_plan": (_c_int, [_vp, _c_i32, _c_i32, _c_i32, _vp, _c_i32, _vp]),
    "pa_decode_step_prepare": (_c_int, [_vp, _vp, _c_i32, _vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                        _vp, _vp, _c_i32, _vp]),
    "pa_decode": (_c_int, [_vp, _vp, _vp, _vp, _c_i32, _vp, _c_i32, _vp, _c_i32, _c_i32,
                           _c_i32, _c_i32, _c_i32, _c_i32, _f, _c_i32, _vp, _c_i32, _vp, _c_sz,
                           _c_i32, _vp]),
    "pa_decode_append": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _vp, _c_i32, _vp,
                                  _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _f, _c_i32,
                                  _vp, _c_i32, _vp, _c_sz, _c_i32, _vp]),
    "pa_decode_append_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _vp, _c_i32, _vp,
                                          _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _f,
                                          _c_i32, _vp, _c_i32, _c_i32, _vp]),
    "pa_decode_fp8": (_c_int, [_vp, _vp, _vp, _vp, _c_i32, _vp, _c_i32, _vp, _c_i32, _c_i32,
                               _c_i32, _c_i32, _c_i32, _c_i32, _f, _f, _f, _c_i32, _vp, _c_i32,
                               _vp, _c_sz, _vp]),
    "pa_decode_append_fp8": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _vp, _c_i32, _vp,
                                      _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _f, _f, _f,
                                      _c_i32, _vp, _c_i32, _vp, _c_sz, _vp]),
    "pa_decode_multi_workspace_bytes": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                                _c_i32]),
    "pa_decode_multi": (_c_int, [_vp, _vp, _vp, _vp, _c_i32, _vp, _c_i32, _vp, _c_i32, _c_i32,
                                 _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _f, _c_i32, _vp, _c_i32,
                                 _vp, _c_sz, _c_i32, _vp]),
    "pa_decode_multi_fp8": (_c_int, [_vp, _vp, _vp, _vp, _c_i32, _vp, _c_i32, _vp, _c_i32,
                                     _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _f, _f, _f,
                                     _c_i32, _vp, _c_i32, _vp, _c_sz, _vp]),
    "pa_prefill_chunk": (_c_int, [_vp, _vp, _vp, _vp, _c_i32, _c_i32, _vp, _c_i32, _vp, _c_i32,
                                  _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _f,
                                  _c_i32, _vp]),
    "pa_varlen_plan": (_c_int, [_vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _c_i32,
                                _vp, _vp]),
    "pa_attention_varlen": (_c_int, [_vp, _vp, _vp, _vp, _c_i32, _vp, _c_i32, _vp, _c_i32, _vp,
                                     _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _f, _c_i32,
                                     _vp, _c_i32, _vp, _c_sz, _c_i32, _vp]),
    "pa_decode_graphs_create": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _vp,
                                         _c_i32, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _f,
                                         _c_i32, _vp, _c_sz, _c_i32, _vp, _c_i32, _vp,
                                         ctypes.POINTER(_vp)]),
    "pa_decode_graphs_replay": (_c_int, [_vp, _c_i32, _vp, _vp]),
    "pa_decode_graphs_count": (_c_i32, [_vp, _vp, _c_i32]),
    "pa_decode_graphs_destroy": (None, [_vp]),
}

_lib = None


class PAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


def lib(path: Optional[str] = None) -> ctypes.CDLL:
    """Loads libpa.so (built in-tree by paged_attention_kv_block_amd.build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with "
                           "`python -m paged_attention_kv_block_amd.build` (no CPU fallback)")
    L = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = L
    return L


def _check(status: int):
    if status != PA_OK:
        raise PAError(status, lib().pa_last_error().decode())


def _np_ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ---------------------------------------------------------------------------
# host entry points
# ---------------------------------------------------------------------------
def kv_block_bytes(block_size: int, num_kv_heads: int, head_size: int, dtype_bytes: int) -> int:
    return int(lib().pa_kv_block_bytes(block_size, num_kv_heads, head_size, dtype_bytes))


def num_blocks_for_budget(budget_bytes: int, block_bytes: int, num_layers: int) -> int:
    n = int(lib().pa_num_blocks_for_budget(budget_bytes, block_bytes, num_layers))
    if n < 0:
        raise PAError(PA_EINVAL, "block_bytes and num_layers must be positive")
    return n


class NoFreeBlocks(PAError):
    pass


class Allocator:
    """The free_block_queue allocator of libpa (FIFO, ref-counted)."""

    def __init__(self, num_blocks: int, initial_order: Optional[Sequence[int]] = None):
        self._h = ctypes.c_void_p()
        order = None if initial_order is None else np.ascontiguousarray(initial_order, dtype=np.int32)
        _check(lib().pa_allocator_create(int(num_blocks), None if order is None else _np_ptr(order),
                                         ctypes.byref(self._h)))

    def close(self):
        if self._h:
            lib().pa_allocator_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def allocate(self, n: int) -> list:
        out = np.empty(max(int(n), 1), dtype=np.int32)
        st = lib().pa_allocator_allocate(self._h, int(n), _np_ptr(out))
        if st == PA_ENOBLOCKS:
            raise NoFreeBlocks(st, lib().pa_last_error().decode())
        _check(st)
        return out[:max(int(n), 0)].tolist()

    def build_tables(self, seq_lens, block_size: int, width: Optional[int] = None) -> np.ndarray:
        """int32 [B, width] block tables of a batch, allocated in one call
        (sequence order, -1 padding; width defaults to the longest row)."""
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        need = -(-sl.astype(np.int64) // int(block_size)) if sl.size else np.zeros(0, np.int64)
        w = int(max(int(need.max()) if sl.size else 0, 1)) if width is None else int(width)
        out = np.empty((sl.size, max(w, 1)), dtype=np.int32)
        st = lib().pa_allocator_build_tables(self._h, _np_ptr(sl), sl.size, int(block_size), w,
                                             _np_ptr(out))
        if st == PA_ENOBLOCKS:
            raise NoFreeBlocks(st, lib().pa_last_error().decode())
        _check(st)
        return out[:, :w]

    def share(self, ids) -> None:
        a = np.ascontiguousarray(ids, dtype=np.int32)
        _check(lib().pa_allocator_share(self._h, _np_ptr(a), a.size))

    def free(self, ids) -> None:
        a = np.ascontiguousarray(ids, dtype=np.int32)
        _check(lib().pa_allocator_free(self._h, _np_ptr(a), a.size))

    @property
    def num_free(self) -> int:
        return int(lib().pa_allocator_num_free(self._h))

    @property
    def num_blocks(self) -> int:
        return int(lib().pa_allocator_num_blocks(self._h))

    def export(self):
        q = np.empty(max(self.num_free, 1), dtype=np.int32)
        rc = np.empty(max(self.num_blocks, 1), dtype=np.int32)
        _check(lib().pa_allocator_export(self._h, _np_ptr(q), _np_ptr(rc)))
        return q[:self.num_free].tolist(), rc[:self.num_blocks].tolist()

    def stats(self, seq_lens, block_size: int):
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        used, waste = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().pa_allocator_stats(self._h, _np_ptr(sl), sl.size, int(block_size),
                                        ctypes.byref(used), ctypes.byref(waste)))
        return used.value, waste.value

    # prefix cache ---------------------------------------------------------
    def enable_prefix_cache(self, block_size: int) -> None:
        _check(lib().pa_prefix_cache_enable(self._h, int(block_size)))

    def acquire_prefix(self, tokens) -> list:
        """Ids of the cached blocks of the longest cached prefix (referenced)."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        out = np.empty(max(t.size, 1), dtype=np.int32)   # >= full blocks for any block size
        hit = ctypes.c_int32()
        _check(lib().pa_prefix_cache_acquire(self._h, _np_ptr(t), t.size, _np_ptr(out),
                                             ctypes.byref(hit)))
        return out[:hit.value].tolist()

    def insert_prefix(self, tokens, block_ids) -> None:
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        ids = np.ascontiguousarray(block_ids, dtype=np.int32)
        _check(lib().pa_prefix_cache_insert(self._h, _np_ptr(t), t.size, _np_ptr(ids), ids.size))

    def export_prefix_cache(self):
        """(cached flag per block, (cached blocks, hit blocks, evictions))."""
        c = np.empty(max(self.num_blocks, 1), dtype=np.int32)
        st = np.empty(3, dtype=np.int64)
        _check(lib().pa_prefix_cache_export(self._h, _np_ptr(c), _np_ptr(st)))
        return c[:self.num_blocks].tolist(), tuple(int(x) for x in st)


def slot_mapping(block_tables: np.ndarray, start_pos, num_tokens, block_size: int) -> np.ndarray:
    """Slots (int64) of positions start_pos[b] .. +num_tokens[b] for every b."""
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    if bt.ndim == 1:
        bt = bt[None]
    sp = np.ascontiguousarray(np.broadcast_to(start_pos, (bt.shape[0],)), dtype=np.int32)
    nt = np.ascontiguousarray(np.broadcast_to(num_tokens, (bt.shape[0],)), dtype=np.int32)
    out = np.empty(max(int(nt.sum()), 1), dtype=np.int64)
    total = ctypes.c_int64()
    _check(lib().pa_slot_mapping(_np_ptr(bt), bt.shape[1], _np_ptr(sp), _np_ptr(nt), bt.shape[0],
                                 int(block_size), _np_ptr(out), ctypes.byref(total)))
    return out[:total.value]


# ---------------------------------------------------------------------------
# device entry points (torch tensors on the GPU)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype == torch.float32:
        return PA_F32
    raise PAError(PA_ENOTSUP, f"element type {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need_gpu(*ts):
    """Every device argument (None = not given) must be a dense GPU tensor:
    the library reads each as packed rows from its data pointer, so a strided
    view (a slice of a fused QKV tensor, a transposed plan) would be read
    wrongly rather than refused."""
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise PAError(PA_EINVAL, "tensors must be contiguous")
    for t in ts:
        if t is not None and not t.is_cuda:
            raise PAError(PA_EINVAL, "device arguments must be GPU tensors")


def reshape_and_cache(key, value, slot_mapping, kv_cache, stream=None) -> None:
    """key/value [T, H_kv, D]; slot_mapping int64 [T]; kv_cache [N, 2, H_kv, 16, D]."""
    _need_gpu(key, value, slot_mapping, kv_cache)
    N, two, Hkv, bs, D = kv_cache.shape
    if two != 2 or key.shape != value.shape or tuple(key.shape[1:]) != (Hkv, D) \
            or key.dtype != kv_cache.dtype or value.dtype != kv_cache.dtype:
        raise PAError(PA_EINVAL, "shape/dtype mismatch between key/value and kv_cache")
    if slot_mapping.dtype != _torch().int64 or slot_mapping.numel() != key.shape[0]:
        raise PAError(PA_EINVAL, "slot_mapping must be int64 [T]")
    _check(lib().pa_reshape_and_cache(_ptr(key), _ptr(value), _ptr(slot_mapping), key.shape[0],
                                      _ptr(kv_cache), N, bs, Hkv, D, _dtype_code(kv_cache),
                                      _stream(stream)))


def reshape_and_cache_fp8(key, value, slot_mapping, kv_cache, k_scale: float, v_scale: float,
                          stream=None) -> None:
    """key/value bf16 [T, H_kv, D]; slot_mapping int64 [T]; kv_cache uint8
    [N, 2, H_kv, 16, D] holding FP8 E4M3 codes (code * scale = value)."""
    torch = _torch()
    _need_gpu(key, value, slot_mapping, kv_cache)
    N, two, Hkv, bs, D = kv_cache.shape
    if two != 2 or key.shape != value.shape or tuple(key.shape[1:]) != (Hkv, D) \
            or key.dtype != torch.bfloat16 or value.dtype != torch.bfloat16 \
            or kv_cache.dtype != torch.uint8:
        raise PAError(PA_EINVAL, "key/value must be bf16 [T, H_kv, D], kv_cache uint8")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != key.shape[0]:
        raise PAError(PA_EINVAL, "slot_mapping must be int64 [T]")
    _check(lib().pa_reshape_and_cache_fp8(_ptr(key), _ptr(value), _ptr(slot_mapping), key.shape[0],
                                          _ptr(kv_cache), N, bs, Hkv, D, float(k_scale),
                                          float(v_scale), _stream(stream)))


def decode_workspace_bytes(B: int, num_q_heads: int, num_kv_heads: int, head_size: int,
                           max_seq_len: int, partition_size: int) -> int:
    return int(lib().pa_decode_workspace_bytes(B, num_q_heads, num_kv_heads, head_size,
                                               max_seq_len, partition_size))


def decode_workspace_init(workspace, stream=None) -> None:
    """Zero-fills a decode workspace (uint8 GPU tensor) on the stream."""
    _need_gpu(workspace)
    _check(lib().pa_decode_workspace_init(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                          _stream(stream)))


def decode_workspace(B: int, num_q_heads: int, num_kv_heads: int, head_size: int,
                     max_seq_len: int, partition_size: int, device="cuda", stream=None):
    """A zeroed workspace for pa_decode (at least 256 bytes; torch allocates it)."""
    torch = _torch()
    n = decode_workspace_bytes(B, num_q_heads, num_kv_heads, head_size, max_seq_len, partition_size)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    decode_workspace_init(ws, stream)
    return ws


def decode_plan(seq_lens_host, max_seq_len: int, partition_size: int) -> np.ndarray:
    """Host-built work list of pa_decode (int32 entries, longest first)."""
    sl = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    n = ctypes.c_int32()
    lib().pa_decode_plan(_np_ptr(sl), sl.size, int(max_seq_len), int(partition_size), None, 0,
                         ctypes.byref(n))
    out = np.empty(max(n.value, 1), dtype=np.int32)
    _check(lib().pa_decode_plan(_np_ptr(sl), sl.size, int(max_seq_len), int(partition_size),
                                _np_ptr(out), out.size, ctypes.byref(n)))
    return out[:n.value]


def decode_step_prepare(allocator: "Allocator", block_tables: np.ndarray, seq_lens: np.ndarray,
                        block_size: int, max_seq_len: int, partition_size: int,
                        slots: np.ndarray, plan: Optional[np.ndarray] = None) -> int:
    """pa_decode_step_prepare: one token more for every sequence (a block
    from the free queue where the token opens one), the new tokens' slots and
    the decode plan of the new lengths, in one native call.  block_tables
    (int32 [B, width]) and seq_lens (int32 [B]) are updated in place; slots
    (int64 [B]) and plan (int32, any capacity, or None) are written.
    Returns the number of plan entries."""
    for arr, dt, nd in ((block_tables, np.int32, 2), (seq_lens, np.int32, 1), (slots, np.int64, 1)):
        if not isinstance(arr, np.ndarray) or arr.dtype != dt or arr.ndim != nd \
                or not arr.flags.c_contiguous or not arr.flags.writeable:
            raise PAError(PA_EINVAL, "block_tables/seq_lens/slots must be writable C-contiguous "
                                     "int32 [B, width] / int32 [B] / int64 [B] arrays")
    B = seq_lens.size
    if block_tables.shape[0] != B or slots.size != B:
        raise PAError(PA_EINVAL, "block_tables, seq_lens and slots need B rows")
    if plan is not None and (plan.dtype != np.int32 or not plan.flags.c_contiguous
                             or not plan.flags.writeable):
        raise PAError(PA_EINVAL, "plan must be a writable C-contiguous int32 array")
    n = ctypes.c_int32()
    _check(lib().pa_decode_step_prepare(
        allocator._h, _np_ptr(block_tables), block_tables.shape[1], _np_ptr(seq_lens), B,
        int(block_size), int(max_seq_len), int(partition_size), _np_ptr(slots),
        None if plan is None else _np_ptr(plan), 0 if plan is None else plan.size,
        ctypes.byref(n)))
    return n.value


class DecodeStep:
    """The host half of successive decode steps over fixed arrays: the
    arguments of pa_decode_step_prepare are checked and marshalled once, and
    each prepare() is one native call.  block_tables (int32 [B, width]) and
    seq_lens (int32 [B]) are updated in place; after prepare(), slots (int64
    [B]) holds the new tokens' slots and plan[:n] the decode plan, n being
    the value returned."""

    def __init__(self, allocator: "Allocator", block_tables: np.ndarray, seq_lens: np.ndarray,
                 block_size: int, max_seq_len: int, partition_size: int):
        for arr, nd in ((block_tables, 2), (seq_lens, 1)):
            if not isinstance(arr, np.ndarray) or arr.dtype != np.int32 or arr.ndim != nd \
                    or not arr.flags.c_contiguous or not arr.flags.writeable:
                raise PAError(PA_EINVAL, "block_tables/seq_lens must be writable C-contiguous "
                                         "int32 [B, width] / [B] arrays")
        B = seq_lens.size
        if block_tables.shape[0] != B:
            raise PAError(PA_EINVAL, "block_tables and seq_lens need B rows")
        parts = 1 if partition_size <= 0 or max_seq_len <= 0 else -(-int(max_seq_len) //
                                                                      int(partition_size))
        self.block_tables, self.seq_lens = block_tables, seq_lens
        self.slots = np.zeros(B, np.int64)
        self.plan = np.zeros(max(1, B * parts), np.int32)
        self._allocator = allocator
        self._n = ctypes.c_int32()
        self._fn = lib().pa_decode_step_prepare
        self._args = (allocator._h, _np_ptr(block_tables), block_tables.shape[1],
                      _np_ptr(seq_lens), B, int(block_size), int(max_seq_len),
                      int(partition_size), _np_ptr(self.slots), _np_ptr(self.plan),
                      self.plan.size, ctypes.byref(self._n))

    def prepare(self) -> int:
        _check(self._fn(*self._args))
        return self._n.value


def decode(out, query, kv_cache, block_tables, seq_lens, max_seq_len: int, scale: float,
           partition_size: int = 0, workspace=None, lse=None, plan=None, stream=None,
           new_key=None, new_value=None) -> None:
    """out/query [B, H_q, D]; kv_cache [N, 2, H_kv, 16, D]; block_tables int32
    [B, max_blocks]; seq_lens int32 [B]; lse fp32 [B, H_q] or None;
    workspace a uint8 GPU tensor of decode_workspace_bytes(...) bytes; plan an
    int32 GPU tensor holding decode_plan(...) for the same lengths, or None.
    With new_key/new_value ([B, H_kv, D]) the call is pa_decode_append: the
    new token of each sequence is written into the cache in the same launch."""
    _need_gpu(out, query, kv_cache, block_tables, seq_lens, workspace, lse, plan, new_key,
              new_value)
    torch = _torch()
    N, _, Hkv, bs, D = kv_cache.shape
    B, Hq, Dq = query.shape
    if Dq != D or tuple(out.shape) != (B, Hq, D) or out.dtype != kv_cache.dtype \
            or query.dtype != kv_cache.dtype:
        raise PAError(PA_EINVAL, "shape/dtype mismatch between out/query and kv_cache")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32 \
            or block_tables.shape[0] != B or seq_lens.numel() != B:
        raise PAError(PA_EINVAL, "block_tables/seq_lens must be int32 with B rows")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq)):
        raise PAError(PA_EINVAL, "lse must be fp32 [B, H_q]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if plan is not None and plan.dtype != torch.int32:
        raise PAError(PA_EINVAL, "plan must be int32")
    tail = (N, _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), B, int(max_seq_len),
            Hq, Hkv, D, bs, float(scale), int(partition_size), _ptr(plan),
            0 if plan is None else plan.numel(), _ptr(workspace), ws_bytes,
            _dtype_code(kv_cache), _stream(stream))
    if new_key is None and new_value is None:
        _check(lib().pa_decode(_ptr(out), _ptr(lse), _ptr(query), _ptr(kv_cache), *tail))
        return
    for t in (new_key, new_value):
        if t is None or tuple(t.shape) != (B, Hkv, D) or t.dtype != kv_cache.dtype \
                or not t.is_contiguous():
            raise PAError(PA_EINVAL, "new_key/new_value must be contiguous [B, H_kv, D] "
                                     "in the cache dtype")
    _check(lib().pa_decode_append(_ptr(out), _ptr(lse), _ptr(query), _ptr(new_key),
                                  _ptr(new_value), _ptr(kv_cache), *tail))


NOALLOC_SCRATCH_BYTES = 128 << 20   # PA_NOALLOC_SCRATCH_BYTES


def decode_append_noalloc(out, query, kv_cache, block_tables, seq_lens, max_seq_len: int,
                          scale: float, new_key, new_value, partition_size: int = 0, lse=None,
                          plan=None, stream=None) -> None:
    """pa_decode_append_noalloc: decode(..., new_key=, new_value=) without a
    workspace; split-K runs in the library's static device scratch
    (NOALLOC_SCRATCH_BYTES per device, shared by all such calls on a device:
    calls that overlap on one GPU race)."""
    _need_gpu(out, query, kv_cache, block_tables, seq_lens, lse, plan, new_key, new_value)
    torch = _torch()
    N, _, Hkv, bs, D = kv_cache.shape
    B, Hq, Dq = query.shape
    if Dq != D or tuple(out.shape) != (B, Hq, D) or out.dtype != kv_cache.dtype \
            or query.dtype != kv_cache.dtype:
        raise PAError(PA_EINVAL, "shape/dtype mismatch between out/query and kv_cache")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32 \
            or block_tables.shape[0] != B or seq_lens.numel() != B:
        raise PAError(PA_EINVAL, "block_tables/seq_lens must be int32 with B rows")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq)):
        raise PAError(PA_EINVAL, "lse must be fp32 [B, H_q]")
    if plan is not None and plan.dtype != torch.int32:
        raise PAError(PA_EINVAL, "plan must be int32")
    for t in (new_key, new_value):
        if tuple(t.shape) != (B, Hkv, D) or t.dtype != kv_cache.dtype:
            raise PAError(PA_EINVAL, "new_key/new_value must be [B, H_kv, D] in the cache dtype")
    _check(lib().pa_decode_append_noalloc(_ptr(out), _ptr(lse), _ptr(query), _ptr(new_key),
                                          _ptr(new_value), _ptr(kv_cache), N, _ptr(block_tables),
                                          block_tables.shape[1], _ptr(seq_lens), B,
                                          int(max_seq_len), Hq, Hkv, D, bs, float(scale),
                                          int(partition_size), _ptr(plan),
                                          0 if plan is None else plan.numel(),
                                          _dtype_code(kv_cache), _stream(stream)))


def decode_multi_workspace_bytes(B: int, rows: int, num_q_heads: int, num_kv_heads: int,
                                 head_size: int, max_seq_len: int, partition_size: int) -> int:
    return int(lib().pa_decode_multi_workspace_bytes(B, rows, num_q_heads, num_kv_heads,
                                                     head_size, max_seq_len, partition_size))


def decode_multi_workspace(B: int, rows: int, num_q_heads: int, num_kv_heads: int,
                           head_size: int, max_seq_len: int, partition_size: int,
                           device="cuda", stream=None):
    """A zeroed uint8 GPU workspace for decode_multi (at least 256 bytes)."""
    torch = _torch()
    n = decode_multi_workspace_bytes(B, rows, num_q_heads, num_kv_heads, head_size, max_seq_len,
                                     partition_size)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    decode_workspace_init(ws, stream)
    return ws


def decode_multi(out, query, kv_cache, block_tables, seq_lens, max_seq_len: int, scale: float,
                 rows: int, partition_size: int = 0, workspace=None, lse=None, plan=None,
                 stream=None) -> None:
    """pa_decode_multi: every sequence's last `rows` tokens attend causally
    (speculative-decoding verification).  out/query [B * rows, H_q, D];
    lse fp32 [B * rows, H_q] or None; the other arguments as decode().  An
    FP8 cache goes through decode_multi_fp8 (it carries the scales)."""
    _need_gpu(out, query, kv_cache, block_tables, seq_lens, workspace, lse, plan)
    torch = _torch()
    if kv_cache.dtype == torch.uint8:
        raise PAError(PA_EINVAL, "an FP8 cache needs decode_multi_fp8 (its scales)")
    N, _, Hkv, bs, D = kv_cache.shape
    T, Hq, Dq = query.shape
    B = seq_lens.numel()
    if Dq != D or T != B * int(rows) or tuple(out.shape) != (T, Hq, D) \
            or out.dtype != kv_cache.dtype or query.dtype != kv_cache.dtype:
        raise PAError(PA_EINVAL, "out/query must be [B * rows, H_q, D] in the cache dtype")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32 \
            or block_tables.shape[0] != B:
        raise PAError(PA_EINVAL, "block_tables/seq_lens must be int32 with B rows")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (T, Hq)):
        raise PAError(PA_EINVAL, "lse must be fp32 [B * rows, H_q]")
    if plan is not None and plan.dtype != torch.int32:
        raise PAError(PA_EINVAL, "plan must be int32")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_decode_multi(_ptr(out), _ptr(lse), _ptr(query), _ptr(kv_cache), N,
                                 _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), B,
                                 int(max_seq_len), int(rows), Hq, Hkv, D, bs, float(scale),
                                 int(partition_size), _ptr(plan),
                                 0 if plan is None else plan.numel(), _ptr(workspace), ws_bytes,
                                 _dtype_code(kv_cache), _stream(stream)))


def decode_multi_fp8(out, query, kv_cache, block_tables, seq_lens, max_seq_len: int,
                     scale: float, k_scale: float, v_scale: float, rows: int,
                     partition_size: int = 0, workspace=None, lse=None, plan=None,
                     stream=None) -> None:
    """pa_decode_multi_fp8: decode_multi over an FP8 cache (uint8
    [N, 2, H_kv, 16, D] of E4M3 codes with per-tensor scales); out/query
    bf16 [B * rows, H_q, D]."""
    _need_gpu(out, query, kv_cache, block_tables, seq_lens, workspace, lse, plan)
    torch = _torch()
    N, _, Hkv, bs, D = kv_cache.shape
    T, Hq, Dq = query.shape
    B = seq_lens.numel()
    if Dq != D or T != B * int(rows) or tuple(out.shape) != (T, Hq, D) \
            or out.dtype != torch.bfloat16 or query.dtype != torch.bfloat16 \
            or kv_cache.dtype != torch.uint8:
        raise PAError(PA_EINVAL, "out/query must be bf16 [B * rows, H_q, D], kv_cache uint8")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32 \
            or block_tables.shape[0] != B:
        raise PAError(PA_EINVAL, "block_tables/seq_lens must be int32 with B rows")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (T, Hq)):
        raise PAError(PA_EINVAL, "lse must be fp32 [B * rows, H_q]")
    if plan is not None and plan.dtype != torch.int32:
        raise PAError(PA_EINVAL, "plan must be int32")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_decode_multi_fp8(_ptr(out), _ptr(lse), _ptr(query), _ptr(kv_cache), N,
                                     _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens),
                                     B, int(max_seq_len), int(rows), Hq, Hkv, D, bs,
                                     float(scale), float(k_scale), float(v_scale),
                                     int(partition_size), _ptr(plan),
                                     0 if plan is None else plan.numel(), _ptr(workspace),
                                     ws_bytes, _stream(stream)))


def decode_fp8(out, query, kv_cache, block_tables, seq_lens, max_seq_len: int, scale: float,
               k_scale: float, v_scale: float, partition_size: int = 0, workspace=None,
               lse=None, plan=None, stream=None, new_key=None, new_value=None) -> None:
    """pa_decode over an FP8 cache (uint8 [N, 2, H_kv, 16, D] of E4M3 codes):
    out/query bf16 [B, H_q, D]; the other arguments as decode().  With
    new_key/new_value (bf16 [B, H_kv, D]) the call is pa_decode_append_fp8:
    the new tokens are quantised into the cache in the same launch."""
    _need_gpu(out, query, kv_cache, block_tables, seq_lens, workspace, lse, plan, new_key,
              new_value)
    torch = _torch()
    N, _, Hkv, bs, D = kv_cache.shape
    B, Hq, Dq = query.shape
    if Dq != D or tuple(out.shape) != (B, Hq, D) or out.dtype != torch.bfloat16 \
            or query.dtype != torch.bfloat16 or kv_cache.dtype != torch.uint8:
        raise PAError(PA_EINVAL, "out/query must be bf16 [B, H_q, D] and kv_cache uint8")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32 \
            or block_tables.shape[0] != B or seq_lens.numel() != B:
        raise PAError(PA_EINVAL, "block_tables/seq_lens must be int32 with B rows")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq)):
        raise PAError(PA_EINVAL, "lse must be fp32 [B, H_q]")
    if plan is not None and plan.dtype != torch.int32:
        raise PAError(PA_EINVAL, "plan must be int32")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    tail = (N, _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), B, int(max_seq_len),
            Hq, Hkv, D, bs, float(scale), float(k_scale), float(v_scale), int(partition_size),
            _ptr(plan), 0 if plan is None else plan.numel(), _ptr(workspace), ws_bytes,
            _stream(stream))
    if new_key is None and new_value is None:
        _check(lib().pa_decode_fp8(_ptr(out), _ptr(lse), _ptr(query), _ptr(kv_cache), *tail))
        return
    for t in (new_key, new_value):
        if t is None or tuple(t.shape) != (B, Hkv, D) or t.dtype != torch.bfloat16 \
                or not t.is_contiguous():
            raise PAError(PA_EINVAL, "new_key/new_value must be contiguous bf16 [B, H_kv, D]")
    _check(lib().pa_decode_append_fp8(_ptr(out), _ptr(lse), _ptr(query), _ptr(new_key),
                                      _ptr(new_value), _ptr(kv_cache), *tail))


def prefill_chunk(out, query, query_start_loc, max_query_len: int, kv_cache, block_tables,
                  seq_lens, max_seq_len: int, scale: float, lse=None, stream=None) -> None:
    """out/query packed [T, H_q, D] bf16; query_start_loc int32 [B+1]."""
    _need_gpu(out, query, query_start_loc, kv_cache, block_tables, seq_lens, lse)
    torch = _torch()
    N, _, Hkv, bs, D = kv_cache.shape
    T, Hq, Dq = query.shape
    B = seq_lens.numel()
    if Dq != D or tuple(out.shape) != (T, Hq, D) or out.dtype != kv_cache.dtype \
            or query.dtype != kv_cache.dtype:
        raise PAError(PA_EINVAL, "shape/dtype mismatch between out/query and kv_cache")
    if query_start_loc.dtype != torch.int32 or query_start_loc.numel() != B + 1:
        raise PAError(PA_EINVAL, "query_start_loc must be int32 [B+1]")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32 or block_tables.shape[0] != B:
        raise PAError(PA_EINVAL, "block_tables/seq_lens must be int32 with B rows")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (T, Hq)):
        raise PAError(PA_EINVAL, "lse must be fp32 [T, H_q]")
    _check(lib().pa_prefill_chunk(_ptr(out), _ptr(lse), _ptr(query), _ptr(query_start_loc),
                                  int(max_query_len), T, _ptr(kv_cache), N, _ptr(block_tables),
                                  block_tables.shape[1], _ptr(seq_lens), B, int(max_seq_len), Hq,
                                  Hkv, D, bs, float(scale), _dtype_code(kv_cache),
                                  _stream(stream)))


def varlen_plan(query_start_loc_host, seq_lens_host, max_seq_len: int, num_q_heads: int,
                num_kv_heads: int, partition_size: int = 0):
    """Host-built work list of pa_attention_varlen: (int32 entries, number of
    them that are prefill query tiles)."""
    qsl = np.ascontiguousarray(query_start_loc_host, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    if qsl.size != sl.size + 1:
        raise PAError(PA_EINVAL, "query_start_loc must have B+1 entries")
    n, npre = ctypes.c_int32(), ctypes.c_int32()
    lib().pa_varlen_plan(_np_ptr(qsl), _np_ptr(sl), sl.size, int(max_seq_len), int(num_q_heads),
                         int(num_kv_heads), int(partition_size), None, 0, ctypes.byref(n),
                         ctypes.byref(npre))
    out = np.empty(max(n.value, 1), dtype=np.int32)
    _check(lib().pa_varlen_plan(_np_ptr(qsl), _np_ptr(sl), sl.size, int(max_seq_len),
                                int(num_q_heads), int(num_kv_heads), int(partition_size),
                                _np_ptr(out), out.size, ctypes.byref(n), ctypes.byref(npre)))
    return out[:n.value], int(npre.value)


def attention_varlen(out, query, query_start_loc, kv_cache, block_tables, seq_lens,
                     max_seq_len: int, scale: float, plan, partition_size: int = 0,
                     workspace=None, lse=None, stream=None) -> None:
    """One launch over a flattened batch of decode rows and prefill chunks:
    out/query packed bf16 [T, H_q, D]; query_start_loc int32 [B+1]; plan an
    int32 GPU tensor holding varlen_plan(...)[0], built from the same
    lengths and partition_size."""
    _need_gpu(out, query, query_start_loc, kv_cache, block_tables, seq_lens, plan, workspace, lse)
    torch = _torch()
    N, _, Hkv, bs, D = kv_cache.shape
    T, Hq, Dq = query.shape
    B = seq_lens.numel()
    if Dq != D or tuple(out.shape) != (T, Hq, D) or out.dtype != kv_cache.dtype \
            or query.dtype != kv_cache.dtype:
        raise PAError(PA_EINVAL, "shape/dtype mismatch between out/query and kv_cache")
    if query_start_loc.dtype != torch.int32 or query_start_loc.numel() != B + 1:
        raise PAError(PA_EINVAL, "query_start_loc must be int32 [B+1]")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32 or block_tables.shape[0] != B:
        raise PAError(PA_EINVAL, "block_tables/seq_lens must be int32 with B rows")
    if plan.dtype != torch.int32:
        raise PAError(PA_EINVAL, "plan must be int32")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (T, Hq)):
        raise PAError(PA_EINVAL, "lse must be fp32 [T, H_q]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_attention_varlen(_ptr(out), _ptr(lse), _ptr(query), _ptr(query_start_loc), T,
                                     _ptr(kv_cache), N, _ptr(block_tables), block_tables.shape[1],
                                     _ptr(seq_lens), B, int(max_seq_len), Hq, Hkv, D, bs,
                                     float(scale), int(partition_size), _ptr(plan), plan.numel(),
                                     _ptr(workspace), ws_bytes,
                                     _dtype_code(kv_cache), _stream(stream)))


class DecodeGraphs:
    """pa_decode_graphs_*: the attention of a decode step over a stack of
    layers (pa_decode_append per layer) captured once per warm-up batch size
    over static buffers sized for the largest one.

    kv_caches: a list of L caches [N, 2, H_kv, 16, D] (or one cache: L = 1);
    out/query [L, Bmax, H_q, D] (or [Bmax, H_q, D] for L = 1);
    new_key/new_value [L, Bmax, H_kv, D] (or [Bmax, H_kv, D]); block_tables
    int32 [Bmax, max_blocks]; seq_lens int32 [Bmax]; lse fp32 [L, Bmax, H_q]
    (or [Bmax, H_q]) or None; workspace as decode() for Bmax sequences.  The
    object keeps these tensors alive: the graphs read them at their recorded
    addresses.  replay(B) runs a step over their first B rows and returns the
    captured size it used."""

    def __init__(self, out, query, new_key, new_value, kv_caches, block_tables, seq_lens,
                 max_seq_len: int, scale: float, batch_sizes: Sequence[int],
                 partition_size: int = 0, workspace=None, lse=None, stream=None):
        caches = list(kv_caches) if isinstance(kv_caches, (list, tuple)) else [kv_caches]
        _need_gpu(out, query, new_key, new_value, block_tables, seq_lens, workspace, lse,
                  *caches)
        torch = _torch()
        Ls = len(caches)
        N, _, Hkv, bs, D = caches[0].shape
        for c in caches:
            if tuple(c.shape) != tuple(caches[0].shape) or c.dtype != caches[0].dtype:
                raise PAError(PA_EINVAL, "every layer's cache must have one shape and dtype")
        lead = (Ls,) if query.dim() == 4 else ()
        if query.dim() == 3 and Ls != 1:
            raise PAError(PA_EINVAL, "several layers need [L, Bmax, ...] buffers")
        Bmax, Hq, Dq = query.shape[-3:]
        if (query.dim() == 4 and query.shape[0] != Ls) or Dq != D \
                or tuple(out.shape) != lead + (Bmax, Hq, D) \
                or out.dtype != caches[0].dtype or query.dtype != caches[0].dtype:
            raise PAError(PA_EINVAL, "shape/dtype mismatch between out/query and the caches")
        if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32 \
                or block_tables.shape[0] != Bmax or seq_lens.numel() != Bmax:
            raise PAError(PA_EINVAL, "block_tables/seq_lens must be int32 with Bmax rows")
        if lse is not None and (lse.dtype != torch.float32
                                or tuple(lse.shape) != lead + (Bmax, Hq)):
            raise PAError(PA_EINVAL, "lse must be fp32 [(L,) Bmax, H_q]")
        for t in (new_key, new_value):
            if tuple(t.shape) != lead + (Bmax, Hkv, D) or t.dtype != caches[0].dtype:
                raise PAError(PA_EINVAL, "new_key/new_value must be [(L,) Bmax, H_kv, D] in the "
                                         "cache dtype")
        sizes = np.ascontiguousarray(batch_sizes, dtype=np.int32)
        if sizes.size == 0 or int(sizes.max()) != Bmax:
            raise PAError(PA_EINVAL, "the largest batch size must equal the buffers' rows")
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        self._keep = (out, query, new_key, new_value, caches, block_tables, seq_lens,
                      workspace, lse)
        ptrs = (_vp * Ls)(*[c.data_ptr() for c in caches])
        h = _vp()
        _check(lib().pa_decode_graphs_create(
            _ptr(out), _ptr(lse), _ptr(query), _ptr(new_key), _ptr(new_value), ptrs, Ls, N,
            _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), int(max_seq_len), Hq, Hkv,
            D, bs, float(scale), int(partition_size), _ptr(workspace), ws_bytes,
            _dtype_code(caches[0]), _np_ptr(sizes), sizes.size, _stream(stream),
            ctypes.byref(h)))
        self._h = h

    def batch_sizes(self) -> list:
        n = lib().pa_decode_graphs_count(self._h, None, 0)
        a = np.zeros(max(n, 0), dtype=np.int32)
        lib().pa_decode_graphs_count(self._h, _np_ptr(a), a.size)
        return [int(x) for x in a]

    def replay(self, B: int, stream=None) -> int:
        got = ctypes.c_int32(0)
        _check(lib().pa_decode_graphs_replay(self._h, int(B), _stream(stream), ctypes.byref(got)))
        return got.value

    def close(self) -> None:
        if self._h is not None and self._h.value:
            lib().pa_decode_graphs_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
