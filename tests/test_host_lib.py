"""libpa.so on the host (no GPU): exported symbols, the allocator, slot
mapping and closed forms against the oracle and the golden fixtures, and
argument validation of the device entry points (which fails before any HIP
call is made, so it is safe to exercise without a GPU)."""
import json
import os
import re

import numpy as np
import pytest

import oracle
from paged_attention_kv_block_amd import host, inputs, ops
from tests.test_oracle_pins import run_allocator_trace

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    with open(os.path.join(ROOT, "include", "pa.h")) as f:
        txt = f.read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 18
    L = ops.lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert missing == []
    assert set(names) == set(ops.SIGNATURES), "binding and header disagree"


def test_library_has_gfx950_code_object():
    """The shared object built here embeds a gfx950 device code object."""
    with open(ops.LIB_PATH, "rb") as f:
        assert b"amdgcn-amd-amdhsa--gfx950" in f.read()


def _golden(name):
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        return json.load(f)


class _CAlloc:
    """Adapts ops.Allocator to the oracle's exception types for trace replay."""

    def __init__(self, n, order):
        self.a = ops.Allocator(n, order)

    def _wrap(self, fn, *args):
        try:
            return fn(*args)
        except ops.NoFreeBlocks as e:
            raise oracle.NoFreeBlocks(str(e))
        except ops.PAError as e:
            if e.status == ops.PA_EINVAL:
                raise oracle.InvalidArgument(str(e))
            raise

    def allocate(self, n):
        return self._wrap(self.a.allocate, n)

    def share(self, ids):
        return self._wrap(self.a.share, ids)

    def free(self, ids):
        return self._wrap(self.a.free, ids)

    def export(self):
        return self.a.export()


def test_allocator_golden_trace():
    trace = _golden("allocator_fifo_trace_n8.json")
    assert run_allocator_trace(_CAlloc, trace) == []


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_allocator_matches_oracle_on_random_ops(seed):
    rng = np.random.default_rng(seed)
    N = 97
    order = rng.permutation(N)
    o = oracle.OracleAllocator(N, order)
    c = _CAlloc(N, order)
    held = []
    for _ in range(3000):
        r = rng.random()
        if r < 0.35:
            n = int(rng.integers(0, 9))
            res = []
            for a in (o, c):
                try:
                    res.append(a.allocate(n))
                except oracle.NoFreeBlocks:
                    res.append("nb")
            assert res[0] == res[1]
            if res[0] != "nb":
                held.append(res[0])
        elif r < 0.5 and held:
            ids = held[int(rng.integers(len(held)))]
            o.share(ids)
            c.share(ids)
            held.append(list(ids))
        elif r < 0.55:
            bad = [int(rng.integers(-2, N + 2)) for _ in range(3)]
            res = []
            for a in (o, c):
                try:
                    a.free(bad)
                    res.append("ok")
                except oracle.InvalidArgument:
                    res.append("inv")
            assert res[0] == res[1]
            if res[0] == "ok":       # a random free that happened to be valid
                for i in bad:
                    for h in held:
                        if i in h:
                            h.remove(i)
                            break
        elif held:
            ids = held.pop(int(rng.integers(len(held))))
            o.free(ids)
            c.free(ids)
        assert c.export() == o.export()


def test_allocator_errors_leave_state_unchanged():
    a = ops.Allocator(4, [2, 0, 3, 1])
    assert a.allocate(3) == [2, 0, 3]
    before = a.export()
    with pytest.raises(ops.NoFreeBlocks):
        a.allocate(2)
    with pytest.raises(ops.PAError):
        a.share([1])                      # free block
    with pytest.raises(ops.PAError):
        a.free([2, 2])                    # more than held
    with pytest.raises(ops.PAError):
        a.free([0, 7])                    # out of range
    with pytest.raises(ops.PAError):
        a.allocate(-1)
    assert a.export() == before
    with pytest.raises(ops.PAError):
        ops.Allocator(3, [0, 0, 1])       # not a permutation


def test_allocator_stats_match_oracle():
    d = inputs.draw(1)
    o = oracle.OracleAllocator(d.num_blocks, d.pool_order)
    c = ops.Allocator(d.num_blocks, d.pool_order)
    oracle.build_decode_block_tables(o, d.seq_lens, 16)
    host.decode_block_tables(c, d.seq_lens, 16)
    assert c.stats(d.seq_lens, 16) == o.stats(d.seq_lens, 16)


def test_build_tables_equals_allocate_calls():
    """pa_allocator_build_tables is the batch form of one allocate per
    sequence: same ids, same queue and refcounts, -1 padding, and with the
    prefix cache on, the same evictions of cached free blocks."""
    rng = np.random.default_rng(8)
    N = 300
    order = rng.permutation(N)
    for trial in range(20):
        lens = rng.integers(0, 120, size=int(rng.integers(0, 12))).tolist()
        c = ops.Allocator(N, order)
        o = oracle.OracleAllocator(N, order)
        if trial % 2:
            c.enable_prefix_cache(16)
            o.enable_prefix_cache(16)
            toks = rng.integers(0, 4, size=160).tolist()
            ids = c.allocate(10)
            assert ids == o.allocate(10)
            c.insert_prefix(toks, ids)
            o.insert(toks, ids)
            c.free(ids[::-1])
            o.free(ids[::-1])
        width = max([-(-L // 16) for L in lens] + [1]) + 2
        bt = c.build_tables(lens, 16, width)
        want = np.full((len(lens), width), -1, dtype=np.int32)
        for b, L in enumerate(lens):
            n = -(-L // 16)
            want[b, :n] = o.allocate(n)
        np.testing.assert_array_equal(bt, want)
        assert c.export() == o.export()
        if trial % 2:
            assert c.export_prefix_cache() == o.export_prefix_cache()


def test_build_tables_is_all_or_nothing():
    a = ops.Allocator(10, list(range(10))[::-1])
    before = a.export()
    with pytest.raises(ops.NoFreeBlocks):
        a.build_tables([64, 64, 48], 16)        # 11 blocks > 10 free
    assert a.export() == before
    with pytest.raises(ops.PAError):
        a.build_tables([64, 17], 16, width=1)    # a row too narrow
    assert a.export() == before
    bt = a.build_tables([0, 17, 16], 16)
    np.testing.assert_array_equal(bt, [[-1, -1], [9, 8], [7, -1]])
    assert a.num_free == 7


def test_large_pool_allocator():
    """A pool of the size the pages mention (hundreds of thousands of blocks)."""
    N = 400_000
    a = ops.Allocator(N)
    ids = a.allocate(N)
    assert ids[:3] == [0, 1, 2] and a.num_free == 0
    a.free(ids[::-1])
    q, rc = a.export()
    assert q[:3] == [N - 1, N - 2, N - 3] and max(rc) == 0


def _recipe_tables(side, alloc, case, bs):
    """Runs one case of the block-table fixture on the oracle or the library."""
    if case["recipe"] == "decode":
        L = case["seq_lens"]
        width = max(-(-x // bs) for x in L)
        if side == "oracle":
            return oracle.build_decode_block_tables(alloc, L, bs, width)
        return host.decode_block_tables(alloc, L, bs, width)
    args = (alloc, case["num_seqs"], case["prefix_tokens"], case["own_tokens"], bs,
            case["share_prefix"])
    if side == "oracle":
        return oracle.build_prefill_block_tables(*args)
    return host.prefill_block_tables(*args)


@pytest.mark.parametrize("side", ["oracle", "library"])
def test_block_table_recipes_golden(side):
    """Hand-derived tables, queues and refcounts of the decode and
    shared-prefix recipes (tests/golden/block_table_recipes_n12.json): the
    order of prefix shares, prefix copies and private allocations is fixed."""
    g = _golden("block_table_recipes_n12.json")
    for case in g["cases"]:
        if side == "oracle":
            a = oracle.OracleAllocator(g["num_blocks"], g["initial_order"])
        else:
            a = ops.Allocator(g["num_blocks"], g["initial_order"])
        bt = _recipe_tables(side, a, case, g["block_size"])
        np.testing.assert_array_equal(bt, np.array(case["table"], dtype=np.int32))
        q, rc = a.export()
        assert list(q) == case["queue"] and list(rc) == case["refcount"], case


def test_block_table_recipe_golden_catches_interleaved_copies():
    """A planted mistake in the oracle's prefix recipe (each unshared copy
    followed at once by that sequence's private blocks) fails the fixture."""
    g = _golden("block_table_recipes_n12.json")
    case = next(c for c in g["cases"] if c["recipe"] == "prefill" and not c["share_prefix"])
    a = oracle.OracleAllocator(g["num_blocks"], g["initial_order"])
    npre = case["prefix_tokens"] // 16
    nown = -(-case["own_tokens"] // 16)
    wrong = [a.allocate(npre) + a.allocate(nown) for _ in range(case["num_seqs"])]
    assert wrong != case["table"]


@pytest.mark.parametrize("wl_index", [0, 1, 2, 3, 4])
def test_block_tables_match_oracle(wl_index):
    d = inputs.draw(wl_index)
    wl = d.wl
    o = oracle.OracleAllocator(d.num_blocks, d.pool_order)
    c = ops.Allocator(d.num_blocks, d.pool_order)
    if wl.kind == "prefill":
        own = int(d.seq_lens[0]) - wl.prefix_tokens
        bo = oracle.build_prefill_block_tables(o, wl.num_seqs, wl.prefix_tokens, own, 16)
        bc = host.prefill_block_tables(c, wl.num_seqs, wl.prefix_tokens, own, 16)
    else:
        bo = oracle.build_decode_block_tables(o, d.seq_lens, 16)
        bc = host.decode_block_tables(c, d.seq_lens, 16)
    np.testing.assert_array_equal(bc, bo)
    assert c.export() == o.export()
    # slot mapping of each sequence's last token (decode) / chunk (prefill)
    for b in range(min(wl.num_seqs, 32)):
        L = int(d.seq_lens[b])
        n = 1 if wl.kind == "decode" else wl.chunk_lens()[b]
        if L == 0:
            continue
        np.testing.assert_array_equal(ops.slot_mapping(bc[b], L - n, n, 16),
                                      oracle.slot_mapping(bo[b], L - n, n, 16))


def test_slot_mapping_golden_and_batched():
    g = _golden("closed_forms.json")["slot_mapping"]
    for c in g["cases"]:
        got = ops.slot_mapping(np.array(g["row"], np.int32), c["start"], c["n"], g["block_size"])
        assert got.tolist() == c["slots"]
    bt = np.array([[5, 2, 7], [1, -1, -1]], np.int32)
    got = ops.slot_mapping(bt, [15, 3], [3, 2], 16)
    assert got.tolist() == [95, 32, 33, 19, 20]
    with pytest.raises(ops.PAError):
        ops.slot_mapping(bt, [0, 15], [1, 2], 16)        # seq 1 position 16 has no block
    with pytest.raises(ops.PAError):
        ops.slot_mapping(bt, [47, 0], [2, 1], 16)        # beyond the table width


def test_closed_forms_golden():
    g = _golden("closed_forms.json")
    for c in g["block_bytes"]["cases"]:
        assert ops.kv_block_bytes(c["block_size"], c["num_kv_heads"], c["head_size"],
                                  c["dtype_bytes"]) == c["bytes"]
    for c in g["blocks_for_budget"]["cases"]:
        assert ops.num_blocks_for_budget(c["budget"], c["block_bytes"], c["num_layers"]) == c["blocks"]
    assert ops.kv_block_bytes(0, 1, 1, 1) == 0
    with pytest.raises(ops.PAError):
        ops.num_blocks_for_budget(10, 0, 1)


# ---------------------------------------------------------------------------
# argument validation of the device entry points: returns before any HIP call
# ---------------------------------------------------------------------------
def _decode_status(**kw):
    args = dict(out=16, lse=None, q=16, cache=16, nb=4, bt=16, mbps=4, sl=16, B=1, msl=64,
                hq=8, hkv=2, d=128, bs=16, scale=0.1, P=0, ws=None, wsb=0, dtype=ops.PA_BF16)
    args.update(kw)
    L = ops.lib()
    st = L.pa_decode(args["out"], args["lse"], args["q"], args["cache"], args["nb"], args["bt"],
                     args["mbps"], args["sl"], args["B"], args["msl"], args["hq"], args["hkv"],
                     args["d"], args["bs"], args["scale"], args["P"], args.get("plan"),
                     args.get("plan_n", 0), args["ws"], args["wsb"], args["dtype"], None)
    return st, L.pa_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(hq=7), ops.PA_EINVAL),             # H_q not a multiple of H_kv
    (dict(d=96), ops.PA_ENOTSUP),            # head size
    (dict(bs=32), ops.PA_ENOTSUP),           # block size
    (dict(P=24), ops.PA_EINVAL),             # partition not a multiple of 16
    (dict(msl=65), ops.PA_EINVAL),           # beyond the table
    (dict(P=16), ops.PA_EINVAL),             # workspace missing
    (dict(out=8), ops.PA_EINVAL),            # misaligned output
    (dict(dtype=5), ops.PA_EINVAL),          # unknown dtype
    (dict(hq=48, hkv=2, d=128), ops.PA_ENOTSUP),  # group 24
    (dict(scale=float("nan")), ops.PA_EINVAL),
    (dict(plan=16, plan_n=0), ops.PA_EINVAL),     # a plan without entries
    (dict(plan=18, plan_n=2), ops.PA_EINVAL),     # misaligned plan
])
def test_decode_validation(kw, status):
    st, msg = _decode_status(**kw)
    assert st == status, msg
    assert msg


def _append_status(nk=16, nv=16, **kw):
    args = dict(out=16, lse=None, q=16, cache=16, nb=4, bt=16, mbps=4, sl=16, B=1, msl=64,
                hq=8, hkv=2, d=128, bs=16, scale=0.1, P=0, ws=None, wsb=0, dtype=ops.PA_BF16)
    args.update(kw)
    L = ops.lib()
    st = L.pa_decode_append(args["out"], args["lse"], args["q"], nk, nv, args["cache"],
                            args["nb"], args["bt"], args["mbps"], args["sl"], args["B"],
                            args["msl"], args["hq"], args["hkv"], args["d"], args["bs"],
                            args["scale"], args["P"], None, 0, args["ws"], args["wsb"],
                            args["dtype"], None)
    return st, L.pa_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(nk=None), ops.PA_EINVAL),          # new key missing
    (dict(nv=None), ops.PA_EINVAL),          # new value missing
    (dict(nk=24), ops.PA_EINVAL),            # misaligned new key
    (dict(hq=7), ops.PA_EINVAL),             # the decode checks apply too
    (dict(d=96), ops.PA_ENOTSUP),
    (dict(P=16), ops.PA_EINVAL),             # workspace missing
])
def test_decode_append_validation(kw, status):
    st, msg = _append_status(**kw)
    assert st == status, msg
    assert "pa_decode_append" in msg


def test_decode_append_empty_batch_is_a_no_op():
    st, _ = _append_status(nk=None, nv=None, B=0)
    assert st == ops.PA_OK


def test_decode_workspace_size():
    assert ops.decode_workspace_bytes(4, 8, 2, 128, 64, 0) == 0
    assert ops.decode_workspace_bytes(4, 8, 2, 128, 64, 64) == 0       # one partition
    n = ops.decode_workspace_bytes(4, 8, 2, 128, 100, 32)              # 4 partitions
    rows = 4 * 8 * 4
    assert n >= rows * (128 + 2) * 4 + 4 * 2 * 4
    L = ops.lib()
    assert L.pa_decode_workspace_init(None, 0, None) == ops.PA_OK
    assert L.pa_decode_workspace_init(None, 256, None) == ops.PA_EINVAL
    assert L.pa_decode_workspace_init(128, 256, None) == ops.PA_EINVAL   # misaligned


def _multi_status(**kw):
    args = dict(out=16, lse=None, q=16, cache=16, nb=4, bt=16, mbps=4, sl=16, B=1, msl=64,
                rows=4, hq=8, hkv=2, d=128, bs=16, scale=0.1, P=0, ws=None, wsb=0,
                dtype=ops.PA_BF16)
    args.update(kw)
    L = ops.lib()
    st = L.pa_decode_multi(args["out"], args["lse"], args["q"], args["cache"], args["nb"],
                           args["bt"], args["mbps"], args["sl"], args["B"], args["msl"],
                           args["rows"], args["hq"], args["hkv"], args["d"], args["bs"],
                           args["scale"], args["P"], args.get("plan"), args.get("plan_n", 0),
                           args["ws"], args["wsb"], args["dtype"], None)
    return st, L.pa_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(rows=0), ops.PA_EINVAL),
    (dict(rows=65), ops.PA_EINVAL),
    (dict(dtype=ops.PA_F32), ops.PA_ENOTSUP),           # several rows need bf16
    (dict(dtype=ops.PA_FP8), ops.PA_EINVAL),            # needs pa_decode_multi_fp8
    (dict(hq=34, hkv=1), ops.PA_ENOTSUP),               # group 34 > 16
    (dict(P=16), ops.PA_EINVAL),                        # workspace missing
    (dict(P=16, ws=256, wsb=1024), ops.PA_EINVAL),      # workspace too small
    (dict(hq=7), ops.PA_EINVAL),                        # the decode checks apply too
    (dict(d=96), ops.PA_ENOTSUP),
    (dict(msl=65), ops.PA_EINVAL),
])
def test_decode_multi_validation(kw, status):
    st, msg = _multi_status(**kw)
    assert st == status, msg
    assert "pa_decode_multi" in msg


def test_decode_multi_empty_batch_is_a_no_op():
    assert _multi_status(B=0)[0] == ops.PA_OK


def _multi_fp8_status(**kw):
    args = dict(out=16, lse=None, q=16, cache=16, nb=4, bt=16, mbps=4, sl=16, B=1, msl=64,
                rows=4, hq=8, hkv=2, d=128, bs=16, scale=0.1, ks=0.01, vs=0.01, P=0, ws=None,
                wsb=0)
    args.update(kw)
    L = ops.lib()
    st = L.pa_decode_multi_fp8(args["out"], args["lse"], args["q"], args["cache"], args["nb"],
                               args["bt"], args["mbps"], args["sl"], args["B"], args["msl"],
                               args["rows"], args["hq"], args["hkv"], args["d"], args["bs"],
                               args["scale"], args["ks"], args["vs"], args["P"], None, 0,
                               args["ws"], args["wsb"], None)
    return st, L.pa_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(rows=0), ops.PA_EINVAL),
    (dict(rows=65), ops.PA_EINVAL),
    (dict(ks=0.0), ops.PA_EINVAL),                       # scales positive and finite
    (dict(vs=float("inf")), ops.PA_EINVAL),
    (dict(ks=float("nan")), ops.PA_EINVAL),
    (dict(hq=34, hkv=1), ops.PA_ENOTSUP),                # group 34 > 16
    (dict(P=16), ops.PA_EINVAL),                         # workspace missing
    (dict(d=96), ops.PA_ENOTSUP),
    (dict(msl=65), ops.PA_EINVAL),
])
def test_decode_multi_fp8_validation(kw, status):
    st, msg = _multi_fp8_status(**kw)
    assert st == status, msg
    assert "pa_decode_multi_fp8" in msg


def test_decode_multi_fp8_empty_batch_is_a_no_op():
    assert _multi_fp8_status(B=0)[0] == ops.PA_OK


def test_decode_multi_workspace_size():
    """Records of 16 columns (floor(16 / G) rows with their G heads), or 32 at
    head size 64 when the rows need more than one 16-column tile, per
    (sequence, KV head, column group, partition), after the counter region;
    one row is pa_decode's workspace."""
    for B, Hq, Hkv, D, msl, P in [(4, 8, 2, 128, 100, 32), (64, 32, 4, 64, 2048, 256),
                                  (3, 16, 1, 64, 300, 32)]:
        assert (ops.decode_multi_workspace_bytes(B, 1, Hq, Hkv, D, msl, P) ==
                ops.decode_workspace_bytes(B, Hq, Hkv, D, msl, P))
        G = Hq // Hkv
        parts = -(-msl // P)
        base = ops.decode_multi_workspace_bytes(B, 2, Hq, Hkv, D, 64, 64)
        assert base == 0                                  # one partition: no workspace
        for rows in (2, 3, 4, 7):
            cols = 32 if D == 64 and rows > 16 // G else 16
            rpg = max(1, cols // G)
            groups = -(-rows // rpg)
            rec = cols * D * 4 + 128
            n = ops.decode_multi_workspace_bytes(B, rows, Hq, Hkv, D, msl, P)
            assert n >= B * Hkv * groups * parts * rec, (B, rows, n)
            assert n < B * Hkv * groups * parts * rec + 65536 * 4 + 256
    assert ops.decode_multi_workspace_bytes(4, 2, 34, 1, 128, 100, 32) == 0   # G > 16


def test_reshape_validation():
    L = ops.lib()
    assert L.pa_reshape_and_cache(16, 16, 16, 4, 16, 4, 16, 2, 80, ops.PA_BF16, None) == ops.PA_ENOTSUP
    assert L.pa_reshape_and_cache(16, 16, 16, -1, 16, 4, 16, 2, 64, ops.PA_BF16, None) == ops.PA_EINVAL
    assert L.pa_reshape_and_cache(16, 16, 12, 4, 16, 4, 16, 2, 64, ops.PA_BF16, None) == ops.PA_EINVAL
    assert L.pa_reshape_and_cache(None, None, None, 0, None, 4, 16, 2, 64, ops.PA_BF16, None) == ops.PA_OK


def test_prefill_validation():
    L = ops.lib()
    # fp32 prefill is not supported
    st = L.pa_prefill_chunk(16, None, 16, 16, 4, 4, 16, 4, 16, 4, 16, 1, 64, 8, 2, 128, 16, 0.1,
                            ops.PA_F32, None)
    assert st == ops.PA_ENOTSUP
    # H_q not a multiple of H_kv
    st = L.pa_prefill_chunk(16, None, 16, 16, 4, 4, 16, 4, 16, 4, 16, 1, 64, 7, 2, 128, 16, 0.1,
                            ops.PA_BF16, None)
    assert st == ops.PA_EINVAL
    # a NaN scale is refused (the check survives the kernel's no-NaN build flags)
    st = L.pa_prefill_chunk(16, None, 16, 16, 4, 4, 16, 4, 16, 4, 16, 1, 64, 8, 2, 128, 16,
                            float("nan"), ops.PA_BF16, None)
    assert st == ops.PA_EINVAL, L.pa_last_error().decode()


def test_fp8_dtype_refused_alike_by_every_entry_point_without_scales():
    """An FP8 cache handed to an entry point that takes no scales is one and
    the same argument error everywhere (the *_fp8 entry points carry them);
    validation returns before anything is enqueued."""
    L = ops.lib()
    FP8, EINVAL = ops.PA_FP8, ops.PA_EINVAL
    got = {
        "pa_decode": _decode_status(dtype=FP8),
        "pa_decode_append": _append_status(dtype=FP8),
        "pa_decode_multi": _multi_status(dtype=FP8),
        "pa_reshape_and_cache": (L.pa_reshape_and_cache(16, 16, 16, 4, 16, 4, 16, 2, 64, FP8,
                                                        None), L.pa_last_error().decode()),
        "pa_prefill_chunk": (L.pa_prefill_chunk(16, None, 16, 16, 4, 4, 16, 4, 16, 4, 16, 1, 64,
                                                8, 2, 128, 16, 0.1, FP8, None),
                             L.pa_last_error().decode()),
        "pa_attention_varlen": _varlen_status(dtype=FP8),
    }
    for fn, (st, msg) in got.items():
        assert st == EINVAL, (fn, st, msg)
        assert fn in msg


class _Strided:
    """A CPU tensor view that is not contiguous (every other row)."""

    @staticmethod
    def rows(*shape, dtype=None):
        import torch
        full = torch.zeros((shape[0] * 2,) + tuple(shape[1:]), dtype=dtype or torch.bfloat16)
        return full[::2]


def test_binding_refuses_strided_tensors():
    """A strided view (a slice of a fused QKV tensor, a sliced plan) would be
    read as packed rows from its data pointer: every device wrapper refuses
    it before anything reaches the library."""
    import torch
    bf, i32 = torch.bfloat16, torch.int32
    q = _Strided.rows(4, 8, 64)
    cache = torch.zeros((4, 2, 2, 16, 64), dtype=bf)
    bt = torch.zeros((4, 4), dtype=i32)
    sl = torch.ones(4, dtype=i32)
    qsl = torch.arange(5, dtype=i32)
    with pytest.raises(ops.PAError, match="contiguous"):
        ops.prefill_chunk(torch.zeros((4, 8, 64), dtype=bf), q, qsl, 1, cache, bt, sl, 16, 0.1)
    with pytest.raises(ops.PAError, match="contiguous"):
        ops.prefill_chunk(torch.zeros((4, 8, 64), dtype=bf), torch.zeros((4, 8, 64), dtype=bf),
                          qsl, 1, cache, bt[:, ::2], sl, 16, 0.1)
    plan = torch.zeros(8, dtype=i32)[::2]
    with pytest.raises(ops.PAError, match="contiguous"):
        ops.decode(torch.zeros((4, 8, 64), dtype=bf), torch.zeros((4, 8, 64), dtype=bf), cache,
                   bt, sl, 16, 0.1, 0, None, None, plan)
    with pytest.raises(ops.PAError, match="contiguous"):
        ops.decode_fp8(torch.zeros((4, 8, 64), dtype=bf), torch.zeros((4, 8, 64), dtype=bf),
                       torch.zeros((4, 2, 2, 16, 64), dtype=torch.uint8), bt, sl, 16, 0.1, 1.0,
                       1.0, 0, None, None, plan)
    with pytest.raises(ops.PAError, match="contiguous"):
        ops.decode_multi(torch.zeros((8, 8, 64), dtype=bf), torch.zeros((8, 8, 64), dtype=bf),
                         cache, bt, sl, 16, 0.1, 2, 0, None, None, plan)
    with pytest.raises(ops.PAError, match="contiguous"):
        ops.attention_varlen(torch.zeros((4, 8, 64), dtype=bf), q, qsl, cache, bt, sl, 16, 0.1,
                             torch.zeros(4, dtype=i32))
    with pytest.raises(ops.PAError, match="contiguous"):
        ops.reshape_and_cache(_Strided.rows(4, 2, 64), torch.zeros((4, 2, 64), dtype=bf),
                              torch.zeros(4, dtype=torch.int64), cache)


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        ops.lib(str(tmp_path / "libpa.so"))


def test_decode_plan_lists_nonempty_partitions_longest_first():
    sl = np.array([0, 100, 512, 513, 1100], np.int32)
    plan = ops.decode_plan(sl, 1100, 512)
    ent = [(int(e) & 0xFFFF, int(e) >> 16) for e in plan]
    # (b, part): b0 -> 1 (empty row), b1 -> 1, b2 -> 1, b3 -> 2, b4 -> 3
    assert sorted(ent) == [(0, 0), (1, 0), (2, 0), (3, 0), (3, 1), (4, 0), (4, 1), (4, 2)]
    sizes = {(0, 0): 0, (1, 0): 100, (2, 0): 512, (3, 0): 512, (3, 1): 1, (4, 0): 512,
             (4, 1): 512, (4, 2): 76}
    got = [sizes[e] for e in ent]
    assert got == sorted(got, reverse=True)
    assert ops.decode_plan(sl, 1100, 0).size == 5               # one item per sequence
    with pytest.raises(ops.PAError):
        ops.decode_plan(np.array([5000], np.int32), 1100, 512)   # beyond max_seq_len


def _varlen_items(qsl, sl, msl, G, P):
    """Expected (kind, b, x, work) of a flattened batch, written out from the
    plan's definition: one decode item per non-empty partition of a sequence
    with one row; a chunk of C_b >= 2 rows that fits 4 groups of 16 / G rows
    gives one multi-row decode item per group (x = 2^14 + group, work = the
    sequence's tokens); longer chunks go in tiles of 128 / G rows."""
    TQ = 128 // G
    RPG = 16 // G
    parts = 1 if P == 0 or msl <= P else -(-msl // P)
    pre, dec = [], []
    for b in range(len(sl)):
        C, L = qsl[b + 1] - qsl[b], int(sl[b])
        if C == 1:
            ptok = P if parts > 1 else L
            for p in range(-(-L // ptok)):
                dec.append((b, p, min(ptok, L - p * ptok)))
        elif C > 1 and -(-C // RPG) <= 4:
            for cg in range(-(-C // RPG)):
                dec.append((b, (1 << 14) + cg, L))
        elif C > 1:
            for t in range(-(-C // TQ)):
                rows = min(TQ, C - t * TQ)
                pre.append((b, t, rows * (L - C + t * TQ + rows)))
    return pre, dec


def test_varlen_plan_orders_tiles_then_decode_items():
    qsl = np.array([0, 1, 40, 40, 41, 341, 342, 345, 352], np.int32)  # C = 1, 39, 0, 1, 300, 1, 3, 7
    sl = np.array([700, 39, 5, 1, 900, 1300, 64, 500], np.int32)
    for G, P in [(4, 0), (8, 512), (1, 256), (2, 0)]:
        plan, npre = ops.varlen_plan(qsl, sl, 1300, 8 * G, 8, P)
        pre, dec = _varlen_items(qsl, sl, 1300, G, P)
        assert npre == len(pre) and plan.size == len(pre) + len(dec)
        u = plan.view(np.uint32).astype(np.int64)
        kinds = list(u >> 31)
        got = [(int(e) & 0xFFFF, (int(e) >> 16) & 0x7FFF) for e in u]
        assert kinds == [1] * npre + [0] * (plan.size - npre)   # the tiles come first
        assert sorted(got[:npre]) == sorted((b, x) for b, x, _ in pre)
        assert sorted(got[npre:]) == sorted((b, x) for b, x, _ in dec)
        wd = {(b, x): w for b, x, w in dec}
        assert [wd[e] for e in got[npre:]] == sorted(wd.values(), reverse=True)
        # tiles grouped by sequence, sequences by total work, tiles longest first
        sw = {}
        for b, x, w in pre:
            sw[b] = sw.get(b, 0) + w
        want = sorted(((b, x) for b, x, _ in pre), key=lambda e: (-sw[e[0]], e[0], -e[1]))
        assert got[:npre] == want


def test_varlen_plan_rejects_bad_metadata():
    sl = np.array([10, 10], np.int32)
    with pytest.raises(ops.PAError):            # more rows than tokens
        ops.varlen_plan(np.array([0, 11, 12], np.int32), sl, 16, 8, 2)
    with pytest.raises(ops.PAError):            # decreasing start locations
        ops.varlen_plan(np.array([0, 5, 3], np.int32), sl, 16, 8, 2)
    with pytest.raises(ops.PAError):            # first start location not 0
        ops.varlen_plan(np.array([1, 5, 6], np.int32), sl, 16, 8, 2)
    with pytest.raises(ops.PAError):            # group size 3
        ops.varlen_plan(np.array([0, 5, 6], np.int32), sl, 16, 6, 2)
    with pytest.raises(ops.PAError):            # beyond max_seq_len
        ops.varlen_plan(np.array([0, 5, 6], np.int32), sl, 8, 8, 2)
    plan, npre = ops.varlen_plan(np.array([0, 0, 0], np.int32), sl, 16, 8, 2)
    assert plan.size == 0 and npre == 0


def _varlen_status(**kw):
    args = dict(out=16, lse=None, q=16, qsl=16, T=4, cache=16, nb=4, bt=16, mbps=4, sl=16, B=1,
                msl=64, hq=8, hkv=2, d=128, bs=16, scale=0.1, P=0, plan=16, plan_n=1,
                ws=None, wsb=0, dtype=ops.PA_BF16)
    args.update(kw)
    L = ops.lib()
    st = L.pa_attention_varlen(args["out"], args["lse"], args["q"], args["qsl"], args["T"],
                               args["cache"], args["nb"], args["bt"], args["mbps"], args["sl"],
                               args["B"], args["msl"], args["hq"], args["hkv"], args["d"],
                               args["bs"], args["scale"], args["P"], args["plan"],
                               args["plan_n"], args["ws"], args["wsb"], args["dtype"], None)
    return st, L.pa_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(hq=7), ops.PA_EINVAL),             # H_q not a multiple of H_kv
    (dict(hq=32, hkv=2), ops.PA_ENOTSUP),    # group 16: no prefill tile for it
    (dict(d=96), ops.PA_ENOTSUP),
    (dict(bs=32), ops.PA_ENOTSUP),
    (dict(dtype=ops.PA_F32), ops.PA_ENOTSUP),
    (dict(dtype=ops.PA_FP8), ops.PA_EINVAL),
    (dict(P=24), ops.PA_EINVAL),
    (dict(P=16), ops.PA_EINVAL),             # workspace missing
    (dict(plan=None), ops.PA_EINVAL),
    (dict(plan=18), ops.PA_EINVAL),          # misaligned plan
    (dict(qsl=None), ops.PA_EINVAL),
    (dict(out=8), ops.PA_EINVAL),
    (dict(msl=65), ops.PA_EINVAL),           # beyond the table
    (dict(scale=float("nan")), ops.PA_EINVAL),
])
def test_varlen_validation(kw, status):
    st, msg = _varlen_status(**kw)
    assert st == status, msg
    assert "pa_attention_varlen" in msg


def test_varlen_empty_batch_is_a_no_op():
    assert _varlen_status(B=0)[0] == ops.PA_OK
    assert _varlen_status(plan=None, plan_n=0)[0] == ops.PA_OK


def test_decode_graphs_refuse_bad_arguments_before_any_device_call():
    """pa_decode_graphs_create checks its arguments before it touches the
    device (capture and instantiation come last); replay, count and destroy
    take a NULL handle safely."""
    import ctypes
    L = ops.lib()
    EINVAL = ops.PA_EINVAL
    sizes = np.array([4, 8], dtype=np.int32)
    h = ctypes.c_void_p()

    caches = (ctypes.c_void_p * 2)(16, 16)

    def create(handle=True, sizes_=sizes, n=None, stream=16, seq_lens=16, P=0, ws_bytes=0,
               layers=2, dtype=ops.PA_BF16, out=16):
        return L.pa_decode_graphs_create(
            out, None, 16, 16, 16, caches, layers, 4, 16, 4, seq_lens, 64, 8, 4, 64, 16, 0.125,
            P, None, ws_bytes, dtype, None if sizes_ is None else sizes_.ctypes.data,
            len(sizes_) if n is None else n, stream, ctypes.byref(h) if handle else None)

    assert create(handle=False) == EINVAL and "NULL handle" in L.pa_last_error().decode()
    assert create(layers=0) == EINVAL and "no layers" in L.pa_last_error().decode()
    assert create(dtype=ops.PA_FP8) == EINVAL
    assert create(out=None) == EINVAL and "NULL pointer" in L.pa_last_error().decode()
    assert create(n=0) == EINVAL and "no batch sizes" in L.pa_last_error().decode()
    assert create(sizes_=np.array([0, 8], np.int32)) == EINVAL
    assert create(sizes_=np.array([8, 65536], np.int32)) == EINVAL
    assert create(stream=None) == EINVAL and "null stream" in L.pa_last_error().decode()
    assert create(seq_lens=None) == EINVAL
    # split-K over 64 tokens at P = 16 needs a workspace for batch 8
    need = L.pa_decode_workspace_bytes(8, 8, 4, 64, 64, 16)
    assert need > 0
    assert create(P=16, ws_bytes=need - 1) == EINVAL
    assert "workspace" in L.pa_last_error().decode()
    assert h.value is None
    got = ctypes.c_int32(5)
    assert L.pa_decode_graphs_replay(None, 1, None, ctypes.byref(got)) == EINVAL
    assert L.pa_decode_graphs_count(None, None, 0) == -1
    L.pa_decode_graphs_destroy(None)


def _plan_by_rule(lens, max_seq_len, P):
    """The decode plan written out from its rule: one item per (sequence,
    partition) with tokens, one (empty) item for a sequence of length 0,
    ordered by tokens descending, then partition, then sequence."""
    parts = 1 if P <= 0 or max_seq_len <= 0 else -(-max_seq_len // P)
    items = []
    for b, L in enumerate(int(x) for x in lens):
        ptok = P if parts > 1 else max(L, 1)
        n = 1 if L == 0 else -(-L // ptok)
        for p in range(n):
            items.append((min(ptok, L - p * ptok), p, b))
    items.sort(key=lambda t: (-t[0], t[1], t[2]))
    return [(p << 16) | b for _, p, b in items]


@pytest.mark.parametrize("P", [0, 16, 32, 512])
def test_decode_plan_follows_its_ordering_rule(P):
    rng = np.random.default_rng(77 + P)
    for trial in range(20):
        B = int(rng.integers(1, 300))
        msl = int(rng.integers(1, 4000))
        lens = rng.integers(0, msl + 1, size=B).astype(np.int32)
        lens[rng.random(B) < 0.1] = 0
        if P:
            k = rng.random(B) < 0.2            # whole partitions
            lens[k] = np.minimum((lens[k] // P) * P, msl)
        got = ops.decode_plan(lens, msl, P)
        assert [int(x) for x in got] == _plan_by_rule(lens, msl, P), (trial, B, msl)


@pytest.mark.parametrize("P,bs", [(0, 16), (64, 16), (32, 8)])
def test_decode_step_prepare_equals_the_oracle_step(P, bs):
    """Forty steps of pa_decode_step_prepare against the same step done by
    the oracle: its allocator pops the new blocks (sequences in order), its
    slot mapping gives the new tokens' slots, and the plan follows the rule;
    tables, lengths, slots, plan and the allocator state agree every step."""
    rng = np.random.default_rng(5 + P + bs)
    B, steps = 37, 40
    lens0 = rng.integers(1, 200, size=B).astype(np.int32)
    lens0[:5] = [bs, 2 * bs, bs - 1, 1, 3 * bs]              # block boundaries
    N = int(sum(-(-(int(L) + steps) // bs) for L in lens0)) + 9
    order = rng.permutation(N).astype(np.int32)
    width = int(max(-(-(int(L) + steps) // bs) for L in lens0))
    msl = int(lens0.max()) + steps
    ca = ops.Allocator(N, order)
    oa = oracle.OracleAllocator(N, order)
    bt = host.decode_block_tables(ca, lens0, bs, width)
    obt = oracle.build_decode_block_tables(oa, lens0, bs, width)
    np.testing.assert_array_equal(bt, obt)
    lens, olens = lens0.copy(), lens0.copy()
    slots = np.zeros(B, np.int64)
    plan = np.zeros(B * (msl // 16 + 2), np.int32)
    for step in range(steps):
        n = ops.decode_step_prepare(ca, bt, lens, bs, msl, P, slots, plan)
        opens = [b for b in range(B) if olens[b] % bs == 0]
        ids = oa.allocate(len(opens))
        for b, i in zip(opens, ids):
            obt[b, olens[b] // bs] = i
        oslots = [oracle.slot_mapping(obt[b], int(olens[b]), 1, bs)[0] for b in range(B)]
        olens += 1
        np.testing.assert_array_equal(bt, obt)
        np.testing.assert_array_equal(lens, olens)
        assert [int(s) for s in slots] == [int(s) for s in oslots], step
        assert [int(x) for x in plan[:n]] == _plan_by_rule(olens, msl, P), step
        assert ca.export() == oa.export()


def test_decode_step_prepare_is_all_or_nothing():
    """Each refusal leaves the tables, lengths, allocator and outputs as
    they were."""
    bs = 16
    lens0 = np.array([16, 5, 32, 31], np.int32)     # sequences 0 and 2 open a block
    ca = ops.Allocator(12, None)
    bt0 = host.decode_block_tables(ca, lens0, bs, 4)
    state0 = ca.export()

    def attempt(bt, lens, msl=1000, plan=None, alloc=ca):
        slots = np.full(lens.size, -7, np.int64)
        with pytest.raises(ops.PAError) as e:
            ops.decode_step_prepare(alloc, bt, lens, bs, msl, 32, slots, plan)
        assert (slots == -7).all()
        return e.value.status

    bt, lens = bt0.copy(), lens0.copy()
    assert attempt(bt, lens, msl=32) == ops.PA_EINVAL             # sequence 2 reaches 32
    bad = bt0.copy()
    bad[0, 1] = 3                                                   # entry already holds a block
    assert attempt(bad, lens) == ops.PA_EINVAL
    bad = bt0.copy()
    bad[1, 0] = -1                                                  # token 5 finds no block
    assert attempt(bad, lens) == ops.PA_EINVAL
    assert attempt(bt, lens, plan=np.zeros(2, np.int32)) == ops.PA_EINVAL   # capacity
    np.testing.assert_array_equal(bt, bt0)
    np.testing.assert_array_equal(lens, lens0)
    assert ca.export() == state0
    taken = ca.allocate(ca.num_free - 1)                            # one block left, two needed
    state1 = ca.export()
    assert attempt(bt, lens) == ops.PA_ENOBLOCKS
    np.testing.assert_array_equal(bt, bt0)
    np.testing.assert_array_equal(lens, lens0)
    assert ca.export() == state1
    ca.free(taken)
    slots = np.zeros(4, np.int64)
    plan = np.zeros(16, np.int32)
    assert ops.decode_step_prepare(ca, bt, lens, bs, 1000, 32, slots, plan) == 5
    assert list(lens) == [17, 6, 33, 32]


def test_decode_step_object_equals_the_function():
    """ops.DecodeStep (arguments marshalled once) gives the same tables,
    lengths, slots and plans as ops.decode_step_prepare step after step."""
    bs, P, steps = 16, 32, 30
    rng = np.random.default_rng(9)
    lens0 = rng.integers(1, 100, size=11).astype(np.int32)
    order = rng.permutation(200).astype(np.int32)
    a1, a2 = ops.Allocator(200, order), ops.Allocator(200, order)
    bt1 = host.decode_block_tables(a1, lens0, bs, 12)
    bt2 = host.decode_block_tables(a2, lens0, bs, 12)
    l1, l2 = lens0.copy(), lens0.copy()
    st = ops.DecodeStep(a1, bt1, l1, bs, 400, P)
    slots = np.zeros(11, np.int64)
    plan = np.zeros(11 * 13, np.int32)
    for _ in range(steps):
        n1 = st.prepare()
        n2 = ops.decode_step_prepare(a2, bt2, l2, bs, 400, P, slots, plan)
        assert n1 == n2
        np.testing.assert_array_equal(st.plan[:n1], plan[:n2])
        np.testing.assert_array_equal(st.slots, slots)
        np.testing.assert_array_equal(bt1, bt2)
        np.testing.assert_array_equal(l1, l2)
    assert a1.export() == a2.export()
