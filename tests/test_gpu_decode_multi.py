"""GPU parity of pa_decode_multi: several query rows per sequence on the
decode path (speculative-decoding verification).

The oracle is ``prefill_chunk``: sequence b's `rows` query rows are its last
`rows` tokens, each attending causally up to itself, which is exactly a
chunk of that length.  Bar: max |error| <= 2e-2 on bf16 outputs and on lse,
every checked output finite; rows before position 0 are zero with lse -inf.
"""
import numpy as np
import pytest
import torch

from paged_attention_kv_block_amd import inputs
from tests.conftest import gpu_available
from tests.oracle_setup import OracleSide

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL = 2e-2


def _f64(t):
    import oracle
    from tests.gpu_setup import from_device
    return oracle.to_f64(from_device(t))


def _draw(seq_lens, rows, Hq, Hkv, D, seed=7):
    return inputs.custom(kind="prefill", seq_lens=seq_lens, chunk_lens=[rows] * len(seq_lens),
                         num_q_heads=Hq, num_kv_heads=Hkv, head_size=D, seed=seed)


def _run(g, rows, P, use_plan, with_lse=True):
    from paged_attention_kv_block_amd import ops
    from tests.gpu_setup import to_device
    d, wl = g.d, g.wl
    q = to_device(d.query(), wl)
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda") \
        if with_lse else None
    msl = int(max(d.seq_lens))
    ws = ops.decode_multi_workspace(wl.num_seqs, rows, wl.num_q_heads, wl.num_kv_heads,
                                    wl.head_size, msl, P)
    plan = torch.from_numpy(ops.decode_plan(d.seq_lens, msl, P)).cuda() if use_plan else None
    ops.decode_multi(out, q, g.pool, g.bt_dev, g.seq_lens_dev, msl, float(wl.scale), rows, P,
                     ws, lse, plan)
    torch.cuda.synchronize()
    return out, lse


def check(d, rows, P, use_plan, seqs=None, o=None, g=None):
    from tests.gpu_setup import GpuSide
    if o is None:
        o = OracleSide(d, seqs=seqs)
    if g is None:
        g = GpuSide(d, fill=seqs is None)
        if seqs is not None:
            g.fill(seqs)
    np.testing.assert_array_equal(g.block_tables, o.block_tables)
    out, lse = _run(g, rows, P, use_plan)
    B = d.wl.num_seqs
    sel = range(B) if seqs is None else seqs
    ok_seqs = [b for b in sel if int(d.seq_lens[b]) >= rows]
    ref, ref_lse = o.prefill(seqs=ok_seqs)
    got, gl = _f64(out), lse.cpu().numpy().astype(np.float64)
    idx = np.array([b * rows + i for b in ok_seqs for i in range(rows)], dtype=int)
    if idx.size:
        assert np.all(np.isfinite(got[idx]))
        err = float(np.max(np.abs(got[idx] - ref[idx])))
        lerr = float(np.max(np.abs(gl[idx] - ref_lse[idx])))
        assert err <= TOL and lerr <= TOL, (rows, P, use_plan, err, lerr)
    # sequences shorter than `rows`: rows at positions >= 0 are a shorter
    # chunk; rows before position 0 see nothing
    import oracle
    wl = d.wl
    G = wl.num_q_heads // wl.num_kv_heads
    for b in sel:
        L = int(d.seq_lens[b])
        if L >= rows:
            continue
        K, V = oracle.gather_kv(o.pool, o.block_tables[b], L)
        for i in range(rows):
            r, pos = b * rows + i, L - rows + i
            if pos < 0:
                assert np.all(got[r] == 0.0) and np.all(np.isneginf(gl[r])), (b, i)
                continue
            qi = oracle.to_f64(d.query()[r])
            for gk in range(wl.num_kv_heads):
                hs = slice(gk * G, (gk + 1) * G)
                ro, rl = oracle.attention(qi[hs], K[:pos + 1, gk], V[:pos + 1, gk],
                                          float(wl.scale))
                assert np.max(np.abs(got[r, hs] - ro)) <= TOL, (b, i)
                assert np.max(np.abs(gl[r, hs] - rl)) <= TOL, (b, i)
    return out, lse


CASES = [
    # (name, seq_lens, rows, H_q, H_kv, D)
    ("g8-d64-rows2", (1, 2, 17, 33, 160, 300, 47), 2, 16, 2, 64),
    ("g8-d128-rows4", (4, 16, 17, 100, 257, 530), 4, 8, 1, 128),
    ("g4-d128-rows3", (3, 15, 16, 31, 64, 200, 513), 3, 8, 2, 128),
    ("g1-d64-rows5", (5, 6, 21, 80, 129), 5, 2, 2, 64),
    ("g16-d64-rows3", (3, 18, 40, 99), 3, 16, 1, 64),
    ("g2-d128-rows8", (8, 9, 24, 200, 345), 8, 4, 2, 128),
    ("g4-d64-rows16", (16, 17, 33, 100, 600), 16, 8, 2, 64),
    ("g8-d64-short", (1, 2, 3, 40), 4, 8, 1, 64),        # sequences shorter than rows
    ("g4-d128-empty", (0, 5, 0, 33, 1), 2, 8, 2, 128),  # empty sequences
]


@pytest.mark.parametrize("P,use_plan", [(0, False), (0, True), (16, False), (32, True),
                                        (512, True)])
@pytest.mark.parametrize("name,seq_lens,rows,Hq,Hkv,D", CASES, ids=[c[0] for c in CASES])
def test_decode_multi_shapes(name, seq_lens, rows, Hq, Hkv, D, P, use_plan):
    check(_draw(seq_lens, rows, Hq, Hkv, D), rows, P, use_plan)


def test_one_row_is_pa_decode():
    """rows == 1 is pa_decode itself: bit-identical outputs."""
    from paged_attention_kv_block_amd import ops
    from tests.gpu_setup import GpuSide
    d = _draw((5, 40, 200), 1, 8, 2, 128)
    g = GpuSide(d)
    for P in (0, 32):
        out, lse = _run(g, 1, P, False)
        ref = torch.empty_like(out)
        rl = torch.empty_like(lse)
        ws = ops.decode_workspace(3, 8, 2, 128, 200, P)
        from tests.gpu_setup import to_device
        ops.decode(ref, to_device(d.query(), d.wl), g.pool, g.bt_dev, g.seq_lens_dev, 200,
                   float(d.wl.scale), P, ws, rl)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        assert torch.equal(lse, rl)


def test_repeated_calls_share_the_workspace():
    """Split-K counters return to zero: two calls on one workspace, the second
    with other queries, each match the oracle."""
    from paged_attention_kv_block_amd import ops
    from tests.gpu_setup import GpuSide, to_device
    d = _draw((40, 300, 77, 129), 4, 16, 2, 64)
    o, g = OracleSide(d), GpuSide(d)
    ref, _ = o.prefill()
    ws = ops.decode_multi_workspace(4, 4, 16, 2, 64, 300, 32)
    q = to_device(d.query(), d.wl)
    for k in range(3):
        out = torch.full_like(q, float("nan"))
        ops.decode_multi(out, q, g.pool, g.bt_dev, g.seq_lens_dev, 300, float(d.wl.scale), 4,
                         32, ws)
        torch.cuda.synchronize()
        assert float(np.max(np.abs(_f64(out) - ref))) <= TOL, k


def test_unit_values_give_unit_output():
    from tests.gpu_setup import GpuSide
    d = _draw((4, 17, 90), 4, 16, 2, 128)
    g = GpuSide(d)
    g.pool[:, 1] = 1.0
    for P, plan in ((0, False), (32, True)):
        out, _ = _run(g, 4, P, plan)
        np.testing.assert_array_equal(_f64(out), 1.0)


def test_llama3_shape_sampled():
    """The Llama-3-8B-shaped decode batch at full size (256 sequences,
    log-normal lengths to 8192) verifying 4 rows per sequence with split-K
    512 and the plan; the oracle checks the longest, the shortest and a few
    others (only their blocks are filled; the rest read NaN poison)."""
    base = inputs.draw(2)
    L = base.seq_lens
    d = _draw(tuple(int(x) for x in L), 4, 32, 8, 128, seed=2002)
    seqs = sorted({int(np.argmax(L)), int(np.argmin(L)), 0, 77, 255})
    check(d, 4, 512, True, seqs=seqs)


def test_tinyllama_shape_sampled():
    """The TinyLlama-shaped batch (64 sequences, G = 8, head size 64) with 4
    rows per sequence (two column groups), one pass and split-K 256."""
    base = inputs.draw(1)
    L = base.seq_lens
    d = _draw(tuple(int(x) for x in L), 4, 32, 4, 64, seed=2001)
    seqs = sorted({int(np.argmax(L)), int(np.argmin(L)), 5, 63})
    from tests.gpu_setup import GpuSide
    o = OracleSide(d, seqs=seqs)
    g = GpuSide(d, fill=False)
    g.fill(seqs)
    check(d, 4, 0, True, seqs=seqs, o=o, g=g)
    check(d, 4, 256, True, seqs=seqs, o=o, g=g)


def _graph_replays_match(step, out):
    """Captures step() in a HIP graph after an eager warm-up and replays it
    four times with eager work between replays; each replay must equal the
    eager result bit for bit."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        out.zero_()
        _ = (eager.float() * 2).sum()            # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), rep
    return eager


@pytest.mark.parametrize("rows,P", [(2, 64), (4, 64), (4, 0)])
def test_multi_rows_in_a_hip_graph(rows, P):
    """pa_decode_multi (split-K counters and records, one or two column
    groups) captured in a HIP graph: every replay equals the eager call,
    which matches the oracle."""
    from paged_attention_kv_block_amd import ops
    from tests.gpu_setup import GpuSide, to_device
    d = _draw((300, 45, 17, 1000, 64, 130), rows, 32, 4, 64, seed=31)
    o, g = OracleSide(d), GpuSide(d)
    q = to_device(d.query(), d.wl)
    out = torch.empty_like(q)
    ws = ops.decode_multi_workspace(6, rows, 32, 4, 64, 1000, P)
    plan = torch.from_numpy(ops.decode_plan(d.seq_lens, 1000, P)).cuda()

    def step():
        ops.decode_multi(out, q, g.pool, g.bt_dev, g.seq_lens_dev, 1000, float(d.wl.scale), rows,
                         P, ws, plan=plan)

    eager = _graph_replays_match(step, out)
    ref, _ = o.prefill()
    assert float(np.max(np.abs(_f64(eager) - ref))) <= TOL


def test_varlen_short_chunks_in_a_hip_graph():
    """A flattened batch with decode rows, short chunks (multi-row items) and
    a tiled chunk, split-K 64, captured in a HIP graph."""
    from paged_attention_kv_block_amd import ops
    from tests.gpu_setup import GpuSide, to_device
    d = inputs.custom(kind="prefill", seq_lens=(300, 45, 17, 1000, 64, 3),
                      chunk_lens=(4, 1, 2, 8, 40, 3), num_q_heads=16, num_kv_heads=2,
                      head_size=128, seed=32)
    o, g = OracleSide(d), GpuSide(d)
    q = to_device(d.query(), d.wl)
    out = torch.empty_like(q)
    qsl = g.query_start_loc()
    plan, _ = ops.varlen_plan(qsl, d.seq_lens, 1000, 16, 2, 64)
    plan = torch.from_numpy(plan).cuda()
    qsl_dev = torch.from_numpy(qsl).cuda()
    ws = ops.decode_workspace(6, 16, 2, 128, 1000, 64)

    def step():
        ops.attention_varlen(out, q, qsl_dev, g.pool, g.bt_dev, g.seq_lens_dev, 1000,
                             float(d.wl.scale), plan, 64, ws)

    eager = _graph_replays_match(step, out)
    ref, _ = o.prefill()
    assert float(np.max(np.abs(_f64(eager) - ref))) <= TOL


def test_physical_permutation_is_bit_exact():
    """The same sequences over another physical block assignment (the free
    queue reversed) give bit-identical outputs and lse: the arithmetic order
    depends on logical positions only."""
    from tests.gpu_setup import GpuSide
    lens = (40, 300, 77, 129, 5)
    d1 = _draw(lens, 4, 16, 2, 64, seed=51)
    d2 = _draw(lens, 4, 16, 2, 64, seed=51)
    d2.pool_order = d2.pool_order[::-1].copy()
    g1, g2 = GpuSide(d1), GpuSide(d2)
    assert not np.array_equal(g1.block_tables, g2.block_tables)
    for P, plan in ((0, False), (32, True)):
        o1, l1 = _run(g1, 4, P, plan)
        o2, l2 = _run(g2, 4, P, plan)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), P
        assert torch.equal(l1, l2), P
