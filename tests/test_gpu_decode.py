"""GPU parity of pa_reshape_and_cache and pa_decode against the fp64 oracle.

Both sides start from the same seeded draws (paged_attention_kv_block_amd.inputs).
The oracle side allocates, maps slots, fills its pool and attends with
``oracle``; the GPU side does the same through libpa (C allocator and slot
mapping, pa_reshape_and_cache, pa_decode).  Bars: bit-exact for block
tables, allocator state, slot mapping and the cache contents; max |error|
<= 2e-2 for bf16 and <= 1e-5 for fp32 attention outputs; lse within the same
bars (lse is fp32 in both cases).
"""
import numpy as np
import pytest
import torch

from paged_attention_kv_block_amd import inputs
from tests.conftest import gpu_available
from tests.oracle_setup import OracleSide

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL = {"f32": 1e-5, "bf16": 2e-2}


def _gpu():
    from tests.gpu_setup import GpuSide, from_device
    return GpuSide, from_device


def out_f64(t):
    from tests.gpu_setup import from_device
    import oracle
    return oracle.to_f64(from_device(t))


def check_tables(o, g):
    np.testing.assert_array_equal(g.block_tables, o.block_tables)
    assert g.alloc.export() == o.alloc.export()


def check_pool(o, g):
    _, from_device = _gpu()
    got = from_device(g.pool)
    if got.dtype == np.float32:
        np.testing.assert_array_equal(got.view(np.uint32), o.pool.view(np.uint32))
    else:
        np.testing.assert_array_equal(got, o.pool)


def run_decode_case(d, partition_size=None, seqs=None, check_pool_bits=True, use_plan=False,
                    full_pool=False):
    """seqs limits the oracle's attention to a sample of sequences; with
    full_pool the oracle still fills every sequence, so the whole GPU pool is
    compared bit for bit (its scatter is a cheap host loop)."""
    GpuSide, _ = _gpu()
    o = OracleSide(d, seqs=None if full_pool else seqs)
    g = GpuSide(d)
    check_tables(o, g)
    if check_pool_bits and (seqs is None or full_pool):
        check_pool(o, g)
    out, lse = g.decode(partition_size=partition_size, use_plan=use_plan)
    ref, ref_lse = o.decode(seqs=seqs)
    rows = list(range(d.wl.num_seqs)) if seqs is None else list(seqs)
    got = out_f64(out)[rows]
    err = np.max(np.abs(got - ref[rows]))
    lerr = np.max(np.abs(lse.cpu().numpy().astype(np.float64)[rows] - ref_lse[rows]))
    tol = TOL[d.wl.dtype]
    assert np.all(np.isfinite(got)), "non-finite output"
    assert err <= tol, f"max abs error {err} > {tol}"
    assert lerr <= tol, f"lse max abs error {lerr} > {tol}"
    return err, out, lse, g


def test_tiny_fp32_workload():
    err, *_ = run_decode_case(inputs.draw(0))
    print("tiny fp32 max err", err)


@pytest.mark.parametrize("P", [0, 16, 48])
def test_tiny_fp32_workload_split(P):
    run_decode_case(inputs.draw(0), partition_size=P)


EDGE = [
    # (name, kwargs)
    ("ragged-bf16-g8-d64", dict(seq_lens=(1, 15, 16, 17, 33, 64, 100, 257), num_q_heads=32,
                                num_kv_heads=4, head_size=64)),
    ("ragged-bf16-g4-d128", dict(seq_lens=(1, 2, 31, 32, 47, 200), num_q_heads=32, num_kv_heads=8,
                                 head_size=128)),
    ("bf16-g8-d128", dict(seq_lens=(5, 77, 300), num_q_heads=64, num_kv_heads=8, head_size=128)),
    ("bf16-g16-d64", dict(seq_lens=(3, 90), num_q_heads=32, num_kv_heads=2, head_size=64)),
    ("bf16-g2-d128", dict(seq_lens=(9, 130), num_q_heads=4, num_kv_heads=2, head_size=128)),
    ("bf16-mha-d64", dict(seq_lens=(40, 1), num_q_heads=3, num_kv_heads=3, head_size=64)),
    ("bf16-mha-d128", dict(seq_lens=(70,), num_q_heads=2, num_kv_heads=2, head_size=128)),
    ("f32-g8-d128", dict(seq_lens=(33, 100), num_q_heads=16, num_kv_heads=2, head_size=128,
                         dtype="f32")),
    ("f32-g1-d64", dict(seq_lens=(17, 2), num_q_heads=2, num_kv_heads=2, head_size=64, dtype="f32")),
    ("f32-g16-d64", dict(seq_lens=(50,), num_q_heads=16, num_kv_heads=1, head_size=64, dtype="f32")),
    ("f32-g4-d128", dict(seq_lens=(23, 64), num_q_heads=8, num_kv_heads=2, head_size=128,
                         dtype="f32")),
]


@pytest.mark.parametrize("name,kw", EDGE, ids=[e[0] for e in EDGE])
@pytest.mark.parametrize("P", [0, 32, 64])
def test_decode_edge_shapes(name, kw, P):
    run_decode_case(inputs.custom(kind="decode", **kw), partition_size=P)


@pytest.mark.parametrize("name,kw", EDGE[:5], ids=[e[0] for e in EDGE[:5]])
@pytest.mark.parametrize("P", [0, 32])
def test_decode_edge_shapes_planned(name, kw, P):
    run_decode_case(inputs.custom(kind="decode", **kw), partition_size=P, use_plan=True)


# Many short ragged sequences: enough (sequence, KV head[, partition]) items
# that the launch uses small workgroups (4 waves from 2 items per compute
# unit, 2 waves from 8), with tails and one-token sequences among them.
MANY = [
    ("many-g8-d64-b300", 300, 32, 4, 64),     # 1 200 items: 4-wave workgroups
    ("many-g8-d64-b600", 600, 32, 4, 64),     # 2 400 items: 2-wave workgroups
    ("many-g4-d128-b600", 600, 32, 8, 128),   # 4 800 items
]


@pytest.mark.parametrize("name,B,hq,hkv,D", MANY, ids=[m[0] for m in MANY])
@pytest.mark.parametrize("P,use_plan", [(0, True), (0, False), (32, True)])
def test_decode_many_items(name, B, hq, hkv, D, P, use_plan):
    rng = np.random.default_rng(B + D)
    lens = rng.integers(1, 97, B)
    lens[:3] = (1, 16, 17)
    d = inputs.custom(kind="decode", seq_lens=tuple(int(x) for x in lens), num_q_heads=hq,
                      num_kv_heads=hkv, head_size=D, seed=B)
    run_decode_case(d, partition_size=P, use_plan=use_plan)


# Split-K over partitions of 1024 tokens or more: the decode launch only
# writes its records and a second launch merges them (one workgroup per
# (sequence, KV head), or four per slot when there are fewer slots than two
# per compute unit).  Sequences at, just above and well past a partition
# boundary, one-token rows, every group size and both cache dtypes.
LONGPART = [
    ("bf16-g8-d128", dict(seq_lens=(1, 1023, 1024, 1025, 2049, 3000), num_q_heads=64,
                          num_kv_heads=8, head_size=128)),
    ("bf16-g16-d64", dict(seq_lens=(1024, 2500, 17), num_q_heads=32, num_kv_heads=2,
                          head_size=64)),
    ("bf16-g1-d64", dict(seq_lens=(4097, 1030), num_q_heads=2, num_kv_heads=2, head_size=64)),
    ("bf16-g4-d64", dict(seq_lens=(2048, 2047, 1), num_q_heads=16, num_kv_heads=4,
                         head_size=64)),
    ("f32-g4-d128", dict(seq_lens=(1500, 2100), num_q_heads=8, num_kv_heads=2, head_size=128,
                         dtype="f32")),
    ("f32-g2-d64", dict(seq_lens=(3100, 5), num_q_heads=4, num_kv_heads=2, head_size=64,
                        dtype="f32")),
]


@pytest.mark.parametrize("name,kw", LONGPART, ids=[e[0] for e in LONGPART])
@pytest.mark.parametrize("P,use_plan", [(1024, False), (1024, True), (2048, True)])
def test_decode_merge_launch(name, kw, P, use_plan):
    run_decode_case(inputs.custom(kind="decode", **kw), partition_size=P, use_plan=use_plan)


@pytest.mark.parametrize("use_plan", [False, True])
def test_decode_merge_launch_many_slots(use_plan):
    """640 (sequence, KV head) slots, more than two per compute unit: one
    merge workgroup per slot."""
    rng = np.random.default_rng(31)
    lens = rng.integers(1, 2600, 160)
    lens[:4] = (1, 1024, 1025, 2599)
    d = inputs.custom(kind="decode", seq_lens=tuple(int(x) for x in lens), num_q_heads=32,
                      num_kv_heads=4, head_size=64, seed=160)
    run_decode_case(d, partition_size=1024, use_plan=use_plan)


def test_zero_length_row():
    GpuSide, _ = _gpu()
    d = inputs.custom(kind="decode", seq_lens=(0, 20, 0), num_q_heads=8, num_kv_heads=2,
                      head_size=64, num_blocks=4)
    g = GpuSide(d)
    for P, up in ((0, False), (16, False), (0, True), (16, True)):
        out, lse = g.decode(partition_size=P, use_plan=up)
        o = out_f64(out)
        assert np.all(o[0] == 0) and np.all(o[2] == 0)
        assert np.all(np.isneginf(lse[0].cpu().numpy())) and np.all(np.isneginf(lse[2].cpu().numpy()))
        assert np.all(np.isfinite(o[1]))


def test_tinyllama_workload_parity():
    err, *_ = run_decode_case(inputs.draw(1))
    print("tinyllama-shaped max err", err)


@pytest.mark.parametrize("P", [256, 512])
@pytest.mark.parametrize("use_plan", [False, True])
def test_tinyllama_workload_split(P, use_plan):
    run_decode_case(inputs.draw(1), partition_size=P, use_plan=use_plan)


def test_llama3_workload_sampled():
    """Full-size 256-sequence workload, split-K 512 as benchmarked; the oracle
    computes a sample of sequences (including the longest and shortest)."""
    d = inputs.draw(2)
    L = d.seq_lens
    seqs = sorted({int(np.argmax(L)), int(np.argmin(L)), 0, 1, 100, 255})
    run_decode_case(d, partition_size=512, seqs=seqs, use_plan=True, full_pool=True)
    run_decode_case(d, partition_size=512, seqs=seqs[:3], use_plan=False)


def test_llama3_workload_more_sequences():
    """The same launch on 24 more sequences spread over the length range
    (every 11th by length), so the sample covers one to sixteen partitions."""
    d = inputs.draw(2)
    order = np.argsort(d.seq_lens, kind="stable")
    seqs = sorted(int(x) for x in order[::11][:24])
    run_decode_case(d, partition_size=512, seqs=seqs, use_plan=True)


def test_long_context_workload_sampled():
    """Full-size long-context workload (16 sequences of 32K-131K tokens, a
    5.4 GB pool), split-K 1024 with the plan, in the launch bench.py times.
    Both pools hold the sampled sequences (the longest and the shortest); the
    GPU's other rows read NaN poison and are not compared."""
    GpuSide, _ = _gpu()
    d = inputs.draw(4)
    L = d.seq_lens
    seqs = sorted({int(np.argmax(L)), int(np.argmin(L))})
    o = OracleSide(d, seqs=seqs)
    g = GpuSide(d, fill=False)
    g.fill(seqs)
    check_tables(o, g)
    out, lse = g.decode(partition_size=1024, use_plan=True)
    ref, ref_lse = o.decode(seqs=seqs)
    got = out_f64(out)[seqs]
    assert np.all(np.isfinite(got))
    err = np.max(np.abs(got - ref[seqs]))
    lerr = np.max(np.abs(lse.cpu().numpy().astype(np.float64)[seqs] - ref_lse[seqs]))
    print("long-context max err", err, "lse", lerr)
    assert err <= TOL["bf16"] and lerr <= TOL["bf16"]


def test_unit_values_give_unit_output():
    """V == 1 everywhere: softmax rows sum to one, so every output is 1."""
    GpuSide, _ = _gpu()
    d = inputs.custom(kind="decode", seq_lens=(3, 40, 129), num_q_heads=16, num_kv_heads=2,
                      head_size=128)
    g = GpuSide(d)
    g.pool[:, 1] = 1.0
    for P in (0, 32):
        out, _ = g.decode(partition_size=P)
        np.testing.assert_array_equal(out_f64(out), 1.0)


def test_physical_permutation_is_bit_exact():
    GpuSide, _ = _gpu()
    d1 = inputs.draw(1)
    d2 = inputs.draw(1)
    d2.pool_order = d2.pool_order[::-1].copy()
    g1, g2 = GpuSide(d1), GpuSide(d2)
    assert not np.array_equal(g1.block_tables, g2.block_tables)
    for P in (0, 256):
        o1, l1 = g1.decode(partition_size=P)
        o2, l2 = g2.decode(partition_size=P)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)


def test_workspace_reused_across_calls_and_shapes():
    """The split-K arrival counters reset themselves: one zeroed workspace
    serves many calls, including calls with different batch shapes."""
    from paged_attention_kv_block_amd import ops
    from tests.gpu_setup import GpuSide
    d1 = inputs.draw(1)
    d2 = inputs.custom(kind="decode", seq_lens=(300, 17, 1000), num_q_heads=32, num_kv_heads=4,
                       head_size=64)
    g1, g2 = GpuSide(d1), GpuSide(d2)
    o1 = OracleSide(d1).decode()[0]
    o2 = OracleSide(d2).decode()[0]
    nbytes = max(ops.decode_workspace_bytes(64, 32, 4, 64, int(d1.seq_lens.max()), 128),
                 ops.decode_workspace_bytes(3, 32, 4, 64, int(d2.seq_lens.max()), 128))
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ops.decode_workspace_init(ws)
    from tests.gpu_setup import to_device
    for rep in range(3):
        for g, d, ref in ((g1, d1, o1), (g2, d2, o2)):
            q = to_device(d.query(), d.wl)
            out = torch.empty_like(q)
            ops.decode(out, q, g.pool, g.bt_dev, g.seq_lens_dev, int(d.seq_lens.max()),
                       float(d.wl.scale), 128, ws)
            torch.cuda.synchronize()
            err = np.max(np.abs(out_f64(out) - ref))
            assert err <= 2e-2, (rep, err)


def test_decode_step_in_a_hip_graph():
    """The decode step (cache write + split-K decode) captured in a HIP graph
    and replayed several times, with eager work between replays: every
    replay matches the eager result bit for bit, and the eager result
    matches the oracle's reshape_and_cache of the same new K/V followed by
    its decode (pool bit for bit, outputs within the bf16 bar)."""
    import oracle
    from paged_attention_kv_block_amd import ops
    from tests.gpu_setup import GpuSide, to_device
    d = inputs.draw(1)
    g = GpuSide(d)
    wl = d.wl
    L = d.seq_lens
    msl = int(L.max())
    q = to_device(d.query(), wl)
    newk = torch.zeros((wl.num_seqs, wl.num_kv_heads, wl.head_size), dtype=torch.bfloat16, device="cuda")
    newv = torch.ones_like(newk)
    slots = torch.from_numpy(ops.slot_mapping(g.block_tables, L - 1, 1, 16)).cuda()
    o = OracleSide(d)
    zero = np.zeros((wl.num_seqs, wl.num_kv_heads, wl.head_size), dtype=np.uint16)
    one = np.full_like(zero, 0x3F80)                     # bf16 1.0
    oracle.reshape_and_cache(o.pool, zero, one,
                             np.array([o.slots_for(b, int(L[b]) - 1, 1)[0]
                                       for b in range(wl.num_seqs)]))
    ref, _ = o.decode()
    ws = ops.decode_workspace(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_size, msl, 256)
    out = torch.empty_like(q)

    def step():
        ops.reshape_and_cache(newk, newv, slots, g.pool)
        ops.decode(out, q, g.pool, g.bt_dev, g.seq_lens_dev, msl, float(wl.scale), 256, ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                   # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = out.clone()
    check_pool(o, g)
    err = np.max(np.abs(out_f64(eager) - ref))
    assert err <= TOL["bf16"], err
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        out.zero_()
        _ = (q.float() * 2).sum()                # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), rep
    check_pool(o, g)


@pytest.mark.parametrize("P", [128, 1024])
def test_split_k_partials_never_stale(P):
    """Two different inputs of the same shape alternate through one
    workspace: the partials of call n+1 occupy the addresses call n used, so
    a merge that read a stale partial would differ from the first result
    (P 128: the merge in the decode launch; P 1024: the merge launch)."""
    from paged_attention_kv_block_amd import ops
    from tests.gpu_setup import GpuSide, to_device
    d = inputs.draw(1)
    g = GpuSide(d)
    wl = d.wl
    msl = int(d.seq_lens.max())
    qa = to_device(d.query(), wl)
    qb = -qa
    ws = ops.decode_workspace(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_size, msl, P)
    outs = {}
    for it in range(12):
        for name, q in (("a", qa), ("b", qb)):
            out = torch.empty_like(q)
            ops.decode(out, q, g.pool, g.bt_dev, g.seq_lens_dev, msl, float(wl.scale), P, ws)
            torch.cuda.synchronize()
            if name not in outs:
                outs[name] = out
            else:
                assert torch.equal(out.view(torch.int16), outs[name].view(torch.int16)), (it, name)
    assert not torch.equal(outs["a"].view(torch.int16), outs["b"].view(torch.int16))
