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


def run_decode_case(d, partition_size=None, seqs=None, check_pool_bits=True):
    GpuSide, _ = _gpu()
    o = OracleSide(d, seqs=seqs)
    g = GpuSide(d)
    check_tables(o, g)
    if check_pool_bits and seqs is None:
        check_pool(o, g)
    out, lse = g.decode(partition_size=partition_size)
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


def test_zero_length_row():
    GpuSide, _ = _gpu()
    d = inputs.custom(kind="decode", seq_lens=(0, 20, 0), num_q_heads=8, num_kv_heads=2,
                      head_size=64, num_blocks=4)
    g = GpuSide(d)
    for P in (0, 16):
        out, lse = g.decode(partition_size=P)
        o = out_f64(out)
        assert np.all(o[0] == 0) and np.all(o[2] == 0)
        assert np.all(np.isneginf(lse[0].cpu().numpy())) and np.all(np.isneginf(lse[2].cpu().numpy()))
        assert np.all(np.isfinite(o[1]))


def test_tinyllama_workload_parity():
    err, *_ = run_decode_case(inputs.draw(1))
    print("tinyllama-shaped max err", err)


@pytest.mark.parametrize("P", [256, 512])
def test_tinyllama_workload_split(P):
    run_decode_case(inputs.draw(1), partition_size=P)


def test_llama3_workload_sampled():
    """Full-size 256-sequence workload, split-K 512 as benchmarked; the oracle
    computes a sample of sequences (including the longest and shortest)."""
    d = inputs.draw(2)
    L = d.seq_lens
    seqs = sorted({int(np.argmax(L)), int(np.argmin(L)), 0, 1, 100, 255})
    run_decode_case(d, partition_size=512, seqs=seqs)


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
