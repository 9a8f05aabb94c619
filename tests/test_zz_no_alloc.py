"""pa_decode_append_noalloc: the fused decode step without a workspace (its
split-K scratch is a static device array inside the library), for callers
that cannot allocate device memory.

Its output, lse and cache writes must equal pa_decode_append's with a
workspace, bit for bit (the same kernels run on the same inputs), on two
calls in a row, the second with a smaller batch of another shape; sizes
beyond the static scratch are refused before anything is enqueued.
"""
import numpy as np
import pytest

from paged_attention_kv_block_amd import inputs, ops
from tests.conftest import gpu_available


def _case(d, P):
    """Both entry points on identical copies of one pool; returns
    (out, lse, pool) of each."""
    import torch
    from tests.gpu_setup import GpuSide, to_device
    wl = d.wl
    g = GpuSide(d)
    L = d.seq_lens
    msl = int(L.max())
    rng = np.random.default_rng(7)
    bits = lambda: (rng.standard_normal((wl.num_seqs, wl.num_kv_heads, wl.head_size))
                    .astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    nk, nv = to_device(bits(), wl), to_device(bits(), wl)
    q = to_device(d.query(), wl)
    plan = torch.from_numpy(ops.decode_plan(L, msl, P)).cuda()
    res = []
    for noalloc in (False, True):
        pool = g.pool.clone()
        out = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            ops.decode_append_noalloc(out, q, pool, g.bt_dev, g.seq_lens_dev, msl,
                                      float(wl.scale), nk, nv, P, lse, plan)
        else:
            ws = ops.decode_workspace(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads,
                                      wl.head_size, msl, P)
            ops.decode(out, q, pool, g.bt_dev, g.seq_lens_dev, msl, float(wl.scale), P, ws,
                       lse, plan, new_key=nk, new_value=nv)
        torch.cuda.synchronize()
        res.append((out, lse, pool))
    return res


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs a GPU")
def test_noalloc_with_the_merge_launch():
    """1024-token partitions (records merged by a second launch, which reads
    them from the static scratch as well): bit for bit again, twice, the
    second call smaller."""
    import torch
    big = inputs.draw(1)
    small = inputs.custom(kind="decode", seq_lens=(1100, 5, 2100), num_q_heads=8,
                          num_kv_heads=2, head_size=128, seed=4)
    for d in (big, small):
        (o1, l1, p1), (o2, l2, p2) = _case(d, 1024)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), d.wl.name
        assert torch.equal(l1, l2), d.wl.name
        assert torch.equal(p1.view(torch.int16), p2.view(torch.int16)), d.wl.name
        assert not torch.isnan(o2.float()).any()


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs a GPU")
def test_noalloc_equals_workspace_entry_point_twice():
    import torch
    big = inputs.draw(1)                                   # 64 sequences, G 8, D 64
    small = inputs.custom(kind="decode", seq_lens=(5, 300, 17, 64, 1), num_q_heads=16,
                          num_kv_heads=4, head_size=128, seed=3)
    for d, P in ((big, 256), (small, 32)):                 # the second call is smaller
        (o1, l1, p1), (o2, l2, p2) = _case(d, P)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), d.wl.name
        assert torch.equal(l1, l2), d.wl.name
        assert torch.equal(p1.view(torch.int16), p2.view(torch.int16)), d.wl.name
        assert not torch.isnan(o2.float()).any()


def test_noalloc_refuses_layouts_beyond_the_scratch():
    """The split-K layout of 65 536 sequences x 8 KV heads x 64 partitions is
    far beyond the static scratch: refused on the host, nothing enqueued."""
    need = ops.decode_workspace_bytes(65536, 64, 8, 128, 64 * 512, 512)
    assert need > ops.NOALLOC_SCRATCH_BYTES
    L = ops.lib()
    st = L.pa_decode_append_noalloc(16, None, 16, 16, 16, 16, 1, 16, 64, 16, 65536, 64 * 512, 64,
                                    8, 128, 16, 0.1, 512, None, 0, ops.PA_BF16, None)
    assert st == ops.PA_EINVAL
    assert "scratch" in L.pa_last_error().decode()
