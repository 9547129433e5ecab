"""GPU parity of the block mode's host-offload tier ("MemDecay" section
III-E: pages offloaded to host memory before they are dropped and recovered
when relevant again; the "Attention-Aware Block Eviction" page: a block's
state survives its eviction) through the C ABI: a context that re-admits
from its pinned host pool against one that is handed the original K/V, and
the pool's contents against the oracle's ring model."""
import numpy as np
import pytest

from conftest import gpu_available
from decode_kv_cache_gqa_amd import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _gu():
    import gpu_util
    return gpu_util


def _scaled(**kw):
    base = dict(n_layers=2, n_q_heads=8, n_kv_heads=2, prefill_lens=(300, 517, 704, 1000),
                n_epochs=3, epoch_steps=16)
    base.update(kw)
    return synth.workload("lrfu64").scaled(**base)


@pytest.mark.parametrize("path", [0, 2], ids=["auto", "whole"])
def test_offload_pool_large_enough_for_every_eviction(path):
    """Every block evicted by the first selection fits the pool: each epoch's
    heavy blocks come back from host memory, bit-exact (also with the
    whole-cache attention over the block tables, which the full-size
    workload takes)."""
    st = _gu().run_offload_twins(_scaled(attn_path=path), 48, 512)
    assert st["readmitted"] > 0 and st["dropped"] == 0 and st["refused"] == 0


def test_offload_pool_overflow_and_ring_reuse():
    """A pool smaller than the first selection's evictions (only the last ones
    by (sequence, block id) are kept) and ring reuse afterwards; blocks no
    longer in the pool are refused."""
    st = _gu().run_offload_twins(_scaled(), 48, 24)
    assert st["dropped"] > 0 and st["readmitted"] > 0 and st["refused"] > 0


def test_offload_with_background_prefetch():
    """Blocks prefetched into device staging one step before their
    re-admission (the copy overlaps that step) come back bit-exact; a pool
    smaller than the first selection keeps some prefetch targets out."""
    st = _gu().run_offload_twins(_scaled(), 48, 512, prefetch=64)
    assert st["prefetched"] > 0 and st["readmitted"] > 0
    st = _gu().run_offload_twins(_scaled(), 48, 24, prefetch=4)
    assert st["prefetched"] > 0


@pytest.mark.parametrize("min_score", [0.01, 1e9])
def test_offload_score_threshold(min_score):
    """The graded rule: evicted blocks scoring below the threshold are
    dropped, the rest offloaded (1e9: nothing reaches the pool, every
    recovery is refused); the pool still matches the oracle's model."""
    st = _gu().run_offload_twins(_scaled(), 40, 64, min_score=min_score, prefetch=8)
    assert st["below_threshold"] > 0
    if min_score > 1e8:
        assert st["offloaded"] == 0 and st["readmitted"] == 0


def test_offload_separate_calls_fp32():
    """kvev_decode_step + kvev_evict (the standalone selection offloads too),
    fp32, d = 64, one layer."""
    w = _scaled(dtype="f32", head_dim=64, prefill_lens=(257, 640), n_layers=1)
    st = _gu().run_offload_twins(w, 40, 64, fused=False)
    assert st["readmitted"] > 0


def test_offload_refusals():
    import torch
    from decode_kv_cache_gqa_amd import kvev
    w = _scaled(prefill_lens=(320,))
    off = kvev.context_for(w, max_steps=4, offload_blocks=8)
    plain = kvev.context_for(w, max_steps=4)
    K, V = w.prefill_kv(0, device="cuda")
    for c in (off, plain):
        c.prefill(0, K.contiguous(), V.contiguous(), w.region_labels(0))
        c.set_budget(0, w.block_budget(0))
    out = torch.empty((w.n_layers, 1, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    q, kn, vn = w.step_inputs(1, device="cuda")
    off.step(q, kn, vn, out)
    slots = off.offload_state(0)
    res = np.asarray(off.block_state(0)[2], dtype=bool)
    pooled = np.flatnonzero(slots >= 0)
    assert len(pooled) == min(8, int((~res).sum()))
    L = kvev.lib()
    ids = np.array([int(np.flatnonzero(res)[0])], dtype=np.int64)  # a resident block
    assert L.kvev_readmit_offloaded(off._h, 0, 1, ids.ctypes.data) == kvev.EINVAL
    dropped = [j for j in np.flatnonzero(~res) if slots[j] < 0]
    if dropped:
        ids = np.array([dropped[0]], dtype=np.int64)
        assert L.kvev_readmit_offloaded(off._h, 0, 1, ids.ctypes.data) == kvev.ESTATE
    ids = np.array([int(pooled[0])], dtype=np.int64)
    assert L.kvev_readmit_offloaded(plain._h, 0, 1, ids.ctypes.data) == kvev.ESTATE  # offload off
    import ctypes
    buf = np.zeros(64, np.int32)
    n = ctypes.c_int64()
    assert L.kvev_offload_state(plain._h, 0, buf.ctypes.data, 64, ctypes.byref(n)) == kvev.ESTATE
    st, tr, rs = off.block_state(0)
    kk = torch.zeros((w.n_layers, w.n_kv_heads, 16, w.head_dim), dtype=w.torch_dtype, device="cuda")
    assert L.kvev_import_blocks(off._h, 0, len(st), st.ctypes.data, tr.ctypes.data, rs.ctypes.data, 16,
                                kk.data_ptr(), kk.data_ptr()) == kvev.ESTATE
    # the refused calls left the context intact: a recovery and a step still work
    off.readmit_offloaded(0, [int(pooled[0])])
    assert off.offload_state(0)[pooled[0]] == -1
    q, kn, vn = w.step_inputs(2, device="cuda")
    off.step(q, kn, vn, out)
    off.sync()
    off.close()
    plain.close()


def test_readmit_with_caller_kv_releases_the_slot():
    """kvev_readmit (K/V from the caller) on an offload context also releases
    the block's pool slot (a resident block holds none), so a later eviction
    of the block takes a fresh slot and the pool follows the oracle's model."""
    import torch
    from decode_kv_cache_gqa_amd import kvev
    import gpu_util
    import oracle as orc
    w = _scaled(prefill_lens=(640,), n_epochs=1, epoch_steps=0)
    ctx = kvev.context_for(w, max_steps=40, offload_blocks=64)
    K, V = w.prefill_kv(0, device="cuda")
    ctx.prefill(0, K.contiguous(), V.contiguous(), w.region_labels(0))
    ctx.set_budget(0, w.block_budget(0))
    pool = orc.HostOffloadPool(64)
    out = torch.empty((w.n_layers, 1, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    readmitted = False
    for t in range(1, 41):
        before = np.asarray(ctx.block_state(0)[2], dtype=bool)
        q, kn, vn = w.step_inputs(t, device="cuda")
        ctx.step(q, kn, vn, out)
        now = np.asarray(ctx.block_state(0)[2], dtype=bool)
        was = np.zeros_like(now)
        was[:len(before)] = before
        pool.offload([(0, int(j)) for j in np.flatnonzero(was & ~now)])
        slots = ctx.offload_state(0)
        np.testing.assert_array_equal(slots, [pool.slot((0, j)) for j in range(len(slots))],
                                      err_msg=f"step {t}: pool slots")
        if t == 3:
            j = int(np.flatnonzero(slots >= 0)[0])
            Kr, Vr = gpu_util.block_rows(w, 0, [j], "cuda")
            ctx.readmit(0, [j], Kr, Vr)
            pool.readmit((0, j))
            assert ctx.offload_state(0)[j] == -1
            readmitted = True
    assert readmitted
    ctx.sync()
    ctx.close()
