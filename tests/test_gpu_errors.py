"""Error handling of the C ABI on live contexts (GPU).

Every rejected call returns its status code, leaves the state as it was, and
the context keeps working afterwards: invalid arguments and calls out of
order are reported, never turned into device work.
"""
import ctypes

import numpy as np
import pytest

from conftest import gpu_available
from decode_kv_cache_gqa_amd import synth

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="no GPU")]


def _status(fn, *a, **kw):
    from decode_kv_cache_gqa_amd import kvev
    with pytest.raises(kvev.KvevError) as e:
        fn(*a, **kw)
    return e.value.status


def _small(**kw):
    base = dict(n_layers=2, prefill_lens=(40,), budget=24, n_sink=2, n_recent=4)
    base.update(kw)
    return synth.workload("llama8b_32k").scaled(**base)


def _out(w):
    import torch
    return torch.empty((w.n_layers, w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")


def test_token_context_rejections_leave_it_usable():
    import torch
    from decode_kv_cache_gqa_amd import kvev
    w = _small()
    ctx = kvev.context_for(w, max_steps=8)
    K, V = w.prefill_kv(0, device="cuda")
    out = _out(w)
    q, kn, vn = w.step_inputs(1, device="cuda")
    # a step before any prefill
    assert _status(ctx.step, q, kn, vn, out) == kvev.ESTATE
    assert _status(ctx.decode_step, q, kn, vn, out) == kvev.ESTATE
    # zero tokens, a null pointer, a sequence out of range, more tokens than the capacity
    assert kvev.lib().kvev_prefill(ctx._h, 0, ctypes.c_void_p(K.data_ptr()), ctypes.c_void_p(V.data_ptr()),
                                   0, None) == kvev.EINVAL
    assert kvev.lib().kvev_prefill(ctx._h, 0, None, ctypes.c_void_p(V.data_ptr()), 40, None) == kvev.EINVAL
    assert kvev.lib().kvev_prefill(ctx._h, 1, ctypes.c_void_p(K.data_ptr()), ctypes.c_void_p(V.data_ptr()),
                                   40, None) == kvev.EINVAL
    cap = ctx.cfg.max_tokens
    big = torch.zeros((w.n_layers, w.n_kv_heads, cap, w.head_dim), dtype=torch.bfloat16, device="cuda")
    assert _status(ctx.prefill, 0, big, big) == kvev.EINVAL
    del big
    # the rejected calls changed nothing: a normal prefill and steps follow
    ctx.prefill(0, K, V)
    assert len(ctx.retained(0, 0)) == 40
    # a budget below the protected tokens (2 sinks + 4 recent)
    assert _status(ctx.evict, 5) == kvev.EINVAL
    # calls of the other modes
    assert _status(ctx.tier_state, 0) == kvev.EINVAL
    assert _status(ctx.block_state, 0) == kvev.EINVAL
    # group index out of range
    assert _status(ctx.retained, 0, w.n_kv_heads) in (kvev.EINVAL, kvev.ERANGE)
    for t in range(1, 4):
        q, kn, vn = w.step_inputs(t, device="cuda")
        ctx.step(q, kn, vn, out)
    for h in range(w.n_kv_heads):
        assert len(ctx.retained(0, h)) == w.budget
    # prefill after the first decode step
    assert _status(ctx.prefill, 0, K, V) == kvev.ESTATE
    q, kn, vn = w.step_inputs(4, device="cuda")
    ctx.step(q, kn, vn, out)
    assert torch.isfinite(out).all()
    ctx.sync()
    ctx.close()


def test_token_capacity_exhaustion_is_reported():
    """With a budget that never binds, the slots fill one per step; the step
    that would need a slot past the capacity is refused and the cache keeps
    its contents."""
    from decode_kv_cache_gqa_amd import kvev
    w = _small(budget=1000)
    ctx = kvev.context_for(w, max_steps=6)  # capacity 40 + 6 + 1 = 47
    K, V = w.prefill_kv(0, device="cuda")
    ctx.prefill(0, K, V)
    out = _out(w)
    cap = ctx.cfg.max_tokens
    refused = None
    for t in range(1, 20):
        q, kn, vn = w.step_inputs(t, device="cuda")
        try:
            ctx.step(q, kn, vn, out)
        except kvev.KvevError as e:
            refused = (t, e.status)
            break
    assert refused is not None and refused[1] == kvev.ESTATE
    kept = ctx.retained(0, 0)
    assert len(kept) == cap
    np.testing.assert_array_equal(np.sort(kept), np.arange(cap))
    ctx.close()


def test_tier_context_rejections():
    from decode_kv_cache_gqa_amd import kvev
    w = synth.workload("qevict131k").scaled(n_layers=2, prefill_lens=(600,), fp_windows=4, int2_windows=6)
    ctx = kvev.context_for(w, max_steps=4)
    out = _out(w)
    q, kn, vn = w.step_inputs(1, device="cuda")
    assert _status(ctx.step, q, kn, vn, out) == kvev.ESTATE
    K, V = w.prefill_kv(0, device="cuda")
    ctx.prefill(0, K, V)
    # the token-granular copy-outs do not apply to windows
    assert _status(ctx.retained, 0, 0) == kvev.EINVAL
    assert _status(ctx.export_kv, 0, 0) == kvev.EINVAL
    # layer out of range
    assert _status(ctx.tier_state, w.n_layers) == kvev.EINVAL
    ctx.step(q, kn, vn, out)
    score, tiers, ledger = ctx.tier_state(0)
    assert len(score) == len(tiers) == len(ledger)
    ctx.sync()
    ctx.close()
