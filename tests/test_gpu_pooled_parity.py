"""GPU parity of the sequence-pooled token mode (one utility and one retained
set per sequence, "What Matters ...", section 3.1 Eq.1) against the CPU
oracle, through the C ABI: the pooled post kernel after the split attention,
or the fold kernel pooling a sequence's KV head groups after the whole-cache
attention (fused step), and the per-sequence selection with the shared
moves (separate evict call)."""
import pytest

from conftest import gpu_available
from decode_kv_cache_gqa_amd import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _gu():
    import gpu_util
    return gpu_util


def _w(**kw):
    base = dict(n_layers=3, prefill_lens=(1500,), budget=160)
    base.update(kw)
    return synth.workload("llama8b_32k_pooled").scaled(**base)


# attention kernels: split (1) and whole-cache (2, its fold pools the sequence's groups)
PATHS = pytest.mark.parametrize("path", [1, 2], ids=["split", "whole"])


@PATHS
@pytest.mark.parametrize("fused", [False, True])
def test_pooled_llama_shape(fused, path):
    st = _gu().run_pooled_lockstep(_w(attn_path=path), 24, fused=fused)
    assert st.steps == 24


@PATHS
def test_pooled_batch_lazy_refresh(path):
    w = _w(n_layers=2, prefill_lens=(700, 513, 900), budget=120, refresh_interval=4,
           n_sink=0, n_recent=8, attn_path=path)
    _gu().run_pooled_lockstep(w, 18, fused=True, sample_seqs=[0, 1, 2])


def test_pooled_scorers_group_7():
    w = _w(n_layers=2, n_q_heads=28, n_kv_heads=4, prefill_lens=(800,), budget=100,
           scorer="vnorm+entropy")
    _gu().run_pooled_lockstep(w, 16)
    _gu().run_pooled_lockstep(w, 16, fused=True)


def test_pooled_fp32_vector_path():
    w = synth.workload("tiny").scaled(granularity="sequence", scorer="entropy")
    st = _gu().run_pooled_lockstep(w, 24, fused=True)
    assert st.max_out_err <= 1e-5 and st.max_score_err <= 1e-5


@PATHS
def test_pooled_single_kv_head_and_cumulative(path):
    w = _w(n_layers=2, n_q_heads=8, n_kv_heads=1, prefill_lens=(600,), budget=90,
           policy="cumulative", attn_path=path)
    _gu().run_pooled_lockstep(w, 12)


@PATHS
def test_pooled_smaller_budget_after_single_token_evictions(path):
    """The per-sequence free slot (left by single-token evictions of the
    fused step) is filled from the last slot of every KV head before a
    kvev_evict with a smaller budget selects."""
    import numpy as np
    import torch
    import oracle as orc
    from decode_kv_cache_gqa_amd import kvev
    gu = _gu()
    w = _w(n_layers=2, prefill_lens=(400,), budget=90, n_sink=2, n_recent=5, attn_path=path)
    ctx = kvev.context_for(w, max_steps=16)
    o = orc.PooledTokenOracle(w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim, budget=90,
                              alpha_new=w.alpha_new, n_sink=2, n_recent=5, capacity=420)
    K, V = w.prefill_kv(0, device="cuda")
    ctx.prefill(0, K, V)
    Kc, Vc = w.prefill_kv(0, device="cpu")
    o.prefill(0, Kc.float().numpy(), Vc.float().numpy())
    out = torch.empty((w.n_layers, 1, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")

    def compare(what):
        gp0 = ctx.retained(0, 0)
        gps, gss = gu.by_position(gp0, ctx.scores(0, 0))
        ops, oss = gu.by_position(o.positions(0), o.scores(0))
        np.testing.assert_array_equal(gps, ops, err_msg=f"{what} positions")
        gu.check_scores(gss, oss, 2e-3, f"{what} scores")
        st = o.seqs[0]
        for h in range(w.n_kv_heads):
            np.testing.assert_array_equal(ctx.retained(0, h), gp0)
            gk, gv = ctx.export_kv(0, h)
            rk = torch.from_numpy(gu.rows_by_position(st.K[:, h], st.pos[:st.n], gp0).copy()).to(torch.bfloat16)
            rv = torch.from_numpy(gu.rows_by_position(st.V[:, h], st.pos[:st.n], gp0).copy()).to(torch.bfloat16)
            assert torch.equal(gk.cpu(), rk) and torch.equal(gv.cpu(), rv), f"{what} kvh={h} K/V"

    for t in range(1, 7):
        q, kn, vn = w.step_inputs(t, device="cuda")
        ctx.step(q, kn, vn, out, 90)
        qc, knc, vnc = w.step_inputs(t, device="cpu")
        o.decode_step(t, qc.float().numpy(), knc.float().numpy(), vnc.float().numpy(), [0])
        o.evict(90)
    compare("after single-token evictions")
    ctx.evict(75)
    o.evict(75)
    compare("after the smaller budget")
    ctx.sync()
    ctx.close()


@PATHS
@pytest.mark.parametrize("fused", [False, True])
def test_pooled_new_token_mean_init(fused, path):
    st = _gu().run_pooled_lockstep(_w(new_token_init=1, attn_path=path), 16, fused=fused)
    assert st.steps == 16
