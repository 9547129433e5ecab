"""GPU parity of the token-granular path (append, split attention, probability
pass + layer-sequential fold, radix-select, hole-fill compaction) against
the CPU oracle, through the C ABI."""
import numpy as np
import pytest

from conftest import gpu_available
from decode_kv_cache_gqa_amd import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _gu():
    import gpu_util
    return gpu_util


def test_generator_identical_on_cpu_and_gpu():
    import torch
    w = synth.workload("llama8b_32k").scaled(n_layers=2, prefill_lens=(3000,))
    Kg, Vg = w.prefill_kv(0, device="cuda", layers=[1], heads=[3, 6])
    Kc, Vc = w.prefill_kv(0, device="cpu", layers=[1], heads=[3, 6])
    assert torch.equal(Kg.cpu(), Kc) and torch.equal(Vg.cpu(), Vc)
    for t in (1, 77):
        g = w.step_inputs(t, device="cuda")
        c = w.step_inputs(t, device="cpu")
        for a, b in zip(g, c):
            assert torch.equal(a.cpu(), b)


def test_tiny_fp32_full_run():
    """1 layer, 8 query / 2 KV heads, d=64, fp32, prefill 512, 64 steps, B=128."""
    st = _gu().run_token_lockstep(synth.workload("tiny"), 64)
    assert st.steps == 64 and st.exact_selection_checks == 128
    assert st.max_out_err <= 1e-5 and st.max_score_err <= 1e-5


def test_tiny_fp32_fused_step():
    st = _gu().run_token_lockstep(synth.workload("tiny"), 64, fused=True)
    assert st.steps == 64


def test_llama_shape_fused_step():
    w = synth.workload("llama8b_32k").scaled(n_layers=3, prefill_lens=(2083,), budget=209)
    _gu().run_token_lockstep(w, 40, fused=True)


def test_lazy_fused_step():
    w = synth.workload("lazy16x8k").scaled(n_layers=2, prefill_lens=(1000, 1000, 1000), budget=250)
    _gu().run_token_lockstep(w, 20, fused=True)


def test_fused_step_bitwise_equals_separate_calls():
    """kvev_step == kvev_decode_step + kvev_evict, bit for bit (outputs,
    utilities, slot layout and cached K/V), including the first step's
    large compaction and many single-eviction steps."""
    import torch
    from decode_kv_cache_gqa_amd import kvev
    w = synth.workload("llama8b_32k").scaled(n_layers=4, prefill_lens=(5000,), budget=500)
    ctxs = [kvev.context_for(w, max_steps=24) for _ in range(2)]
    K, V = w.prefill_kv(0, device="cuda")
    for c in ctxs:
        c.prefill(0, K, V)
    outs = [torch.empty((4, 1, 32, 128), dtype=torch.float32, device="cuda") for _ in range(2)]
    for t in range(1, 25):
        q, kn, vn = w.step_inputs(t, device="cuda")
        ctxs[0].step(q, kn, vn, outs[0])
        ctxs[1].decode_step(q, kn, vn, outs[1])
        ctxs[1].evict()
        assert torch.equal(outs[0], outs[1]), t
        for h in range(w.n_kv_heads):
            np.testing.assert_array_equal(ctxs[0].retained(0, h), ctxs[1].retained(0, h))
            np.testing.assert_array_equal(ctxs[0].scores(0, h), ctxs[1].scores(0, h))
    for h in (0, 7):
        a = ctxs[0].export_kv(0, h)
        b = ctxs[1].export_kv(0, h)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    for c in ctxs:
        c.sync()
        c.close()


def test_llama_shape_scaled_ragged():
    """Llama-8B head shape, bf16, 3 layers, ragged prefill, 4 sinks + 32 recent."""
    w = synth.workload("llama8b_32k").scaled(n_layers=3, prefill_lens=(2083,), budget=209)
    st = _gu().run_token_lockstep(w, 40)
    assert st.steps == 40


def test_cumulative_policy():
    w = synth.workload("llama8b_32k").scaled(n_layers=2, prefill_lens=(700,), budget=100,
                                             policy="cumulative")
    _gu().run_token_lockstep(w, 12)


def test_lazy_refresh_batch():
    """Batched lazy refresh (r=8), no protection, 3 sequences of a ragged length."""
    w = synth.workload("lazy16x8k").scaled(n_layers=2, prefill_lens=(1000, 1000, 1000), budget=250)
    _gu().run_token_lockstep(w, 20, sample_seqs=[0, 2])


def test_score_free_batch():
    w = synth.workload("scorefree16x8k").scaled(n_layers=2, prefill_lens=(900, 900), budget=240)
    _gu().run_token_lockstep(w, 20)


def test_edge_budget_not_binding_and_tiny_prefill():
    # prefill of 1 token, budget larger than the cache: evict is a no-op
    w = synth.workload("llama8b_32k").scaled(n_layers=1, prefill_lens=(1, 17), budget=40,
                                             n_sink=1, n_recent=2)
    _gu().run_token_lockstep(w, 30)


def test_capacity_not_multiple_of_16_filled():
    """The budget never binds and the slot capacity (prefill + steps + 1 = 45)
    is not a multiple of 16: on the last steps the logit rows, whose stride is
    the slot count rounded up to 16 (48), must stay inside their buffer."""
    w = synth.workload("llama8b_32k").scaled(n_layers=2, prefill_lens=(20,), budget=100,
                                             n_sink=1, n_recent=2)
    _gu().run_token_lockstep(w, 24)


def test_equal_scores_resolved_by_position():
    """All-zero keys give every token the same logits, so utilities tie
    exactly; the cut must fall by position (more recent kept)."""
    import torch
    from decode_kv_cache_gqa_amd import kvev
    w = synth.workload("llama8b_32k").scaled(n_layers=2, prefill_lens=(300,), budget=50,
                                             n_sink=0, n_recent=0)
    ctx = kvev.context_for(w, max_steps=4)
    K, V = w.prefill_kv(0, device="cuda")
    ctx.prefill(0, torch.zeros_like(K), V.contiguous())
    q, kn, vn = w.step_inputs(1, device="cuda")
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ctx.decode_step(q, torch.zeros_like(kn), vn, out)
    s = ctx.scores(0, 0)
    assert np.all(s == s[0])
    ctx.evict()
    for h in range(w.n_kv_heads):
        got = np.sort(ctx.retained(0, h))
        np.testing.assert_array_equal(got, np.arange(301 - 50, 301))
    ctx.close()


def test_determinism_bitwise():
    import torch
    from decode_kv_cache_gqa_amd import kvev
    w = synth.workload("llama8b_32k").scaled(n_layers=2, prefill_lens=(1500,), budget=150)
    runs = []
    for _ in range(2):
        ctx = kvev.context_for(w, max_steps=6)
        K, V = w.prefill_kv(0, device="cuda")
        ctx.prefill(0, K, V)
        out = torch.empty((2, 1, 32, 128), dtype=torch.float32, device="cuda")
        outs = []
        for t in range(1, 7):
            ctx.decode_step(*w.step_inputs(t, device="cuda"), out)
            ctx.evict()
            outs.append(out.cpu().clone())
        runs.append((outs, [ctx.scores(0, h) for h in range(8)], [ctx.retained(0, h) for h in range(8)]))
        ctx.close()
    for a, b in zip(runs[0][0], runs[1][0]):
        assert torch.equal(a, b)
    for a, b in zip(runs[0][1], runs[1][1]):
        np.testing.assert_array_equal(a, b)
    for a, b in zip(runs[0][2], runs[1][2]):
        np.testing.assert_array_equal(a, b)


def test_llama8b_32k_full_size_sampled():
    """The full 32-layer, 32,768-token workload in the benchmark's launch
    configuration; the oracle follows two sampled KV-head groups."""
    w = synth.workload("llama8b_32k")
    st = _gu().run_token_lockstep(w, 6, sample_heads=[0, 5], kv_every=3, ctx_steps=w.steps)
    assert st.steps == 6


def test_lazy16x8k_full_size_sampled():
    """The full batched lazy workload (16 sequences, 8,192-token prefill, 32
    layers, budget 2,048, observations at t = 1, 9, 17, ...) in the
    benchmark's launch configuration; the oracle follows two sequences' first
    and last KV heads through the first eviction, the unobserved steps and
    the observation at t = 9."""
    w = synth.workload("lazy16x8k")
    st = _gu().run_token_lockstep(w, 10, sample_seqs=[0, 15], sample_heads=[0, 7], kv_every=5,
                                  ctx_steps=w.steps, fused=True)
    assert st.steps == 10


def test_scorefree16x8k_full_size_sampled():
    """The full batched score-free workload (scores observed at t = 1 only,
    new tokens take the mean) in the benchmark's launch configuration."""
    w = synth.workload("scorefree16x8k")
    st = _gu().run_token_lockstep(w, 6, sample_seqs=[7], sample_heads=[3], kv_every=3, ctx_steps=w.steps,
                                  fused=True)
    assert st.steps == 6


def test_llama8b_32k_full_size_fused_sampled():
    w = synth.workload("llama8b_32k")
    st = _gu().run_token_lockstep(w, 6, sample_heads=[3], kv_every=3, ctx_steps=w.steps, fused=True)
    assert st.steps == 6


# --- query group sizes other than 4 ----------------------------------------------

@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (24, 8), (20, 4), (30, 5), (28, 4), (32, 4)])
def test_group_sizes_matrix_core_path(hq, hkv):
    """bf16, head_dim 128 (matrix-core kernel) with 1..8 query heads per KV
    head; (28, 4) is the Qwen2.5-7B attention shape."""
    w = synth.workload("llama8b_32k").scaled(n_layers=2, n_q_heads=hq, n_kv_heads=hkv,
                                             prefill_lens=(700, 433), budget=120)
    _gu().run_token_lockstep(w, 12)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("f32", 128)])
def test_group_size_7_vector_path(dtype, d):
    w = synth.workload("tiny").scaled(n_q_heads=14, n_kv_heads=2, head_dim=d, dtype=dtype,
                                      prefill_lens=(300,), budget=90)
    _gu().run_token_lockstep(w, 16)


# --- scorer variants ([InertiaKV] section 5.1) ------------------------------------

@pytest.mark.parametrize("scorer", ["vnorm", "entropy", "vnorm+entropy"])
def test_scorers_matrix_core_path(scorer):
    w = synth.workload("llama8b_32k").scaled(n_layers=3, prefill_lens=(1100,), budget=150,
                                             scorer=scorer)
    _gu().run_token_lockstep(w, 16)


@pytest.mark.parametrize("scorer", ["vnorm", "entropy", "vnorm+entropy"])
def test_scorers_fp32_vector_path(scorer):
    st = _gu().run_token_lockstep(synth.workload("tiny").scaled(scorer=scorer), 24)
    assert st.max_out_err <= 1e-5 and st.max_score_err <= 1e-5


def test_scorers_with_lazy_refresh_and_group_7():
    """Observations only every 4th step (the scorer outputs are skipped in
    between) on a group of 7, batch of 2."""
    w = synth.workload("lazy16x8k").scaled(n_layers=2, n_q_heads=28, n_kv_heads=4,
                                           prefill_lens=(640, 515), budget=160,
                                           refresh_interval=4, scorer="vnorm+entropy")
    _gu().run_token_lockstep(w, 14)


def test_scorers_fused_step():
    w = synth.workload("llama8b_32k").scaled(n_layers=2, prefill_lens=(900,), budget=100,
                                             scorer="vnorm+entropy")
    _gu().run_token_lockstep(w, 12, fused=True)


@pytest.mark.parametrize("fused", [True, False])
def test_smaller_budget_after_single_token_evictions(fused):
    """A single-token eviction leaves its slot free inside the cache (the
    next token takes it).  A later kvev_evict with a smaller budget first
    moves the last token into that slot, then selects; the result must match
    the oracle by position (retained set, utilities, K/V rows)."""
    import torch
    import oracle as orc
    from decode_kv_cache_gqa_amd import kvev
    gu = _gu()
    w = synth.workload("llama8b_32k").scaled(n_layers=2, prefill_lens=(500,), budget=120,
                                             n_sink=2, n_recent=6)
    ctx = kvev.context_for(w, max_steps=16)
    o = orc.TokenModeOracle(w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim, budget=120,
                            alpha_new=w.alpha_new, n_sink=2, n_recent=6, capacity=520)
    K, V = w.prefill_kv(0, device="cuda")
    ctx.prefill(0, K, V)
    Kc, Vc = w.prefill_kv(0, device="cpu")
    o.prefill(0, Kc.float().numpy(), Vc.float().numpy())
    out = torch.empty((w.n_layers, 1, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")

    def step(t, B):
        q, kn, vn = w.step_inputs(t, device="cuda")
        if fused:
            ctx.step(q, kn, vn, out, B)
        else:
            ctx.decode_step(q, kn, vn, out)
            ctx.evict(B)
        qc, knc, vnc = w.step_inputs(t, device="cpu")
        o.decode_step(t, qc.float().numpy(), knc.float().numpy(), vnc.float().numpy(), [0])
        o.evict(B)

    def compare(what):
        for h in range(w.n_kv_heads):
            gp = ctx.retained(0, h)
            gps, gss = gu.by_position(gp, ctx.scores(0, h))
            ops, oss = gu.by_position(o.positions(0, h), o.scores(0, h))
            np.testing.assert_array_equal(gps, ops, err_msg=f"{what} kvh={h} positions")
            gu.check_scores(gss, oss, 2e-3, f"{what} kvh={h} scores")
            gk, gv = ctx.export_kv(0, h)
            g = o.groups[(0, h)]
            rk = torch.from_numpy(gu.rows_by_position(g.K, g.pos[:g.n], gp).copy()).to(torch.bfloat16)
            rv = torch.from_numpy(gu.rows_by_position(g.V, g.pos[:g.n], gp).copy()).to(torch.bfloat16)
            assert torch.equal(gk.cpu(), rk) and torch.equal(gv.cpu(), rv), f"{what} kvh={h} K/V"

    for t in range(1, 7):
        step(t, 120)  # t = 1 compacts 501 -> 120, then single-token evictions
    compare("after single-token evictions")
    ctx.evict(100)
    o.evict(100)
    compare("after the smaller budget")
    for t in range(7, 12):
        step(t, 100)
    compare("after further steps")
    ctx.sync()
    ctx.close()
