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


@pytest.mark.parametrize("path", [1, 2])
def test_llama_shape_fused_step(path):
    w = synth.workload("llama8b_32k").scaled(n_layers=3, prefill_lens=(2083,), budget=209, attn_path=path)
    _gu().run_token_lockstep(w, 40, fused=True)


@pytest.mark.parametrize("path", [1, 2])
def test_lazy_fused_step(path):
    w = synth.workload("lazy16x8k").scaled(n_layers=2, prefill_lens=(1000, 1000, 1000), budget=250,
                                           attn_path=path)
    _gu().run_token_lockstep(w, 20, fused=True)


@pytest.mark.parametrize("path", [1, 2])
def test_fused_step_bitwise_equals_separate_calls(path):
    """kvev_step == kvev_decode_step + kvev_evict, bit for bit (outputs,
    utilities, slot layout and cached K/V), including the first step's
    large compaction and many single-eviction steps."""
    import torch
    from decode_kv_cache_gqa_amd import kvev
    w = synth.workload("llama8b_32k").scaled(n_layers=4, prefill_lens=(5000,), budget=500, attn_path=path)
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


@pytest.mark.parametrize("path", [1, 2])
def test_llama_shape_scaled_ragged(path):
    """Llama-8B head shape, bf16, 3 layers, ragged prefill, 4 sinks + 32 recent."""
    w = synth.workload("llama8b_32k").scaled(n_layers=3, prefill_lens=(2083,), budget=209,
                                             attn_path=path)
    st = _gu().run_token_lockstep(w, 40)
    assert st.steps == 40


@pytest.mark.parametrize("path", [1, 2])
def test_cumulative_policy(path):
    w = synth.workload("llama8b_32k").scaled(n_layers=2, prefill_lens=(700,), budget=100,
                                             policy="cumulative", attn_path=path)
    _gu().run_token_lockstep(w, 12)


@pytest.mark.parametrize("path", [1, 2])
def test_lazy_refresh_batch(path):
    """Batched lazy refresh (r=8), no protection, 3 sequences of a ragged length."""
    w = synth.workload("lazy16x8k").scaled(n_layers=2, prefill_lens=(1000, 1000, 1000), budget=250,
                                           attn_path=path)
    _gu().run_token_lockstep(w, 20, sample_seqs=[0, 2])


@pytest.mark.parametrize("path", [1, 2])
def test_score_free_batch(path):
    w = synth.workload("scorefree16x8k").scaled(n_layers=2, prefill_lens=(900, 900), budget=240,
                                                attn_path=path)
    _gu().run_token_lockstep(w, 20)


@pytest.mark.parametrize("path", [1, 2])
def test_edge_budget_not_binding_and_tiny_prefill(path):
    # prefill of 1 token, budget larger than the cache: evict is a no-op
    w = synth.workload("llama8b_32k").scaled(n_layers=1, prefill_lens=(1, 17), budget=40,
                                             n_sink=1, n_recent=2, attn_path=path)
    _gu().run_token_lockstep(w, 30)


@pytest.mark.parametrize("path", [1, 2])
def test_capacity_not_multiple_of_16_filled(path):
    """The budget never binds and the slot capacity (prefill + steps + 1 = 45)
    is not a multiple of 16: on the last steps the logit rows, whose stride is
    the slot count rounded up to 16 (48), must stay inside their buffer."""
    w = synth.workload("llama8b_32k").scaled(n_layers=2, prefill_lens=(20,), budget=100,
                                             n_sink=1, n_recent=2, attn_path=path)
    _gu().run_token_lockstep(w, 24)


@pytest.mark.parametrize("path", [1, 2])
def test_equal_scores_resolved_by_position(path):
    """All-zero keys give every token the same logits, so utilities tie
    exactly; the cut must fall by position (more recent kept)."""
    import torch
    from decode_kv_cache_gqa_amd import kvev
    w = synth.workload("llama8b_32k").scaled(n_layers=2, prefill_lens=(300,), budget=50,
                                             n_sink=0, n_recent=0, attn_path=path)
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


@pytest.mark.parametrize("path", [1, 2])
def test_determinism_bitwise(path):
    import torch
    from decode_kv_cache_gqa_amd import kvev
    w = synth.workload("llama8b_32k").scaled(n_layers=2, prefill_lens=(1500,), budget=150,
                                             attn_path=path)
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


# --- query group sizes other than 4 ----------------------------------------------

@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (24, 8), (20, 4), (30, 5), (28, 4), (32, 4)])
def test_group_sizes_matrix_core_path(hq, hkv, path):
    """bf16, head_dim 128 (matrix-core kernel) with 1..8 query heads per KV
    head; (28, 4) is the Qwen2.5-7B attention shape."""
    w = synth.workload("llama8b_32k").scaled(n_layers=2, n_q_heads=hq, n_kv_heads=hkv,
                                             prefill_lens=(700, 433), budget=120, attn_path=path)
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


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("fused", [True, False])
def test_smaller_budget_after_single_token_evictions(fused, path):
    """A single-token eviction leaves its slot free inside the cache (the
    next token takes it).  A later kvev_evict with a smaller budget first
    moves the last token into that slot, then selects; the result must match
    the oracle by position (retained set, utilities, K/V rows)."""
    import torch
    import oracle as orc
    from decode_kv_cache_gqa_amd import kvev
    gu = _gu()
    w = synth.workload("llama8b_32k").scaled(n_layers=2, prefill_lens=(500,), budget=120,
                                             n_sink=2, n_recent=6, attn_path=path)
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


def test_single_step_rule_alpha_one():
    """alpha_new = 1, the single-step rule ("What Matters ...", section 3.1
    Eq.2): every observation replaces the utility, so after a step's
    layer-sequential fold a token's utility is the last layer's group mass
    and the retained set is the top budget of that mass.  Checked in
    lockstep with the oracle over 12 steps, and on the library's own values:
    the utilities of the first step equal the oracle's last-layer group mass
    and the selection keeps the top budget of them."""
    import torch
    import oracle as orc
    from decode_kv_cache_gqa_amd import kvev
    gu = _gu()
    w = synth.workload("llama8b_32k").scaled(n_layers=3, prefill_lens=(1200,), budget=150, alpha_new=1.0)
    gu.run_token_lockstep(w, 12)
    gu.run_token_lockstep(w, 12, fused=True)
    ctx = kvev.context_for(w, max_steps=2)
    K, V = w.prefill_kv(0, device="cuda")
    ctx.prefill(0, K, V)
    o = orc.TokenModeOracle(w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim, budget=w.budget,
                            alpha_new=1.0, n_sink=w.n_sink, n_recent=w.n_recent, capacity=1300)
    o.prefill(0, K.float().cpu().numpy(), V.float().cpu().numpy())
    q, kn, vn = w.step_inputs(1, device="cuda")
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ctx.decode_step(q, kn, vn, out)
    o.decode_step(1, q.float().cpu().numpy(), kn.float().cpu().numpy(), vn.float().cpu().numpy(), [0])
    pre = {}
    for h in range(w.n_kv_heads):
        gp, gs = ctx.retained(0, h), ctx.scores(0, h)
        gps, gss = gu.by_position(gp, gs)
        last = o.last_G[(w.n_layers - 1, 0, h)]  # oracle slot order = position order before any eviction
        np.testing.assert_array_equal(gps, o.positions(0, h))
        gu.check_scores(gss, last, 2e-3, f"kvh={h}: utility vs the last layer's mass")
        pre[h] = (gs, gp)
    ctx.evict()
    for h in range(w.n_kv_heads):
        gs, gp = pre[h]
        np.testing.assert_array_equal(np.sort(ctx.retained(0, h)),
                                      gu.expected_after_evict(gs, gp, w.budget, w.n_sink, w.n_recent))
    ctx.sync()
    ctx.close()


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("fused", [False, True])
def test_new_token_mean_init(path, fused):
    """new_token_init = mean: on an observation step the new token starts at
    the mean of its group's other utilities, then is folded ("What Matters
    ...", appendix E's rule for the other steps, read for observation steps
    too), with protection, on both attention kernels."""
    w = synth.workload("llama8b_32k").scaled(n_layers=3, prefill_lens=(1100,), budget=120,
                                             new_token_init=1, attn_path=path)
    st = _gu().run_token_lockstep(w, 24, fused=fused)
    assert st.steps == 24


@pytest.mark.parametrize("policy,r", [("cumulative", 1), ("ema", 4)])
def test_new_token_mean_init_cumulative_and_lazy(policy, r):
    w = synth.workload("llama8b_32k").scaled(n_layers=2, prefill_lens=(700, 900), budget=100,
                                             policy=policy, refresh_interval=r, new_token_init=1,
                                             attn_path=2)
    _gu().run_token_lockstep(w, 16, fused=True)
    _gu().run_token_lockstep(w.scaled(attn_path=1), 16)


@pytest.mark.parametrize("path,expect", [(1, "attn"), (2, "attn_whole")])
def test_attention_kernel_choice(path, expect):
    """attn_path picks the kernel the steady steps run (the launches name
    themselves when profiling)."""
    import torch
    from decode_kv_cache_gqa_amd import kvev
    w = synth.workload("llama8b_32k").scaled(n_layers=2, prefill_lens=(700,), budget=100, attn_path=path)
    ctx = kvev.context_for(w, max_steps=6)
    K, V = w.prefill_kv(0, device="cuda")
    ctx.prefill(0, K, V)
    out = torch.empty((w.n_layers, 1, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    ctx.step(*w.step_inputs(1, device="cuda"), out)
    ctx.sync()
    ctx.profile(True)
    for t in range(2, 6):
        ctx.step(*w.step_inputs(t, device="cuda"), out)
    ctx.sync()
    ran = {k: ctx.profile_read(k)[1] for k in ("attn", "attn_whole")}
    ctx.close()
    other = "attn_whole" if expect == "attn" else "attn"
    assert ran[expect] == 4 and ran[other] == 0


@pytest.mark.parametrize("fused", [False, True])
def test_whole_cache_attention_four_wave_workgroups(fused):
    """512 (group, layer) pairs or more (two rounds of the chip) take the
    whole-cache kernel's 4-wave workgroups: 16 sequences x 8 KV heads x 4
    layers, ragged prefills, lazy refresh."""
    lens = tuple(500 + 37 * i for i in range(16))
    w = synth.workload("lazy16x8k").scaled(n_layers=4, prefill_lens=lens, budget=150, attn_path=2)
    st = _gu().run_token_lockstep(w, 12, sample_seqs=[0, 7, 15], fused=fused)
    assert st.steps == 12
