"""GPU parity of the rank-trace diagnostics ("What Matters ...", appendix I,
Table 13; the "QEvict" review, section 3: selection churn and future missed
mass) against the CPU oracle, through the C ABI."""
import ctypes

import pytest

from conftest import gpu_available
from decode_kv_cache_gqa_amd import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _gu():
    import gpu_util
    return gpu_util


def test_diag_tiny_fp32_top_budget():
    """1 layer, 8 query / 2 KV heads, d = 64, fp32, k = the budget."""
    w = synth.workload("tiny")
    hist = _gu().run_diag_lockstep(w, 40, w.budget)
    last = hist[-1]
    assert last["steps"] == 40 and last["pairs"] == 39
    assert last["k"] == w.budget and last["retained"] == w.budget


@pytest.mark.parametrize("path", [1, 2])
def test_diag_llama_shape_topk_below_budget(path):
    """Matrix-core path (split and whole-cache attention), 3 layers,
    protected sinks and recent tokens, k < B."""
    w = synth.workload("llama8b_32k").scaled(n_layers=3, prefill_lens=(2083,), budget=209, attn_path=path)
    _gu().run_diag_lockstep(w, 24, 50)


def test_diag_group7_whole_cache_attention():
    w = synth.workload("qwen7b_32k").scaled(n_layers=2, prefill_lens=(700, 1300), budget=150, attn_path=2)
    _gu().run_diag_lockstep(w, 16, 37)


def test_diag_group7_ragged_batch():
    """Groups of 7 query heads, two sequences of different lengths, a k that
    does not divide anything."""
    w = synth.workload("qwen7b_32k").scaled(n_layers=2, prefill_lens=(700, 1300), budget=150)
    _gu().run_diag_lockstep(w, 16, 37)


def test_diag_cumulative_and_scorers():
    """The raw value is the scored observation (VNorm and entropy factors)."""
    w = synth.workload("llama8b_32k").scaled(n_layers=2, prefill_lens=(900,), budget=120,
                                             scorer="vnorm+entropy")
    _gu().run_diag_lockstep(w, 12, 120)
    w = synth.workload("llama8b_32k").scaled(n_layers=2, prefill_lens=(900,), budget=120,
                                             policy="cumulative")
    _gu().run_diag_lockstep(w, 12, 60)


def test_diag_k_above_token_count():
    """k larger than every step's token count: both top-k sets are all the
    step's tokens, so their overlap is the whole step."""
    w = synth.workload("tiny")
    hist = _gu().run_diag_lockstep(w, 6, 100000)
    for d in hist:
        assert d["k"] == d["n"] == d["raw_util_overlap"]


def test_diag_future_missed_mass_tiny():
    w = synth.workload("tiny")
    _gu().run_diag_lockstep(w, 24, w.budget, fmm=True)


def test_diag_future_missed_mass_matrix_core():
    w = synth.workload("llama8b_32k").scaled(n_layers=2, prefill_lens=(1500,), budget=150)
    _gu().run_diag_lockstep(w, 12, 150, fmm=True)


def test_diag_llama8b_32k_full_size_sampled():
    """The 32-layer, 32,768-token workload in the benchmark's configuration
    (k = the budget): the counts of two sampled groups against the oracle's
    statistics on the library's own inputs, for the first steps (including
    the first step's eviction of 29,492 tokens)."""
    w = synth.workload("llama8b_32k_diag")
    hist = _gu().run_diag_lockstep(w, 5, w.diag_topk, sample_heads=[0, 5], check_values=False)
    assert hist[0]["evicted"] == 32769 - w.budget
    for d in hist[1:]:
        assert d["evicted"] == 1 and d["retained"] == w.budget


def test_diag_state_changes_only_by_step():
    import torch
    from decode_kv_cache_gqa_amd import kvev
    w = synth.workload("tiny")
    ctx = kvev.context_for(w, max_steps=2, diag_topk=16)
    plain = kvev.context_for(w, max_steps=2)
    for b in range(w.batch):
        K, V = w.prefill_kv(b, device="cuda")
        ctx.prefill(b, K.contiguous(), V.contiguous())
        plain.prefill(b, K.contiguous(), V.contiguous())
    out = torch.empty((w.n_layers, w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    q, kn, vn = w.step_inputs(1, device="cuda")
    L = kvev.lib()
    assert L.kvev_decode_step(ctx._h, q.data_ptr(), kn.data_ptr(), vn.data_ptr(), out.data_ptr()) == kvev.ESTATE
    assert L.kvev_evict(ctx._h, 0) == kvev.ESTATE
    # diagnostics off: the read calls refuse
    arr = (kvev.DiagGroup * 1)()
    assert L.kvev_diag_read(plain._h, arr, 1) == kvev.ESTATE
    # one of the two contexts without diagnostics
    fm = (ctypes.c_double * 2)()
    assert L.kvev_diag_fmm(plain._h, ctx._h, fm) == kvev.ESTATE
    for t in (1, 2, 3):
        q, kn, vn = w.step_inputs(t, device="cuda")
        ctx.step(q, kn, vn, out, 0)
    # positions reached max_tokens (prefill + 2 steps + 1): the next step refuses
    q, kn, vn = w.step_inputs(4, device="cuda")
    st = L.kvev_step(ctx._h, q.data_ptr(), kn.data_ptr(), vn.data_ptr(), out.data_ptr(), 0)
    assert st == kvev.ESTATE
    d = ctx.diag_read()
    assert d[0]["steps"] == 3
    ctx.sync()
    ctx.close()
    plain.close()


def test_diag_new_token_mean_init():
    """The diagnostics record the new token's utility after its mean start."""
    w = synth.workload("llama8b_32k").scaled(n_layers=2, prefill_lens=(900,), budget=100, attn_path=2,
                                             new_token_init=1)
    _gu().run_diag_lockstep(w, 12, 40)
