"""GPU parity of the block-granular LRFU path (block open, attention by the
split kernel or the whole-cache kernel over the block tables, block mass
over every layer and head, EMA score and access clock, region
decay priority, pinned selection, stable table compaction, re-admission with
persisted scores) against the CPU oracle, through the C ABI."""
import numpy as np
import pytest

from conftest import gpu_available
from decode_kv_cache_gqa_amd import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _gu():
    import gpu_util
    return gpu_util


# attention kernels: split (1) and whole-cache (2)
PATHS = pytest.mark.parametrize("path", [1, 2], ids=["split", "whole"])


def _scaled(**kw):
    base = dict(n_layers=2, n_q_heads=8, n_kv_heads=2, prefill_lens=(300, 517, 704, 1000),
                n_epochs=3, epoch_steps=16)
    base.update(kw)
    return synth.workload("lrfu64").scaled(**base)


@PATHS
def test_block_lrfu_fused_step_with_readmission(path):
    """4 sequences (ragged, one a multiple of 16), 2 layers, bf16 d=128,
    48 steps over 3 heavy-key epochs with re-admission at each boundary."""
    st = _gu().run_block_lockstep(_scaled(attn_path=path), 48)
    assert st.steps == 48 and st.readmitted > 0 and st.kv_checks > 0


@PATHS
def test_block_lrfu_separate_calls(path):
    st = _gu().run_block_lockstep(_scaled(prefill_lens=(450, 333), attn_path=path), 40, fused=False)
    assert st.steps == 40


def test_block_lrfu_fp32_d64():
    w = _scaled(dtype="f32", head_dim=64, prefill_lens=(257, 640), n_layers=1)
    st = _gu().run_block_lockstep(w, 36)
    assert st.max_out_err <= 1e-5 and st.max_score_err <= 1e-5


@PATHS
def test_block_lrfu_strong_decay_and_tight_budget(path):
    """beta 0.05 and short half-lives make the region decay dominate; the
    budget leaves room for few unpinned blocks."""
    w = _scaled(beta=0.05, region_half_lives=(40.0, 20.0, 10.0, 5.0, 3.0), budget_frac=0.15,
                prefill_lens=(640, 900), attn_path=path)
    _gu().run_block_lockstep(w, 40)


@PATHS
def test_block_lrfu_edge_cases(path):
    """One-token prefill (its block is the tail), a prefill ending on a block
    boundary, and a budget that never binds."""
    w = _scaled(prefill_lens=(1, 16, 47), budget_frac=5.0, n_epochs=1, epoch_steps=0,
                structured=False, attn_path=path)
    st = _gu().run_block_lockstep(w, 40, readmit=False)
    assert st.steps == 40


@PATHS
def test_block_step_bitwise_equals_separate_calls(path):
    import torch
    from decode_kv_cache_gqa_amd import kvev
    w = _scaled(n_layers=3, prefill_lens=(800, 1300), attn_path=path)
    outs, states = [], []
    for fused in (True, False):
        ctx = kvev.context_for(w, max_steps=24)
        for b in range(w.batch):
            K, V = w.prefill_kv(b, device="cuda")
            ctx.prefill(b, K, V, w.region_labels(b))
            ctx.set_budget(b, w.block_budget(b))
        out = torch.empty((w.n_layers, w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
        o_all = []
        for t in range(1, 25):
            q, kn, vn = w.step_inputs(t, device="cuda")
            if fused:
                ctx.step(q, kn, vn, out)
            else:
                ctx.decode_step(q, kn, vn, out)
                ctx.evict()
            o_all.append(out.clone())
        ctx.sync()
        outs.append(torch.stack(o_all).cpu())
        states.append([ctx.block_state(b) for b in range(w.batch)] +
                      [(ctx.retained(b, h), *ctx.export_kv(b, h)) for b in range(w.batch)
                       for h in range(w.n_kv_heads)])
        ctx.close()
    assert torch.equal(outs[0], outs[1])
    for a, b in zip(states[0], states[1]):
        for x, y in zip(a, b):
            if isinstance(x, np.ndarray):
                np.testing.assert_array_equal(x, y)
            else:
                assert torch.equal(x.cpu(), y.cpu())


def test_readmit_rejects_resident_and_unknown_blocks():
    import torch
    from decode_kv_cache_gqa_amd import kvev
    w = _scaled(prefill_lens=(320,))
    ctx = kvev.context_for(w, max_steps=4)
    K, V = w.prefill_kv(0, device="cuda")
    ctx.prefill(0, K, V, w.region_labels(0))
    ctx.set_budget(0, w.block_budget(0))
    Kr = torch.zeros((w.n_layers, w.n_kv_heads, 16, w.head_dim), dtype=w.torch_dtype, device="cuda")
    with pytest.raises(kvev.KvevError):
        ctx.readmit(0, [3], Kr, Kr)                   # resident
    with pytest.raises(kvev.KvevError):
        ctx.readmit(0, [19], Kr, Kr)                  # the block being filled
    with pytest.raises(kvev.KvevError):
        ctx.set_budget(0, 1)                          # below the pinned blocks + 1
    ctx.sync()
    ctx.close()


def test_block_max_positions_sampled():
    """One sequence of 65,520 tokens (4,095 blocks, 20% budget of 819) stepped
    toward the mode's 65,536-position bound, 4 layers, oracle on the whole
    sequence."""
    w = synth.workload("lrfu64").scaled(n_layers=4, prefill_lens=(65520,))
    st = _gu().run_block_lockstep(w, 4, readmit=False, kv_every=4)
    assert st.steps == 4


@pytest.mark.parametrize("path,expect", [(0, "attn"), (1, "attn"), (2, "attn_whole")])
def test_attention_kernel_choice(path, expect):
    """attn_path picks the kernel the steady steps run (the launches name
    themselves when profiling): AUTO takes the split kernel below 224 (group,
    layer) pairs, WHOLE the whole-cache kernel over the block tables."""
    import torch
    from decode_kv_cache_gqa_amd import kvev
    w = _scaled(prefill_lens=(300, 517), attn_path=path)
    ctx = kvev.context_for(w, max_steps=6)
    for b in range(w.batch):
        K, V = w.prefill_kv(b, device="cuda")
        ctx.prefill(b, K, V, w.region_labels(b))
        ctx.set_budget(b, w.block_budget(b))
    out = torch.empty((w.n_layers, w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    ctx.step(*w.step_inputs(1, device="cuda"), out)  # the prefill eviction
    ctx.sync()
    ctx.profile(True)
    for t in range(2, 6):
        ctx.step(*w.step_inputs(t, device="cuda"), out)
    ctx.sync()
    ran = {k: ctx.profile_read(k)[1] for k in ("attn", "attn_whole", "merge")}
    ctx.close()
    other = "attn_whole" if expect == "attn" else "attn"
    assert ran[expect] == 4 and ran[other] == 0
    assert ran["merge"] == (4 if expect == "attn" else 0)
