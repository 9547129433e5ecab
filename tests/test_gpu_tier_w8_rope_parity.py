"""GPU parity of the two-tier window path with the review's own defaults
("QEvict" review, sections 4.2-4.4 and 5): 8-token windows, routing every 8
steps, and the rotary mode (keys quantized before the rotation and rotated
again at their original positions), against the CPU oracle through the C
ABI.  With 8-token windows or the rotary mode an INT2 window is attended
through its reconstruction rounded to bf16, which its full-precision
storage holds from its first demotion on."""
import pytest

from conftest import gpu_available
from decode_kv_cache_gqa_amd import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _gu():
    import gpu_util
    return gpu_util


def _scaled(**kw):
    base = dict(n_layers=2, n_q_heads=8, n_kv_heads=2, prefill_lens=(1500,), fp_windows=12,
                int2_windows=40, n_epochs=3, epoch_steps=16)
    base.update(kw)
    return synth.workload("qevict65k_w8_rope").scaled(**base)


def test_w8_rope_fused_steps():
    """188 windows of 8 (a ragged last one), routing every 8 steps over 3
    re-targeted heavy-key epochs: promotions, demotions on reused codes,
    evictions, with rotated keys and queries."""
    st = _gu().run_tier_lockstep(_scaled(), 48)
    assert st.steps == 48 and st.routing_events == 6 and st.ledger_checks > 0 and st.kv_checks > 0


def test_w8_rope_separate_calls():
    st = _gu().run_tier_lockstep(_scaled(prefill_lens=(1024,)), 40, fused=False)
    assert st.steps == 40 and st.routing_events == 5


def test_w8_without_rotation():
    """8-token windows alone (no rotary embedding), routing every step."""
    st = _gu().run_tier_lockstep(_scaled(rope_theta=0.0, route_interval=1, prefill_lens=(900,)), 32)
    assert st.steps == 32 and st.routing_events == 32


def test_w32_with_rotation():
    """32-token windows in the rotary mode (the bf16-reconstruction kernel
    at 32 tokens a window)."""
    w = _scaled(window_tokens=32, fp_windows=5, int2_windows=12, prefill_lens=(1500,))
    st = _gu().run_tier_lockstep(w, 40)
    assert st.steps == 40 and st.ledger_checks > 0


def test_w8_rope_llama_shape():
    """32 query over 8 KV heads, 4 layers, 1,000 windows of 8, sampled layers."""
    w = _scaled(n_layers=4, n_q_heads=32, n_kv_heads=8, prefill_lens=(8000,), fp_windows=40,
                int2_windows=300, epoch_steps=8, n_epochs=4)
    st = _gu().run_tier_lockstep(w, 32, sample_layers=[0, 3])
    assert st.steps == 32 and st.routing_events == 4


def test_w8_rope_max_windows_sampled():
    """A 98,290-token prefill stepped to near the mode's 12,288-window bound at 8
    tokens a window (the routing kernel's LDS bound), 2 layers; the oracle
    holds layer 1 through the first routing event and every step to the last
    position."""
    w = _scaled(prefill_lens=(98290,), fp_windows=300, int2_windows=2000)
    st = _gu().run_tier_lockstep(w, 4, sample_layers=[1], kv_every=4, ledger_every=4)
    assert st.steps == 4


@pytest.mark.parametrize("W,theta", [(32, 0.0), (8, 500000.0)])
def test_keys_grouped_per_token(W, theta):
    """int2_key_groups = 1: keys quantized per token and 32-channel group
    (the 131k workload's wording read for keys too), with 32-token windows
    and with the rotary 8-token mode: ledger records (key parameters [W,4]),
    bf16 reconstructions, tiers, scores and outputs in lockstep."""
    w = _scaled(n_layers=2, prefill_lens=(1200,), window_tokens=W, rope_theta=theta, int2_key_groups=1,
                fp_windows=5 if W == 32 else 20, int2_windows=12 if W == 32 else 48, route_interval=1)
    st = _gu().run_tier_lockstep(w, 24, ledger_every=4)
    assert st.steps == 24 and st.ledger_checks > 0
