"""GPU parity over each workload's whole specified run, at full size and in
the benchmark's launch configuration, against the CPU oracle (one oracle
object per sampled group, sequence or layer, stepped in threads).

* 32k / 10% (32 layers, 32 query over 8 KV heads, 32,768-token prefill,
  budget 3,277 with 4 sinks and 32 recent): every KV head, all 256 steps.
* 16 x 8k / 25%, lazy refresh every 8 steps and score-free: two and one
  (sequence, KV head) groups over all 512 steps.
* 64 sequences of 4k-16k tokens, paged LRFU with region decay and
  re-admission of each 32-step epoch's heavy blocks: the shortest sequence
  over all 1,024 steps (32 epochs), the median sequence over its first 256
  steps (8 epochs); re-admissions run in the followed sequences.
* 131k two-tier (205 full-precision and 819 INT2 windows per layer): layers
  0 and 31 over all 128 steps, through all four heavy-key epochs.

kvev_step runs beside kvev_decode_step + kvev_evict on the token workloads
and must equal them bit for bit every step; the separate calls are checked
against the oracle before and after the eviction."""
import numpy as np
import pytest

from conftest import gpu_available
from decode_kv_cache_gqa_amd import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _gu():
    import gpu_util
    return gpu_util


def test_llama8b_32k_full_run():
    w = synth.workload("llama8b_32k")
    st = _gu().run_token_lockstep(w, w.steps, twin=True, kv_every=64)
    assert st.steps == 256 and st.exact_selection_checks == 256 * 8
    assert st.near_tie_resyncs <= 8


def test_llama8b_32k_split_attention_full_size():
    """The split-K attention kernel (used for the first step's 32,769 slots,
    the scorer variants and per-sequence granularity) on every steady step
    of the same workload's first 16 steps."""
    w = synth.workload("llama8b_32k").scaled(attn_path=1)
    st = _gu().run_token_lockstep(w, 16, twin=True, kv_every=8, ctx_steps=w.steps)
    assert st.steps == 16


def test_lazy16x8k_full_run():
    w = synth.workload("lazy16x8k")
    st = _gu().run_token_lockstep(w, w.steps, sample_seqs=[0, 15], sample_heads=[0, 7], twin=True,
                                  kv_every=128)
    assert st.steps == 512 and st.near_tie_resyncs <= 8


def test_scorefree16x8k_full_run():
    w = synth.workload("scorefree16x8k")
    st = _gu().run_token_lockstep(w, w.steps, sample_seqs=[7], sample_heads=[3], twin=True,
                                  kv_every=128)
    assert st.steps == 512 and st.near_tie_resyncs <= 8


def test_lrfu64_full_run():
    w = synth.workload("lrfu64")
    lens = np.asarray(w.prefill_lens)
    short = int(lens.argmin())
    median = int(np.argsort(lens, kind="stable")[len(lens) // 2])
    st = _gu().run_block_lockstep(w, w.steps, sample_seqs=[short, median], follow_steps={median: 256},
                                  kv_every=128, readmit_all=False)
    assert st.steps == 1024 and st.readmitted > 0
    assert st.checked_seq_steps + st.near_tie_resyncs == 1024 + 256


def test_qevict131k_full_run():
    w = synth.workload("qevict131k")
    st = _gu().run_tier_lockstep(w, w.steps, sample_layers=[0, 31], kv_every=32, ledger_every=32)
    assert st.steps == 128 and st.routing_events == 128 and st.ledger_checks > 0


def test_qevict65k_w8_rope_full_run():
    """The review's defaults at full size: 65,536-token prefill in 8,192
    windows of 8 per layer, rotary keys and queries, routing every 8 steps,
    byte-budget capacities (245 full-precision and 2,038 INT2 windows), 128
    steps over 4 heavy-key epochs; the oracle holds layers 0 and 31."""
    w = synth.workload("qevict65k_w8_rope")
    st = _gu().run_tier_lockstep(w, w.steps, sample_layers=[0, 31], kv_every=32, ledger_every=32)
    assert st.steps == 128 and st.routing_events == 16 and st.ledger_checks > 0
