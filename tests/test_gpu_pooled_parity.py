"""GPU parity of the sequence-pooled token mode (one utility and one retained
set per sequence, "What Matters ...", section 3.1 Eq.1) against the CPU
oracle, through the C ABI: the pooled post kernel (fused step) and the
per-sequence selection with the shared moves (separate evict call)."""
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


@pytest.mark.parametrize("fused", [False, True])
def test_pooled_llama_shape(fused):
    st = _gu().run_pooled_lockstep(_w(), 24, fused=fused)
    assert st.steps == 24


def test_pooled_batch_lazy_refresh():
    w = _w(n_layers=2, prefill_lens=(700, 513, 900), budget=120, refresh_interval=4,
           n_sink=0, n_recent=8)
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


def test_pooled_single_kv_head_and_cumulative():
    w = _w(n_layers=2, n_q_heads=8, n_kv_heads=1, prefill_lens=(600,), budget=90,
           policy="cumulative")
    _gu().run_pooled_lockstep(w, 12)
