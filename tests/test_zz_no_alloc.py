"""The allocation-free missed-mass entry point (kvev_diag_fmm_noalloc)
against kvev_diag_fmm on the same contexts: bit-identical results on two
calls in a row, the second on contexts with fewer groups."""
import numpy as np
import pytest

from conftest import gpu_available
from decode_kv_cache_gqa_amd import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _pair(w, steps):
    import torch
    from decode_kv_cache_gqa_amd import kvev
    mt = max(w.prefill_lens) + steps + 1
    comp = kvev.context_for(w, max_steps=steps, diag_topk=w.budget)
    full = kvev.context_for(w, max_steps=steps, budget=mt, diag_topk=1)
    for b in range(w.batch):
        K, V = w.prefill_kv(b, device="cuda")
        comp.prefill(b, K.contiguous(), V.contiguous())
        full.prefill(b, K.contiguous(), V.contiguous())
    out = torch.empty((w.n_layers, w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    for t in range(1, steps + 1):
        q, kn, vn = w.step_inputs(t, device="cuda")
        comp.step(q, kn, vn, out, w.budget)
        full.step(q, kn, vn, out, 0)
    return full, comp


def test_fmm_noalloc_matches_allocating_call():
    from decode_kv_cache_gqa_amd import kvev
    big = synth.workload("llama8b_32k").scaled(n_layers=2, prefill_lens=(900, 1300), budget=150)
    small = synth.workload("llama8b_32k").scaled(n_layers=2, n_q_heads=8, n_kv_heads=2,
                                                 prefill_lens=(700,), budget=100)
    for w, steps in ((big, 6), (small, 4)):
        full, comp = _pair(w, steps)
        want = kvev.diag_fmm(full, comp)
        got = kvev.diag_fmm_noalloc(full, comp)
        assert got.shape == (w.batch * w.n_kv_heads,)
        np.testing.assert_array_equal(got, want)
        assert np.all((got >= 0.0) & (got <= 1.0)) and np.any(got > 0.0)
        full.sync()
        comp.sync()
        full.close()
        comp.close()
