"""The seeded generator: determinism, independence of slices, recipe shape."""
import numpy as np
import torch

from decode_kv_cache_gqa_amd import synth


def test_slices_regenerate_independently():
    w = synth.workload("llama8b_32k").scaled(n_layers=3, prefill_lens=(700,))
    K, V = w.prefill_kv(0)
    K1, V1 = w.prefill_kv(0, layers=[2], heads=[5])
    assert torch.equal(K[2, 5], K1[0, 0]) and torch.equal(V[2, 5], V1[0, 0])
    q, k, v = w.step_inputs(7)
    q2, k2, v2 = w.step_inputs(7)
    assert torch.equal(q, q2) and torch.equal(k, k2) and torch.equal(v, v2)
    q3, _, _ = w.step_inputs(8)
    assert not torch.equal(q, q3)


def test_recipe_structure():
    w = synth.workload("llama8b_32k").scaled(n_layers=1, prefill_lens=(4096,))
    K, V = w.prefill_kv(0, heads=[0])
    Kf = K[0, 0].float()
    ck, cq = w._structure(0, 0, 0)
    assert (ck == 8).sum() == 4 and (cq == 8).sum() == 4
    pos = w.heavy_positions(0, 0, 0, 0)
    assert len(pos) == 64 and len(set(pos.tolist())) == 64 and pos.min() >= 4
    u, wv = w._directions(0, 0, 0, 0)
    assert abs(float(u @ wv)) == 0.0 and abs(float(u @ u) - 1) < 1e-6
    cos = (Kf[pos] @ torch.from_numpy(u)) / Kf[pos].norm(dim=1)
    assert torch.allclose(cos, torch.full_like(cos, 0.6), atol=1e-2)
    normal = np.setdiff1d(np.arange(4096), pos)
    col_std = Kf[normal].std(0)
    assert torch.all(col_std[torch.from_numpy(ck == 8)] > 6)
    assert abs(float(V.float().std()) - 1.0) < 0.02


def test_lengths_and_workload_table():
    w = synth.workload("lrfu64")
    assert w.batch == 64 and min(w.prefill_lens) >= 4096 and max(w.prefill_lens) <= 16384
    assert synth.workload("tiny").dtype == "f32"
    for name in synth.WORKLOADS:
        synth.workload(name)


def test_outlier_channels_shared_by_q_and_k():
    """The literal reading of the 32k workload's outlier wording: the same 4
    channels scaled in Q and K.  The logit spread then grows about five
    times (the outlier products add up coherently), against independent
    channel sets."""
    base = synth.workload("llama8b_32k").scaled(n_layers=1, prefill_lens=(4096,))
    shared = base.scaled(outlier_shared_qk=True)
    for w, same in ((base, False), (shared, True)):
        ck, cq = w._structure(0, 0, 0)
        assert (set(np.flatnonzero(ck == 8)) == set(np.flatnonzero(cq == 8))) == same
        ck2, cq2 = w._structure_many(np.array([0]), np.array([0]), np.array([0]))
        assert np.array_equal(ck2[0], ck) and np.array_equal(cq2[0], cq)
    std = []
    for w in (base, shared):
        K, _ = w.prefill_kv(0, heads=[0])
        q, _, _ = w.step_inputs(1)
        s = (q[0, 0, 0].float() @ K[0, 0].float().T) / np.sqrt(128.0)
        std.append(float(s.std()))
    assert 3.0 < std[1] / std[0] < 8.0
