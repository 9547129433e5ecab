"""Pins of the scorer variants and of the sequence-pooled mode of the oracle.

[InertiaKV] §5.1 and App. E define VNorm (each head's attention times the
mean-normalised l2 norm of the value states) and entropy weighting (one
per-layer scalar, the normalised entropy of the attention distribution), and
§3.1 Eq.1 the score pooled over every head.  Each test fixes a value by hand,
by a closed form, a library routine or a property the page states.
"""
import math

import numpy as np
import pytest
from scipy import stats

import oracle as orc


# --- primitives ---------------------------------------------------------------

def test_vnorm_weights_hand_example():
    V = np.array([[3.0, 4.0], [0.0, 1.0], [6.0, 8.0]])  # norms 5, 1, 10; mean 16/3
    np.testing.assert_allclose(orc.vnorm_weights(V), [15 / 16, 3 / 16, 30 / 16], rtol=1e-15)
    # a uniform scale of the values leaves the weights unchanged; they average to 1
    np.testing.assert_allclose(orc.vnorm_weights(7.5 * V), orc.vnorm_weights(V), rtol=1e-15)
    rng = np.random.default_rng(1)
    assert orc.vnorm_weights(rng.standard_normal((50, 16))).mean() == pytest.approx(1.0, rel=1e-14)
    np.testing.assert_array_equal(orc.vnorm_weights(np.zeros((4, 8))), np.ones(4))


def test_normalized_entropy_closed_forms():
    # binary entropy of 1/4 in bits is 2 - (3/4) log2 3
    h = orc.normalized_entropy(np.array([[0.25, 0.75]]))
    assert h[0] == pytest.approx(2 - 0.75 * math.log2(3), rel=1e-14)
    n = 37
    assert orc.normalized_entropy(np.full((1, n), 1.0 / n))[0] == pytest.approx(1.0, rel=1e-14)
    one_hot = np.zeros((1, n))
    one_hot[0, 5] = 1.0
    assert orc.normalized_entropy(one_hot)[0] == 0.0
    np.testing.assert_array_equal(orc.normalized_entropy(np.ones((3, 1))), np.ones(3))


def test_normalized_entropy_matches_library_routine():
    rng = np.random.default_rng(2)
    p = rng.random((5, 40)) ** 3
    p /= p.sum(axis=1, keepdims=True)
    ref = np.array([stats.entropy(row) for row in p]) / math.log(40)
    np.testing.assert_allclose(orc.normalized_entropy(p), ref, rtol=1e-13)


# --- scorers inside the per-KV-head step ----------------------------------------

def test_scorers_hand_example_through_a_step():
    """One layer, one head, d = 1: prefill key 0 / value 1, new key ln 3 /
    value 3, so the probabilities are (1/4, 3/4); alpha_new = 1 stores the
    observation itself."""
    h = 2 - 0.75 * math.log2(3)
    expect = {
        "attention": [0.25, 0.75],
        "vnorm": [0.125, 1.125],          # value norms 1, 3: weights 1/2, 3/2
        "entropy": [0.25 * h, 0.75 * h],
        "vnorm+entropy": [0.125 * h, 1.125 * h],
    }
    for scorer, want in expect.items():
        o = orc.TokenModeOracle(1, 1, 1, 1, budget=100, alpha_new=1.0, scorer=scorer)
        o.prefill(0, np.zeros((1, 1, 1, 1)), np.ones((1, 1, 1, 1)))
        q = np.ones((1, 1, 1, 1))
        kn = np.full((1, 1, 1, 1), math.log(3), dtype=np.float64)
        vn = np.full((1, 1, 1, 1), 3.0)
        o.decode_step(1, q, kn.astype(np.float32), vn, [0])
        # the inputs are stored as fp32, so ln 3 is rounded once (2e-8 relative)
        got = o.scores(0, 0)
        np.testing.assert_allclose(got, want, rtol=2e-7)


def _run(scorer, q_zero=False, v_equal=False, L=2, T=8, seed=21):
    rng = np.random.default_rng(seed)
    Hq, Hkv, d, n0 = 4, 2, 8, 20
    K = rng.standard_normal((L, Hkv, n0, d)).astype(np.float32)
    if v_equal:
        V = np.sign(rng.standard_normal((L, Hkv, n0, d))).astype(np.float32)
    else:
        V = rng.standard_normal((L, Hkv, n0, d)).astype(np.float32)
    o = orc.TokenModeOracle(L, Hq, Hkv, d, budget=12, alpha_new=0.3, scorer=scorer, n_recent=2)
    o.prefill(0, K, V)
    out = []
    for t in range(1, T + 1):
        q = rng.standard_normal((L, 1, Hq, d)).astype(np.float32)
        if q_zero:
            q[:] = 0
        kn = rng.standard_normal((L, 1, Hkv, d)).astype(np.float32)
        vn = (np.sign(rng.standard_normal((L, 1, Hkv, d))) if v_equal
              else rng.standard_normal((L, 1, Hkv, d))).astype(np.float32)
        o.decode_step(t, q, kn, vn, [0])
        o.evict()
        out.append([(o.positions(0, h), o.scores(0, h)) for h in range(Hkv)])
    return out


def _assert_runs_close(a, b, rtol):
    for sa, sb in zip(a, b):
        for (pa, ma), (pb, mb) in zip(sa, sb):
            np.testing.assert_array_equal(pa, pb)
            np.testing.assert_allclose(ma, mb, rtol=rtol)


def test_entropy_weight_is_one_for_uniform_attention():
    _assert_runs_close(_run("entropy", q_zero=True), _run("attention", q_zero=True), 1e-12)


def test_vnorm_weight_is_one_for_equal_value_norms():
    _assert_runs_close(_run("vnorm", v_equal=True), _run("attention", v_equal=True), 1e-12)


def test_scorers_change_the_scores_otherwise():
    a, v, e = _run("attention"), _run("vnorm"), _run("entropy")
    assert not np.allclose(a[0][0][1], v[0][0][1])
    assert not np.allclose(a[0][0][1], e[0][0][1])


def test_entropy_weight_keeps_the_order_within_one_layer():
    """[InertiaKV] §5.1: the per-layer scalar leaves the ordering among tokens
    unchanged, so one layer's first observation retains the same set."""
    for seed in range(4):
        a = _run("attention", L=1, T=1, seed=seed)
        e = _run("entropy", L=1, T=1, seed=seed)
        for (pa, ma), (pe, me) in zip(a[0], e[0]):
            np.testing.assert_array_equal(np.sort(pa), np.sort(pe))
            ratio = me[ma > 0] / ma[ma > 0]
            np.testing.assert_allclose(ratio, ratio[0], rtol=1e-12)
            assert 0 < ratio[0] <= 1


# --- the sequence-pooled mode ----------------------------------------------------

def test_pooled_hand_example():
    """Two query heads with one KV head each; head 0 puts (1/4, 3/4) on the
    two tokens and head 1 (3/4, 1/4): the pooled mean is (1/2, 1/2)."""
    h = 2 - 0.75 * math.log2(3)
    l3 = float(np.float32(math.log(3)))
    p1 = math.exp(l3) / (1 + math.exp(l3))
    expect = {
        "attention": [0.5, 0.5],
        # head 0's values 1, 3 (weights 1/2, 3/2); head 1's values 2, 2 (weights 1)
        "vnorm": [(0.5 * (1 - p1) + p1) / 2, (1.5 * p1 + (1 - p1)) / 2],
        "entropy": [0.5 * h, 0.5 * h],
    }
    for scorer, want in expect.items():
        o = orc.PooledTokenOracle(1, 2, 2, 1, budget=100, alpha_new=1.0, scorer=scorer)
        o.prefill(0, np.zeros((1, 2, 1, 1)), np.array([1.0, 2.0]).reshape(1, 2, 1, 1))
        q = np.array([1.0, -1.0]).reshape(1, 1, 2, 1)
        kn = np.full((1, 1, 2, 1), math.log(3))
        vn = np.array([3.0, 2.0]).reshape(1, 1, 2, 1)
        o.decode_step(1, q, kn, vn, [0])
        np.testing.assert_allclose(o.scores(0), want, rtol=2e-7)
    assert expect["vnorm"][0] == pytest.approx(0.4375, rel=1e-6)
    assert expect["vnorm"][1] == pytest.approx(0.6875, rel=1e-6)


@pytest.mark.parametrize("scorer", orc.SCORERS)
def test_pooled_with_one_kv_head_is_the_per_head_mode(scorer):
    """With one KV head the pooled mean is the group sum divided by Hq."""
    rng = np.random.default_rng(5)
    L, Hq, d, n0, T = 2, 3, 8, 16, 10
    K = rng.standard_normal((L, 1, n0, d)).astype(np.float32)
    V = rng.standard_normal((L, 1, n0, d)).astype(np.float32)
    kw = dict(budget=10, alpha_new=0.2, scorer=scorer, n_sink=1, n_recent=2, refresh_interval=3)
    a = orc.TokenModeOracle(L, Hq, 1, d, **kw)
    b = orc.PooledTokenOracle(L, Hq, 1, d, **kw)
    a.prefill(0, K, V)
    b.prefill(0, K, V)
    for t in range(1, T + 1):
        q = rng.standard_normal((L, 1, Hq, d)).astype(np.float32)
        kn = rng.standard_normal((L, 1, 1, d)).astype(np.float32)
        vn = rng.standard_normal((L, 1, 1, d)).astype(np.float32)
        oa = a.decode_step(t, q, kn, vn, [0])
        ob = b.decode_step(t, q, kn, vn, [0])
        a.evict()
        b.evict()
        np.testing.assert_array_equal(oa, ob)
        np.testing.assert_array_equal(a.positions(0, 0), b.positions(0))
        np.testing.assert_allclose(b.scores(0), a.scores(0, 0) / Hq, rtol=1e-12)


def test_pooled_holds_one_retained_set_for_every_head():
    rng = np.random.default_rng(6)
    L, Hq, Hkv, d, n0, T, B = 2, 4, 2, 8, 30, 12, 14
    K = rng.standard_normal((L, Hkv, n0, d)).astype(np.float32)
    V = rng.standard_normal((L, Hkv, n0, d)).astype(np.float32)
    o = orc.PooledTokenOracle(L, Hq, Hkv, d, budget=B, alpha_new=0.1, n_sink=2, n_recent=3)
    o.prefill(0, K, V)
    Kpos = {p: K[:, :, p].copy() for p in range(n0)}
    for t in range(1, T + 1):
        q = rng.standard_normal((L, 1, Hq, d)).astype(np.float32)
        kn = rng.standard_normal((L, 1, Hkv, d)).astype(np.float32)
        vn = rng.standard_normal((L, 1, Hkv, d)).astype(np.float32)
        Kpos[n0 + t - 1] = kn[:, 0].copy()
        o.decode_step(t, q, kn, vn, [0])
        o.evict()
        pos = o.positions(0)
        assert len(pos) == B and len(set(pos.tolist())) == B
        assert {0, 1} <= set(pos.tolist())
        newest = n0 + t - 1
        assert {newest, newest - 1, newest - 2} <= set(pos.tolist())
        st = o.seqs[0]
        for slot, p in enumerate(pos):
            np.testing.assert_array_equal(st.K[:, :, slot], Kpos[int(p)])
