"""Pins of the oracle's rank-trace diagnostics and future missed mass.

[InertiaKV] App. I, Table 13 defines the rank-trace statistics (raw and EMA
top-k churn, raw / EMA Jaccard overlap, the share of the raw top-k that is
evicted); [QEvict] §3 defines selection churn (the Jaccard distance between
consecutive retained sets) and Future Missed Mass (the share of the full
cache's attention landing on tokens already discarded).  Each test fixes a
value by hand, by brute force, by a closed form or by a special case that
reduces one statistic to another.
"""
import numpy as np
import pytest

import oracle as orc


# --- primitives ---------------------------------------------------------------

def test_jaccard_hand_values():
    assert orc.jaccard({1, 2, 3}, {2, 3, 4}) == 0.5
    assert orc.jaccard({1, 2}, {3}) == 0.0
    assert orc.jaccard({5, 6}, {6, 5}) == 1.0
    assert orc.jaccard(set(), set()) == 1.0
    assert orc.jaccard({1}, set()) == 0.0
    assert orc.jaccard(range(10), range(5, 15)) == 5 / 15


def test_top_k_positions_brute_force():
    """Against a sort of (value, position) pairs written out, values drawn
    from a small set so that ties are common; larger position wins a tie."""
    rng = np.random.default_rng(7)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        vals = rng.integers(0, 4, n).astype(np.float64) * 0.25
        pos = rng.permutation(1000)[:n]
        k = int(rng.integers(0, n + 3))
        pairs = sorted(zip(vals.tolist(), pos.tolist()), reverse=True)
        want = {p for _, p in pairs[:k]}
        assert orc.top_k_positions(vals, pos, k) == want, trial
    assert orc.top_k_positions([1.0, 1.0, 1.0], [5, 7, 6], 2) == {7, 6}
    assert orc.top_k_positions([3.0, 1.0, 2.0], [0, 1, 2], 10) == {0, 1, 2}


# --- rank-trace statistics ------------------------------------------------------

def test_rank_trace_hand_example():
    """Two steps worked out by hand with k = 2.

    Step 1: tokens 0..3, raw (4, 3, 2, 1), util (1, 2, 3, 4), token 0 evicted.
      R = {0, 1}, E = {3, 2}, J(R, E) = 0, R & Ev = {0}: share 1/2.
    Step 2: tokens 1..4, raw (1, 2, 3, 4), util (4, 3, 2, 1), token 3 evicted.
      R = {4, 3}, E = {1, 2}; raw churn 1 - 0/4 = 1; util churn
      1 - |{1,2} & {3,2}| / |{1,2,3}| = 2/3; R & Ev = {3}: share 1/2;
      selection churn 1 - |{1,2,4} & {1,2,3}| / |{1,2,3,4}| = 1/2.
    """
    d = orc.RankTraceDiagnostics(2)
    c1 = d.observe([0, 1, 2, 3], [4, 3, 2, 1], [1, 2, 3, 4], [1, 2, 3])
    assert c1 == {"n": 4, "k": 2, "raw_overlap": 0, "raw_prev": 0, "util_overlap": 0, "util_prev": 0,
                  "raw_util_overlap": 0, "raw_top_evicted": 1, "evicted": 1, "retained": 3,
                  "retained_overlap": 0, "retained_prev": 0}
    c2 = d.observe([1, 2, 3, 4], [1, 2, 3, 4], [4, 3, 2, 1], [1, 2, 4])
    assert c2 == {"n": 4, "k": 2, "raw_overlap": 0, "raw_prev": 2, "util_overlap": 1, "util_prev": 2,
                  "raw_util_overlap": 0, "raw_top_evicted": 1, "evicted": 1, "retained": 3,
                  "retained_overlap": 2, "retained_prev": 3}
    s = d.sums
    assert (s["steps"], s["pairs"]) == (2, 1)
    assert s["sum_raw_churn"] == 1.0
    assert s["sum_util_churn"] == pytest.approx(2 / 3, abs=1e-15)
    assert s["sum_raw_util_jaccard"] == 0.0
    assert s["sum_raw_top_evicted"] == 1.0
    assert s["sum_selection_churn"] == 0.5
    assert d.evicted_at == {0: 1, 3: 2}
    assert d.evicted_before(2) == {0} and d.evicted_before(3) == {0, 3}


def _small_oracle(alpha_new=0.05, n_layers=2, budget=12, n_sink=0, n_recent=0):
    return orc.TokenModeOracle(n_layers, 4, 1, 8, budget=budget, alpha_new=alpha_new,
                               n_sink=n_sink, n_recent=n_recent, capacity=64)


def _run(o, steps, seed, q_scale=1.0, n0=20, track=None, full=None):
    """Prefill n0 tokens, then step; returns per-step (counts, observation)."""
    rng = np.random.default_rng(seed)
    L, d = o.n_layers, o.head_dim
    K = rng.standard_normal((L, 1, n0, d))
    V = rng.standard_normal((L, 1, n0, d))
    o.prefill(0, K, V)
    if full is not None:
        full.prefill(0, K, V)
    out = []
    for t in range(1, steps + 1):
        q = q_scale * rng.standard_normal((L, 1, 4, d))
        kn = rng.standard_normal((L, 1, 1, d))
        vn = rng.standard_normal((L, 1, 1, d))
        o.decode_step(t, q, kn, vn, [0])
        obs = o.step_observation(0, 0)
        fobs = None
        if full is not None:
            full.decode_step(t, q, kn, vn, [0])
            fobs = full.step_observation(0, 0)
        o.evict()
        c = track.observe(*obs, o.positions(0, 0)) if track is not None else None
        out.append((c, obs, fobs))
    return out


def test_raw_observation_sums_to_layers_times_group():
    """Each head's probabilities sum to one, so the layer-summed group mass of
    a step sums to L * group size over the tokens (a dropped layer or head
    breaks it)."""
    o = _small_oracle(n_layers=3)
    for _, (pos, raw, util), _ in _run(o, 5, seed=3):
        assert raw.sum() == pytest.approx(3 * 4, rel=1e-12)
        assert (raw > 0).all()


def test_alpha_one_single_layer_reduces_util_to_raw():
    """With one layer and the whole weight on the new observation, every
    token's utility is its raw observation, so the two top-k sets coincide:
    Jaccard 1 and equal raw and utility churn at every step."""
    o = _small_oracle(alpha_new=1.0, n_layers=1)
    tr = orc.RankTraceDiagnostics(5)
    for c, (pos, raw, util), _ in _run(o, 8, seed=4, track=tr):
        np.testing.assert_array_equal(raw, util)
        assert c["raw_util_overlap"] == c["k"] == 5
        assert c["raw_overlap"] == c["util_overlap"]
    s = tr.sums
    assert s["sum_raw_util_jaccard"] == s["steps"] == 8
    assert s["sum_raw_churn"] == s["sum_util_churn"]


def test_selection_churn_closed_form_single_token_evictions():
    """After the first step (which evicts the prefill down to B), one token
    leaves per step: the retained sets of consecutive steps share B - 1
    tokens out of B + 1, a churn of 2 / (B + 1), or share all B (churn 0)
    when the evicted token is the new one itself."""
    B = 12
    o = _small_oracle(budget=B)
    tr = orc.RankTraceDiagnostics(B)
    res = _run(o, 10, seed=5, track=tr)
    want = 0.0
    for t, (c, (pos, raw, util), _) in enumerate(res, start=1):
        assert c["retained"] == B
        if t == 1:
            assert c["evicted"] == 21 - B
            continue
        newest = 20 + t - 1
        assert int(pos.max()) == newest and c["evicted"] == 1
        if tr.evicted_at.get(newest) == t:
            assert c["retained_overlap"] == B
        else:
            assert c["retained_overlap"] == B - 1
            want += 2 / (B + 1)
    assert tr.sums["sum_selection_churn"] == pytest.approx(want, abs=1e-14)


def test_util_top_budget_equals_kept_set_every_step():
    """With no protected tokens the selection keeps the top-B utilities, so
    the utility top-k at k = B is the kept set (a swapped order or tie rule
    in either breaks it)."""
    B = 12
    o = _small_oracle(budget=B)
    rng_steps = 9
    rng = np.random.default_rng(6)
    L, d = o.n_layers, o.head_dim
    o.prefill(0, rng.standard_normal((L, 1, 20, d)), rng.standard_normal((L, 1, 20, d)))
    for t in range(1, rng_steps + 1):
        o.decode_step(t, rng.standard_normal((L, 1, 4, d)), rng.standard_normal((L, 1, 1, d)),
                      rng.standard_normal((L, 1, 1, d)), [0])
        pos, raw, util = o.step_observation(0, 0)
        o.evict()
        kept = set(o.positions(0, 0).tolist())
        assert orc.top_k_positions(util, pos, B) == kept, t


# --- future missed mass ---------------------------------------------------------

def test_fmm_uniform_attention_closed_form():
    """A zero query attends uniformly, so the full cache's mass on any token
    is 1/n and the missed mass is (tokens evicted before the step) / n."""
    B = 8
    o = _small_oracle(budget=B)
    full = _small_oracle(budget=10 ** 6)
    tr = orc.RankTraceDiagnostics(B)
    res = _run(o, 9, seed=8, q_scale=0.0, full=full, track=tr)
    for t, (c, _, (fpos, fraw, futil)) in enumerate(res, start=1):
        ev = tr.evicted_before(t)
        n = fpos.shape[0]
        assert n == 20 + t
        np.testing.assert_allclose(fraw, np.full(n, 2 * 4 / n), rtol=1e-13)
        assert orc.future_missed_mass(fpos, fraw, ev) == pytest.approx(len(ev) / n, rel=1e-13)
    # step 1 evicts the prefill down to the budget (13 tokens); later steps one each
    assert len(tr.evicted_before(2)) == 21 - B


def test_fmm_zero_without_eviction_and_one_on_everything():
    full = _small_oracle(budget=10 ** 6)
    res = _run(full, 4, seed=9)
    pos, raw, _ = res[-1][1]
    assert orc.future_missed_mass(pos, raw, set()) == 0.0
    assert orc.future_missed_mass(pos, raw, set(pos.tolist())) == pytest.approx(1.0, rel=1e-15)
    # the missed mass of a set is the mass on those positions over the total
    sub = set(pos[::3].tolist())
    want = raw[np.isin(pos, list(sub))].sum() / raw.sum()
    assert orc.future_missed_mass(pos, raw, sub) == pytest.approx(want, rel=1e-14)


def test_fmm_counts_only_earlier_evictions():
    """A position evicted at step t is not missed at step t (the step's
    attention still saw it), only from step t + 1 on."""
    B = 8
    o = _small_oracle(budget=B)
    full = _small_oracle(budget=10 ** 6)
    tr = orc.RankTraceDiagnostics(B)
    res = _run(o, 4, seed=10, full=full, track=tr)
    assert tr.evicted_before(1) == set()
    just = {p for p, e in tr.evicted_at.items() if e == 4}
    assert just and not (just & tr.evicted_before(4))
    assert just <= tr.evicted_before(5)
