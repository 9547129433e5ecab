"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test ties an oracle function to a printed worked example, a closed form
stated on a page, a theorem, a library routine or brute force, so that a
dropped term, a wrong sign or a transposed operand fails here.
"""
import itertools
import math
import os
from decimal import Decimal, ROUND_HALF_UP

import numpy as np
import pytest

import oracle as orc


def _read_table(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# --- EMA ([LRFU-fig] worked table; [InertiaKV] §5.3 unrolled form) --------

def test_ema_table_reproduced_with_page_rounding(golden_dir):
    """The printed column is a 3-decimal round-half-up chain fed forward."""
    rows = _read_table(os.path.join(golden_dir, "lrfu_ema_table.txt"))
    a = Decimal("0.05")
    score = Decimal("0.000")
    for _, new, printed in rows:
        score = orc.ema_update(score, Decimal(new), a)
        score = score.quantize(Decimal("0.001"), rounding=ROUND_HALF_UP)
        assert score == Decimal(printed)


def test_ema_exact_chain_matches_unrolled_closed_form_and_page(golden_dir):
    rows = _read_table(os.path.join(golden_dir, "lrfu_ema_table.txt"))
    xs = [float(r[1]) for r in rows]
    printed = [float(r[2]) for r in rows]
    a = 0.05
    m = 0.0
    for T, (x, pr) in enumerate(zip(xs, printed), start=1):
        m = orc.ema_update(m, x, a)
        # [InertiaKV] §5.3: mu_T = (1-alpha) sum alpha^{T-tau} s_tau + alpha^T mu_0
        # with alpha (on the old state) = 1 - a and mu_0 = 0.
        closed = sum(a * (1 - a) ** (T - tau) * xs[tau - 1] for tau in range(1, T + 1))
        assert abs(m - closed) < 1e-15
        assert abs(m - pr) <= 1.1e-3
    assert abs(m - 0.05830814) < 1e-8
    assert abs(sum(xs) / len(xs) - 0.26) < 1e-12        # "raw average of 0.26"


def test_half_life_and_beta_timescale():
    assert round(orc.ema_half_life(0.05), 1) == 13.5
    # The EMA weight of one observation halves between 13 and 14 steps.
    w = 1.0
    steps = 0
    while w > 0.5:
        w = orc.ema_update(w, 0.0, 0.05)
        steps += 1
    assert steps == 14 and orc.ema_half_life(0.05) < 14
    beta = 0.001
    assert 1 / beta == 1000
    assert round(float(orc.recency_decay(1000, beta)), 2) == 0.63   # "~63% at 1,000 steps"
    assert round(float(orc.recency_decay(2000, beta)), 3) == 0.865  # "0.865"
    assert round(float(orc.recency_decay(50, beta)), 3) == 0.049    # block A "0.049"


def test_priority_examples(golden_dir):
    rows = _read_table(os.path.join(golden_dir, "lrfu_priority_examples.txt"))
    beta = 0.001
    for _, score, idle, printed, tol in rows:
        p = float(orc.lrfu_priority(float(score), float(idle), beta))
        assert abs(p - float(printed)) <= float(tol), (score, idle, p)
    # block A is kept, block B is evicted: B has the higher priority
    pa = orc.lrfu_priority(0.059, 50, beta)
    pb = orc.lrfu_priority(0.02, 2000, beta)
    assert pb > pa
    # the formula is monotone: higher score lowers priority, idleness raises it
    assert orc.lrfu_priority(0.5, 100, beta) < orc.lrfu_priority(0.4, 100, beta)
    assert orc.lrfu_priority(0.5, 100, beta) < orc.lrfu_priority(0.5, 200, beta)
    # beta -> 0 drives the recency factor, hence the priority, to zero
    assert float(orc.lrfu_priority(0.3, 5000, 1e-12)) < 1e-8


def test_region_rates_from_half_lives():
    lam = orc.region_decay_rates([170, 100, 60, 30, 15])
    for h, l in zip([170, 100, 60, 30, 15], lam):
        assert abs(math.exp(-l * h) - 0.5) < 1e-15        # [MemDecay] Eq.7


# --- layer-sequential fold ([InertiaKV] App. E) -----------------------------

def test_layer_fold_closed_form_weights():
    rng = np.random.default_rng(0)
    L, n, a = 32, 50, 0.05
    m0 = rng.random(n)
    G = rng.random((L, n))
    seq = orc.layer_fold(m0, G, a)
    prior, w = orc.layer_fold_weights(a, L)
    closed = prior * m0 + sum(w[l] * G[l] for l in range(L))
    np.testing.assert_allclose(seq, closed, rtol=1e-13)
    assert abs(prior - 0.95 ** 32) < 1e-15
    assert abs(prior + sum(w) - 1.0) < 1e-14       # weights of a convex average
    # layer 31 (last) carries the largest weight a, layer 0 the smallest
    assert w[-1] == a and w[0] < w[1]


def test_layer_fold_alpha_one_keeps_only_last_layer():
    """[InertiaKV] §5.1: the alpha = 0 endpoint (alpha_new = 1) retains only
    the last processed layer."""
    rng = np.random.default_rng(1)
    G = rng.random((4, 10))
    np.testing.assert_array_equal(orc.layer_fold(rng.random(10), G, 1.0), G[-1])


def test_cumulative_fold_is_running_sum():
    rng = np.random.default_rng(2)
    G = rng.random((6, 9))
    m = orc.layer_fold(np.zeros(9), G, None, policy="cumulative")
    np.testing.assert_allclose(m, G.sum(axis=0), rtol=1e-15)


# --- attention --------------------------------------------------------------

def test_attention_matches_library_routines():
    torch = pytest.importorskip("torch")
    from scipy.special import softmax
    rng = np.random.default_rng(3)
    H, n, d = 4, 37, 16
    q = rng.standard_normal((H, d))
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    out, p, s = orc.decode_attention(q, K, V)
    np.testing.assert_allclose(p, softmax(q @ K.T / math.sqrt(d), axis=1), rtol=1e-13)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, :, None, :],
        torch.tensor(K)[None, None].expand(1, H, n, d),
        torch.tensor(V)[None, None].expand(1, H, n, d))
    np.testing.assert_allclose(out, ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-14)
    G = orc.group_mass(p)
    assert abs(G.sum() - H) < 1e-12
    # a single-head group: the group mass is that head's softmax row
    np.testing.assert_array_equal(orc.group_mass(p[1:2]), p[1])


def test_attention_is_shift_invariant_and_uses_sqrt_d():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((2, 8))
    K = rng.standard_normal((5, 8))
    V = rng.standard_normal((5, 8))
    _, p, s = orc.decode_attention(q, K, V)
    # logits are q.k / sqrt(d), written out per element
    for h in range(2):
        for i in range(5):
            assert abs(s[h, i] - sum(q[h, c] * K[i, c] for c in range(8)) / math.sqrt(8)) < 1e-12
    # one key identical to the query direction scaled up dominates
    K2 = K.copy()
    K2[3] = 50 * q[0]
    _, p2, _ = orc.decode_attention(q[:1], K2, V)
    assert p2[0, 3] > 0.999


# --- selection ([MemDecay] Eq.1 optimality) and compaction ------------------

def test_selection_matches_subset_enumeration():
    rng = np.random.default_rng(5)
    for trial in range(40):
        n = int(rng.integers(3, 12))
        B = int(rng.integers(1, n))
        scores = rng.random(n)
        pos = rng.permutation(n)
        n_sink = int(rng.integers(0, 2))
        n_recent = int(rng.integers(0, 2))
        newest = pos.max()
        forced = {i for i in range(n) if pos[i] < n_sink or pos[i] > newest - n_recent}
        if len(forced) > B:
            continue
        best, best_set = -1.0, None
        for sub in itertools.combinations(range(n), B):
            if not forced <= set(sub):
                continue
            val = scores[list(sub)].sum()
            if val > best:
                best, best_set = val, set(sub)
        keep = orc.select_keep(scores, pos, B, n_sink, n_recent)
        assert set(np.flatnonzero(keep)) == best_set
        assert keep.sum() == B


def test_selection_tie_rule_and_no_op():
    scores = np.array([0.5, 0.2, 0.2, 0.2, 0.9])
    pos = np.array([0, 1, 2, 3, 4])
    keep = orc.select_keep(scores, pos, 3)
    # ties at 0.2: the more recent position (3) is kept
    assert list(np.flatnonzero(keep)) == [0, 3, 4]
    assert orc.select_keep(scores, pos, 5).all()
    assert orc.select_keep(scores, pos, 7).all()
    with pytest.raises(ValueError):
        orc.select_keep(scores, pos, 2, n_sink=2, n_recent=2)


def test_hole_fill_preserves_kept_multiset():
    rng = np.random.default_rng(6)
    for _ in range(50):
        n = int(rng.integers(2, 40))
        B = int(rng.integers(1, n + 1))
        keep = np.zeros(n, bool)
        keep[rng.choice(n, size=min(B, n), replace=False)] = True
        if n <= B:
            assert orc.hole_fill_moves(keep, B) == []
            continue
        moves = orc.hole_fill_moves(keep, B)
        payload = np.arange(n) * 10
        after = orc.apply_moves(payload.copy(), moves)[:B]
        assert sorted(after.tolist()) == sorted(payload[keep].tolist())
        assert len(moves) == int((~keep[:B]).sum())
        assert all(s >= B and d < B for s, d in moves)


# --- Proposition 1 and Corollary 2 ([InertiaKV] §5.3) -----------------------

def test_proposition1_variance_bound_monte_carlo():
    rng = np.random.default_rng(7)
    alpha_old = 0.8
    a = 1 - alpha_old
    sigma = 0.3
    T, trials = 200, 20000
    mu_i = np.zeros(trials)
    mu_j = np.zeros(trials)
    for _ in range(T):
        mu_i = orc.ema_update(mu_i, 0.6 + sigma * rng.standard_normal(trials), a)
        mu_j = orc.ema_update(mu_j, 0.5 + sigma * rng.standard_normal(trials), a)
    bound = 2 * (1 - alpha_old) / (1 + alpha_old) * sigma ** 2
    var = np.var(mu_i - mu_j)
    assert var <= bound * 1.05
    assert abs(var - bound) / bound < 0.05          # i.i.d. Gaussian attains it
    assert abs(np.mean(mu_i - mu_j) - 0.1) < 0.01   # expected gap -> delta


def test_corollary2_power_of_two_scaling_keeps_retained_sets():
    rng = np.random.default_rng(8)
    n, B, L = 60, 20, 4
    m1 = np.zeros(n)
    m2 = np.zeros(n)
    pos = np.arange(n)
    for step in range(10):
        G = rng.random((L, n)) ** 4
        m1 = orc.layer_fold(m1, G, 0.05)
        m2 = orc.layer_fold(m2, G * 2.0 ** -7, 0.05)
        k1 = orc.select_keep(m1, pos, B, 2, 3)
        k2 = orc.select_keep(m2, pos, B, 2, 3)
        assert (k1 == k2).all()
        np.testing.assert_array_equal(m1 * 2.0 ** -7, m2)


# --- token-mode step oracle: special cases ----------------------------------

def _small_run(**kw):
    rng = np.random.default_rng(11)
    L, Hq, Hkv, d, n0, T = 2, 4, 2, 8, 24, 12
    K = rng.standard_normal((L, Hkv, n0, d)).astype(np.float32)
    V = rng.standard_normal((L, Hkv, n0, d)).astype(np.float32)
    steps = [(rng.standard_normal((L, 1, Hq, d)).astype(np.float32),
              rng.standard_normal((L, 1, Hkv, d)).astype(np.float32),
              rng.standard_normal((L, 1, Hkv, d)).astype(np.float32)) for _ in range(T)]
    o = orc.TokenModeOracle(L, Hq, Hkv, d, budget=10, alpha_new=kw.pop("alpha_new", 0.05), **kw)
    o.prefill(0, K, V)
    trace = []
    for t, (q, kn, vn) in enumerate(steps, start=1):
        out = o.decode_step(t, q, kn, vn, [0])
        o.evict()
        trace.append((out, [o.positions(0, h) for h in range(Hkv)],
                      [o.scores(0, h) for h in range(Hkv)]))
    return trace


def _same(t1, t2):
    for (o1, p1, s1), (o2, p2, s2) in zip(t1, t2):
        np.testing.assert_array_equal(o1, o2)
        for a, b in zip(p1, p2):
            np.testing.assert_array_equal(a, b)
        for a, b in zip(s1, s2):
            np.testing.assert_array_equal(a, b)


def test_lazy_r1_is_full_refresh():
    _same(_small_run(refresh_interval=1), _small_run())


def test_lazy_beyond_run_is_score_free():
    _same(_small_run(refresh_interval=1000), _small_run(score_free=True))


def test_budget_is_held_and_protection_respected():
    tr = _small_run(n_sink=2, n_recent=3)
    for t, (_, pos, _) in enumerate(tr, start=1):
        for p in pos:
            assert len(p) == 10
            assert {0, 1} <= set(p.tolist())
            newest = 24 + t - 1
            assert {newest, newest - 1, newest - 2} <= set(p.tolist())


def test_single_step_rule_keeps_top_budget_of_last_layer():
    """alpha_new = 1 is [InertiaKV] Eq.2 applied to the last layer."""
    rng = np.random.default_rng(12)
    L, Hq, Hkv, d, n0 = 3, 2, 1, 8, 30
    K = rng.standard_normal((L, Hkv, n0, d)).astype(np.float32)
    V = rng.standard_normal((L, Hkv, n0, d)).astype(np.float32)
    q = rng.standard_normal((L, 1, Hq, d)).astype(np.float32)
    kn = rng.standard_normal((L, 1, Hkv, d)).astype(np.float32)
    vn = rng.standard_normal((L, 1, Hkv, d)).astype(np.float32)
    o = orc.TokenModeOracle(L, Hq, Hkv, d, budget=8, alpha_new=1.0)
    o.prefill(0, K, V)
    o.decode_step(1, q, kn, vn, [0])
    G_last = o.last_G[(L - 1, 0, 0)]
    o.evict()
    Kfull = np.concatenate([K[L - 1, 0], kn[L - 1, 0]], axis=0)
    _, p, _ = orc.decode_attention(q[L - 1, 0], Kfull, Kfull)
    np.testing.assert_allclose(G_last, p.sum(axis=0), rtol=1e-14)
    top = set(np.argsort(p.sum(axis=0))[-8:].tolist())
    assert set(o.positions(0, 0).tolist()) == top


def test_new_token_mean_init_on_non_refresh_steps():
    rng = np.random.default_rng(13)
    L, Hq, Hkv, d, n0 = 1, 2, 1, 4, 6
    K = rng.standard_normal((L, Hkv, n0, d)).astype(np.float32)
    o = orc.TokenModeOracle(L, Hq, Hkv, d, budget=100, alpha_new=0.5, refresh_interval=3)
    o.prefill(0, K, K)
    mk = lambda: (rng.standard_normal((L, 1, Hq, d)).astype(np.float32),
                  rng.standard_normal((L, 1, Hkv, d)).astype(np.float32),
                  rng.standard_normal((L, 1, Hkv, d)).astype(np.float32))
    o.decode_step(1, *mk(), [0])           # refresh
    before = o.scores(0, 0)
    o.decode_step(2, *mk(), [0])           # not a refresh step
    after = o.scores(0, 0)
    np.testing.assert_array_equal(after[:-1], before)       # frozen
    assert after[-1] == before.mean()
    o.decode_step(4, *mk(), [0])           # t=4: (4-1) mod 3 == 0 -> refresh
    assert not np.array_equal(o.scores(0, 0)[:-1], after)


def _two_refresh_steps(**kw):
    rng = np.random.default_rng(14)
    L, Hq, Hkv, d, n0 = 3, 4, 1, 8, 20
    K = rng.standard_normal((L, Hkv, n0, d)).astype(np.float32)
    V = rng.standard_normal((L, Hkv, n0, d)).astype(np.float32)
    steps = [tuple(rng.standard_normal((L, 1, Hx, d)).astype(np.float32) for Hx in (Hq, Hkv, Hkv))
             for _ in range(2)]
    o = orc.TokenModeOracle(L, Hq, Hkv, d, budget=100, **kw)
    o.prefill(0, K, V)
    o.decode_step(1, *steps[0], [0])
    prior = o.scores(0, 0).copy()
    out = o.decode_step(2, *steps[1], [0])
    return prior, o.scores(0, 0), out


@pytest.mark.parametrize("policy,alpha", [("ema", 0.05), ("ema", 0.3), ("cumulative", 0.05)])
def test_new_token_mean_init_on_refresh_steps(policy, alpha):
    """new_token_init = "mean" (the App. E rule applied on refresh steps
    too): the new token starts at the mean of the group's utilities and is
    then folded, so against the zero start its utility moves by the prior's
    fold weight times that mean, (1 - a)^L for the EMA (Eq.4 unrolled over
    the L layers) and 1 for the running sum (Eq.3); nothing else changes."""
    p0, s0, o0 = _two_refresh_steps(policy=policy, alpha_new=alpha)
    p1, s1, o1 = _two_refresh_steps(policy=policy, alpha_new=alpha, new_token_init="mean")
    np.testing.assert_array_equal(p0, p1)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(s0[:-1], s1[:-1])
    w = 1.0 if policy == "cumulative" else (1.0 - alpha) ** 3
    assert abs((s1[-1] - s0[-1]) - w * p0.mean()) <= 1e-15
    assert p0.mean() > 0.0


def test_new_token_init_has_no_effect_with_the_single_step_rule():
    _, s0, _ = _two_refresh_steps(alpha_new=1.0)
    _, s1, _ = _two_refresh_steps(alpha_new=1.0, new_token_init="mean")
    np.testing.assert_array_equal(s0, s1)


# --- tiered routing and byte accounting -------------------------------------

def test_qevict_worked_example(golden_dir):
    g = {r[0]: float(r[1]) for r in _read_table(os.path.join(golden_dir, "qevict_worked_example.txt"))}
    Hkv, d, L = 8, 128, 32
    per_tok_layer = 2 * Hkv * d * 2
    assert per_tok_layer == g["bytes_per_token_layer"]
    assert per_tok_layer * L == g["bytes_per_token_all_layers"]
    m_f = 8 * per_tok_layer * L
    assert m_f == g["m_f_bytes_window8"]
    MB = 1024 * 1024
    k_f, k_q = orc.tier_capacities(100 * MB, 0.70, m_f, 0.131 * MB)
    assert (k_f, k_q) == (g["k_f"], g["k_q"])
    assert 8 * k_f == g["fp_tokens"] and 8 * k_q == g["int2_tokens"]
    assert round((8 * k_f + 8 * k_q) / (8 * k_f), 1) == g["coverage_ratio"]


def test_block_bytes_of_lrfu_figure():
    """"16 tokens = 5.00 mebibytes" is 80 layers x 8 KV heads x 128 x (K+V) x bf16."""
    per_token = 80 * 8 * 128 * 2 * 2
    assert per_token == 320 * 1024
    assert per_token * 16 / 2 ** 20 == 5.00


def test_route_tiers_state_machine():
    """F <-> Q, Q -> E, and E absorbing ([QEvict] §4.4 Eq.4-6)."""
    rng = np.random.default_rng(14)
    nw, k_f, k_q = 60, 5, 12
    S = np.zeros(nw)
    F, Q, E = [], [], set()
    aged = 0
    for event in range(40):
        new_aged = list(range(aged, min(aged + 4, nw)))
        aged = min(aged + 4, nw)
        inc = rng.random(aged) * (np.arange(aged) % 7 == event % 7) + 1e-3 * rng.random(aged)
        inc[list(E)] = 0.0               # evicted windows receive no mass
        S[:aged] += inc
        cand = set(F) | set(Q) | set(new_aged)
        F2, Q2, E2 = orc.route_tiers(S, cand, k_f, k_q)
        assert len(F2) == min(k_f, len(cand))
        assert len(Q2) <= k_q
        assert not (set(F2) | set(Q2)) & E
        assert min(S[F2]) >= max(S[Q2]) if F2 and Q2 else True
        E |= set(E2)
        F, Q = F2, Q2


def test_tier_routing_matches_full_sort():
    rng = np.random.default_rng(15)
    S = rng.random(30)
    F, Q, E = orc.route_tiers(S, range(30), 4, 9)
    order = np.argsort(-S)
    assert F == sorted(order[:4].tolist())
    assert Q == sorted(order[4:13].tolist())
    assert E == sorted(order[13:].tolist())


# --- INT2 quantizer -----------------------------------------------------------

def test_int2_grid_values_round_trip_exactly():
    zero = np.float16(-1.5)
    scale = np.float16(0.25)
    codes_true = np.array([[0, 1, 2, 3] * 8] * 4, dtype=np.uint8).T  # [32, 4]
    x = (codes_true.astype(np.float32) * np.float32(scale) + np.float32(zero)).astype(np.float32)
    codes, s, z = orc.int2_quantize(x, "channel")
    np.testing.assert_array_equal(codes, codes_true)
    np.testing.assert_array_equal(orc.int2_dequantize(codes, s, z, "channel"), x)


def test_int2_bounds_and_degenerate_groups():
    rng = np.random.default_rng(16)
    x = (rng.standard_normal((32, 128)) * 3).astype(np.float32)
    for mode in ("channel", "token32"):
        codes, s, z = orc.int2_quantize(x, mode)
        assert codes.max() <= 3
        xh = orc.int2_dequantize(codes, s, z, mode)
        if mode == "channel":
            sc = np.repeat(np.asarray(s, np.float32)[None], 32, 0)
            mn, mx = x.min(0), x.max(0)
            assert (codes[x.argmin(0), np.arange(128)] == 0).all()
            assert (codes[x.argmax(0), np.arange(128)] == 3).all()
        else:
            sc = np.repeat(np.asarray(s, np.float32), 32, 1)
        # half a step, plus the slop of fp16-rounded parameters
        assert (np.abs(x - xh) <= 0.5 * sc + 2e-3 * (np.abs(x) + sc) + 1e-6).all()
    const = np.full((32, 128), 0.7, np.float32)
    codes, s, z = orc.int2_quantize(const, "channel")
    assert (codes == 0).all() and (np.asarray(s) == 0).all()
    assert np.allclose(orc.int2_dequantize(codes, s, z, "channel"), np.float16(0.7))


def test_int2_requantizing_ledger_codes_is_stable():
    """Quantizing once and reusing codes is bit-stable across migrations."""
    rng = np.random.default_rng(17)
    x = rng.standard_normal((32, 64)).astype(np.float32)
    c1, s1, z1 = orc.int2_quantize(x, "token32")
    xh = orc.int2_dequantize(c1, s1, z1, "token32")
    xh2 = orc.int2_dequantize(c1, s1, z1, "token32")
    np.testing.assert_array_equal(xh, xh2)
