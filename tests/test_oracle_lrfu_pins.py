"""Pins of the block-granular LRFU oracle (priority, region decay, clock,
pinning, selection, persistence) against the pages, closed forms and brute
force.
"""
import itertools
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle as orc


def _read_table(path):
    with open(path) as f:
        return [ln.split() for ln in (x.strip() for x in f) if ln and not ln.startswith("#")]


# --- priority and survival ------------------------------------------------

def test_block_priority_without_region_decay_gives_figure_examples(golden_dir):
    """[LRFU-fig] worked priorities, through the block path (one region, lambda 0)."""
    rows = _read_table(os.path.join(golden_dir, "lrfu_priority_examples.txt"))
    for _, score, idle, printed, tol in rows:
        p = orc.block_priority(float(score), [0] * 16, int(idle), 0.001, [0.0])
        assert abs(p - float(printed)) <= float(tol)
    # exact values (C3): A 0.045893, B 0.847371
    assert abs(orc.block_priority(0.059, [0] * 16, 50, 0.001, [0.0]) - 0.0458926) < 1e-6
    assert abs(orc.block_priority(0.02, [0] * 16, 2000, 0.001, [0.0]) - 0.8473707) < 1e-6


def test_block_priority_reduces_to_lrfu_formula_when_regions_do_not_decay():
    rng = np.random.default_rng(3)
    for _ in range(200):
        s = rng.uniform(0, 1)
        idle = int(rng.integers(0, 6000))
        labels = rng.integers(0, 5, size=16)
        p = orc.block_priority(s, labels, idle, 0.001, [0.0] * 5)
        assert abs(p - float(orc.lrfu_priority(s, idle, 0.001))) < 1e-15


def test_region_survival_halves_at_the_half_life():
    """[MemDecay] §IV-B Eq.7: t_half = ln2 / lambda; with beta = 0 a block of
    one region keeps exactly half its survival at idle = t_half."""
    half = (170.0, 100.0, 60.0, 30.0, 15.0)
    rates = orc.region_decay_rates(half)
    for r, th in enumerate(half):
        assert abs(orc.block_survival([r] * 16, th, 0.0, rates) - 0.5) < 1e-14
        assert abs(orc.block_survival([r] * 16, 2 * th, 0.0, rates) - 0.25) < 1e-14
    # a block straddling two regions averages its tokens ([MemDecay] Eq.5 mean)
    mixed = [3] * 4 + [4] * 12
    want = (4 * 0.5 + 12 * 0.25) / 16               # idle 30: tool halves, scratch quarters
    assert abs(orc.block_survival(mixed, 30, 0.0, rates) - want) < 1e-14
    # beta multiplies in: exp(-beta*idle) times the region factor
    assert abs(orc.block_survival([3] * 16, 30, 0.001, rates) - 0.5 * math.exp(-0.03)) < 1e-14


def test_faster_decaying_region_is_evicted_first():
    rates = orc.region_decay_rates((170.0, 100.0, 60.0, 30.0, 15.0))
    p = [orc.block_priority(0.1, [r] * 16, 40, 0.001, rates) for r in range(5)]
    assert all(a < b for a, b in zip(p, p[1:]))


def test_beta_to_zero_without_regions_gives_zero_priority():
    """The formula (1 - score)(1 - e^{-beta idle}) goes to 0 as beta -> 0 (the
    figure's prose says it 'leaves (1 - score) alone'; the formula is taken)."""
    assert orc.block_priority(0.3, [0] * 16, 1000, 0.0, [0.0]) == 0.0
    assert orc.block_priority(0.3, [0] * 16, 1000, 1e-12, [0.0]) < 1e-9


# --- selection ------------------------------------------------------------------

def test_block_selection_matches_subset_enumeration():
    """[MemDecay] Eq.1 with the pinned set forced: the kept set minimises the
    summed priority over all budget-sized sets holding every pinned block."""
    rng = np.random.default_rng(11)
    for _ in range(150):
        n = int(rng.integers(3, 10))
        ids = np.sort(rng.choice(40, size=n, replace=False))
        prio = rng.uniform(0, 1, size=n)
        pinned = rng.uniform(size=n) < 0.25
        B = int(rng.integers(max(1, pinned.sum()), n + 1))
        kept = orc.select_blocks(ids, prio, pinned, B)
        best, best_set = None, None
        for S in itertools.combinations(range(n), min(B, n)):
            if not all(i in S for i in np.flatnonzero(pinned)):
                continue
            v = prio[list(S)].sum()
            if best is None or v < best - 1e-15:
                best, best_set = v, sorted(ids[list(S)].tolist())
        assert kept == best_set


def test_block_selection_ties_keep_the_higher_id_and_reject_overfull_pins():
    kept = orc.select_blocks([2, 5, 7, 9], [0.5, 0.5, 0.5, 0.9], [False] * 4, 2)
    assert kept == [5, 7]
    assert orc.select_blocks([1, 2], [0.9, 0.1], [False, False], 5) == [1, 2]
    with pytest.raises(ValueError):
        orc.select_blocks([1, 2, 3], [0.1, 0.2, 0.3], [True, True, True], 2)


# --- the step ----------------------------------------------------------------------

def _steered_oracle(page=1, budget=100, **kw):
    """One layer, one head, d = 3: keys e0 and e1 at positions 0 and 1, and
    queries sqrt(3)(log x, log(1-x), -1000) put mass x on token 0, 1-x on
    token 1 and exactly 0 on appended tokens (keys e2)."""
    o = orc.BlockLRFUOracle(1, 1, 1, 3, alpha_new=0.05, beta=0.001, half_lives=(1e9,) * 5,
                            pinned_regions=(), page=page, **kw)
    K = np.zeros((1, 1, 2, 3), np.float32)
    K[0, 0, 0, 0] = 1.0
    K[0, 0, 1, 1] = 1.0
    V = np.zeros_like(K)
    o.prefill(0, K, V, labels=[1, 1], budget=budget)
    return o


def _steer(x):
    q = np.array([math.log(x), math.log(1 - x), -1000.0]) * math.sqrt(3.0)
    kn = np.array([0.0, 0.0, 1.0])
    return (q.reshape(1, 1, 1, 3).astype(np.float32), kn.reshape(1, 1, 1, 3).astype(np.float32),
            np.zeros((1, 1, 1, 3), np.float32))


def test_block_score_follows_worked_ema_table_through_attention(golden_dir):
    """Masses 0.45, 0.12, 0.30, 0.08, 0.35 on block 0 reproduce the page's EMA
    chain (exact values; the printed column within its 3-decimal rounding)."""
    rows = _read_table(os.path.join(golden_dir, "lrfu_ema_table.txt"))
    o = _steered_oracle()
    xs = [float(r[1]) for r in rows]
    for t, (x, printed) in enumerate(zip(xs, (float(r[2]) for r in rows)), start=1):
        o.decode_step(t, *_steer(x), [0])
        o.evict(t)
        exact = sum(0.05 * 0.95 ** (t - tau) * xs[tau - 1] for tau in range(1, t + 1))
        s = o.seqs[0].score[0]
        assert abs(s - exact) < 1e-6            # inputs pass through fp32
        assert abs(s - printed) <= 1.1e-3
        assert abs(o.seqs[0].score[1] - sum(0.05 * 0.95 ** (t - tau) * (1 - xs[tau - 1])
                                            for tau in range(1, t + 1))) < 1e-6


def test_block_masses_sum_to_one_and_equal_softmax_for_single_token_blocks():
    rng = np.random.default_rng(5)
    L, Hq, Hkv, d, n = 2, 8, 2, 16, 37
    o = orc.BlockLRFUOracle(L, Hq, Hkv, d, alpha_new=0.05, beta=0.001, half_lives=(30.0,) * 5,
                            pinned_regions=(), page=4)
    K = rng.standard_normal((L, Hkv, n, d)).astype(np.float32)
    V = rng.standard_normal((L, Hkv, n, d)).astype(np.float32)
    o.prefill(0, K, V, labels=[2] * n, budget=1000)
    q = rng.standard_normal((L, 1, Hq, d)).astype(np.float32)
    kn = rng.standard_normal((L, 1, Hkv, d)).astype(np.float32)
    vn = rng.standard_normal((L, 1, Hkv, d)).astype(np.float32)
    o.decode_step(1, q, kn, vn, [0])
    assert abs(sum(o.seqs[0].last_mass.values()) - 1.0) < 1e-12
    # one layer, one head, page 1: the block mass is the softmax itself
    o1 = orc.BlockLRFUOracle(1, 1, 1, d, alpha_new=0.05, beta=0.001, half_lives=(30.0,) * 5,
                             pinned_regions=(), page=1)
    o1.prefill(0, K[:1, :1], V[:1, :1], labels=[2] * n, budget=1000)
    o1.decode_step(1, q[:1, :, :1], kn[:1, :, :1], vn[:1, :, :1], [0])
    keys = np.concatenate([K[0, 0], kn[0, 0, :1]], axis=0).astype(np.float64)
    want = softmax(keys @ q[0, 0, 0].astype(np.float64) / math.sqrt(d))
    got = np.array([o1.seqs[0].last_mass[j] for j in range(n + 1)])
    assert np.allclose(got, want, rtol=1e-12, atol=1e-300)


def test_access_clock_moves_only_above_twice_the_uniform_level():
    """[MemDecay] §III-C Eq.3 with tau = 2/|K_t| (§IV-A): with n resident
    tokens a one-token block is accessed iff its mass is at least 2/n."""
    o = _steered_oracle()
    s = o.seqs[0]
    # (x on token 0, expected tref of blocks 0 and 1); n = 3, 4, 5, 6, 7
    plan = [(0.9, 1, 0), (0.3, 1, 2), (0.35, 1, 3), (0.5, 4, 4), (0.2, 4, 5)]
    for t, (x, t0, t1) in enumerate(plan, start=1):
        o.decode_step(t, *_steer(x), [0])
        assert (s.tref[0], s.tref[1]) == (t0, t1)
        assert s.tref[t + 1] == t                 # the appended block entered at t
        assert all(s.tref[j] == j - 1 for j in range(2, t + 1))   # zero mass: never accessed


def test_evicted_score_persists_and_is_restored_on_readmission():
    """[LRFU-fig]: an evicted block's key and score are restored, not reset."""
    o = _steered_oracle(budget=3)
    o.decode_step(1, *_steer(0.2), [0])          # blocks 0, 1, 2 (tail)
    o.evict(1)
    o.decode_step(2, *_steer(0.2), [0])          # block 3 opens: 4 resident > 3
    s = o.seqs[0]
    prio = {j: o.priority(0, j, 2) for j in (0, 1, 2)}
    o.evict(2)
    gone = sorted({0, 1, 2, 3} - s.resident)
    assert len(gone) == 1 and gone[0] != 3        # the tail block is pinned
    j = gone[0]
    assert prio[j] == max(prio.values())
    frozen = s.score[j]
    for t in range(3, 7):
        o.decode_step(t, *_steer(0.5), [0])
        o.evict(t)
        assert j not in s.resident and s.score[j] == frozen     # frozen while out
    o.readmit(0, j, 6)
    assert j in s.resident and s.score[j] == frozen and s.tref[j] == 6
    with pytest.raises(ValueError):
        o.readmit(0, j, 6)
    o.decode_step(7, *_steer(0.5), [0])
    if j in (0, 1):
        assert abs(s.score[j] - (0.95 * frozen + 0.05 * 0.5)) < 1e-7   # continues from it


def test_pinned_region_protects_whole_straddling_pages_and_the_tail():
    """[MemDecay] §IV-A: pinning protects whole pages, so a page holding one
    system token is never evicted; the block being filled is pinned too."""
    d = 3
    o = orc.BlockLRFUOracle(1, 1, 1, d, alpha_new=0.05, beta=0.5, half_lives=(1e9,) * 5,
                            pinned_regions=(0,), page=4)
    n = 12
    K = np.zeros((1, 1, n, d), np.float32)
    K[0, 0, 4:, 0] = 1.0                          # blocks 1 and 2 draw the attention
    V = np.zeros_like(K)
    labels = [1, 1, 1, 0] + [3] * 8               # block 0 straddles: one system token
    o.prefill(0, K, V, labels=labels, budget=2)
    q = np.array([30.0, 0.0, 0.0], np.float32).reshape(1, 1, 1, d)
    kn = np.zeros((1, 1, 1, d), np.float32)
    for t in range(1, 4):
        o.decode_step(t, q, kn, kn, [0])
        o.evict(t)
        assert 0 in o.seqs[0].resident
        assert o.tail_block(0) in o.seqs[0].resident
        assert len(o.seqs[0].resident) == 2
    assert o.is_pinned(0, 0) and not o.is_pinned(0, 1)
