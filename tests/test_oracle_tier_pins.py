"""Pins of the two-tier (full precision / INT2 / evicted) window oracle.

The review of QEvict prints no end-to-end values, so the tiered oracle is
pinned by what the mathematics and the other, separately pinned parts fix:
the reduction to token-granular cumulative eviction (window of one token,
no INT2 tier), full softmax attention when nothing is routed away, the
conservation of attention mass in the cumulative score (softmax rows sum to
one, Eq.1 divides by Hq), the tier sizes and ordering of Eq.5, the
absorbing eviction state of Eq.6, and the once-only quantization of the
ledger (§4.4 Algorithm 1) checked against the quantizer applied to
the original inputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle as orc


def _inputs(rng, L, Hq, Hkv, d, n, steps, heavy=0.0):
    K = rng.standard_normal((L, Hkv, n, d)).astype(np.float32)
    V = rng.standard_normal((L, Hkv, n, d)).astype(np.float32)
    q = rng.standard_normal((steps, L, Hq, d)).astype(np.float32)
    if heavy:
        # a drifting query direction makes window scores cross (promotions happen)
        for t in range(steps):
            u = np.zeros(d, np.float32)
            u[(t // 4) % d] = heavy
            q[t] += u
            K[:, :, (t * 7) % n, (t // 4) % d] += heavy
    kn = rng.standard_normal((steps, L, Hkv, d)).astype(np.float32)
    vn = rng.standard_normal((steps, L, Hkv, d)).astype(np.float32)
    return K, V, q, kn, vn


def _run(o, q, kn, vn, after_route=None):
    outs = []
    for t in range(1, q.shape[0] + 1):
        outs.append(o.decode_step(t, q[t - 1], kn[t - 1], vn[t - 1]))
        o.route()
        if after_route:
            after_route(t)
    return outs


def test_capacities_of_the_131k_workload():
    """5% and 20% of 4096 windows, fractions rounded half up: 205 and 819."""
    nw = 131072 // 32
    assert math.floor(0.05 * nw + 0.5) == 205
    assert math.floor(0.20 * nw + 0.5) == 819


def test_window_of_one_without_int2_is_token_cumulative_eviction():
    """W = 1, K_q = 0, one KV head: routing keeps the sinks, the recent
    tokens and the K_f best candidates by cumulative mass -- exactly the
    token-granular cumulative rule with budget K_f + n_sink + n_recent
    (separately pinned).  The tiered score is the token score / Hq."""
    rng = np.random.default_rng(21)
    Hq, Hkv, d, n, T = 4, 1, 32, 40, 30
    k_f, n_sink, n_recent = 9, 2, 3
    K, V, q, kn, vn = _inputs(rng, 1, Hq, Hkv, d, n, T)
    tier = orc.TieredOracle(1, Hq, Hkv, d, k_f=k_f, k_q=0, window=1, n_sink=n_sink,
                            n_recent=n_recent)
    tier.prefill(K, V)
    tok = orc.TokenModeOracle(1, Hq, Hkv, d, budget=k_f + n_sink + n_recent, alpha_new=1.0,
                              policy="cumulative", n_sink=n_sink, n_recent=n_recent)
    tok.prefill(0, K, V)
    for t in range(1, T + 1):
        o1 = tier.decode_step(t, q[t - 1], kn[t - 1], vn[t - 1])
        o2 = tok.decode_step(t, q[t - 1][None], kn[t - 1][None], vn[t - 1][None], [0])
        np.testing.assert_allclose(o1, o2[:, 0], rtol=0, atol=1e-12)
        tier.route()
        tok.evict()
        pos, _ = tier.accessible_positions(0)
        np.testing.assert_array_equal(np.sort(pos), np.sort(tok.positions(0, 0)))
        S, tiers, _ = tier.window_state(0)
        kept = tok.positions(0, 0)
        np.testing.assert_allclose(4.0 * S[kept], tok.scores(0, 0), rtol=1e-12, atol=0)
        assert (tiers[kept] == 0).all()


def test_nothing_routed_away_is_full_softmax_attention():
    """With K_f at least the window count, every step is plain softmax
    attention over the whole cache (torch SDPA in fp64) and no window is
    ever quantized or evicted."""
    rng = np.random.default_rng(22)
    L, Hq, Hkv, d, n, T = 2, 8, 2, 64, 70, 12
    K, V, q, kn, vn = _inputs(rng, L, Hq, Hkv, d, n, T)
    o = orc.TieredOracle(L, Hq, Hkv, d, k_f=100, k_q=5, window=8, n_sink=3, n_recent=8)
    o.prefill(K, V)
    Kall, Vall = K.astype(np.float64), V.astype(np.float64)
    for t in range(1, T + 1):
        out = o.decode_step(t, q[t - 1], kn[t - 1], vn[t - 1])
        Kall = np.concatenate([Kall, kn[t - 1][:, :, None].astype(np.float64)], 2)
        Vall = np.concatenate([Vall, vn[t - 1][:, :, None].astype(np.float64)], 2)
        for l in range(L):
            qq = torch.from_numpy(q[t - 1, l].astype(np.float64)).reshape(Hkv, Hq // Hkv, d)
            ref = torch.nn.functional.scaled_dot_product_attention(
                qq, torch.from_numpy(Kall[l]), torch.from_numpy(Vall[l])).reshape(Hq, d).numpy()
            np.testing.assert_allclose(out[l], ref, rtol=0, atol=1e-12)
        o.route()
        for l in range(L):
            _, tiers, ledger = o.window_state(l)
            assert (tiers == 0).all() and not ledger.any()


def test_cumulative_scores_conserve_attention_mass():
    """Each step hands out exactly one unit of mass per layer (softmax rows
    sum to 1 and Eq.1 divides the head sum by Hq), so after t steps the
    scores of all windows ever seen, evicted ones included, sum to t."""
    rng = np.random.default_rng(23)
    L, Hq, Hkv, d, n, T = 2, 8, 2, 64, 200, 40
    K, V, q, kn, vn = _inputs(rng, L, Hq, Hkv, d, n, T, heavy=6.0)
    o = orc.TieredOracle(L, Hq, Hkv, d, k_f=3, k_q=6, window=8, n_sink=5, n_recent=8)
    o.prefill(K, V)

    def check(t):
        for l in range(L):
            S, tiers, _ = o.window_state(l)
            assert abs(S.sum() - t) < 1e-10
            assert (tiers == 2).any()

    _run(o, q, kn, vn, check)


def test_routing_sizes_order_and_absorbing_eviction():
    """Eq.5: F = the K_f best candidates, Q = the next K_q, the rest
    evicted; Eq.6: an evicted window never returns; pinned and local
    windows are never routed."""
    rng = np.random.default_rng(24)
    L, Hq, Hkv, d, n, T = 1, 8, 2, 64, 240, 48
    K, V, q, kn, vn = _inputs(rng, L, Hq, Hkv, d, n, T, heavy=6.0)
    W, k_f, k_q = 8, 4, 7
    o = orc.TieredOracle(L, Hq, Hkv, d, k_f=k_f, k_q=k_q, window=W, n_sink=5, n_recent=8)
    o.prefill(K, V)
    evicted = set()
    prev_cand = None
    for t in range(1, T + 1):
        o.decode_step(t, q[t - 1], kn[t - 1], vn[t - 1])
        nw = o.n_windows()
        S_pre, tiers_pre, _ = o.window_state(0)
        cand = [w for w in range(nw) if o.is_aged(w) and tiers_pre[w] != 2]
        o.route()
        S, tiers, _ = o.window_state(0)
        F = [w for w in cand if tiers[w] == 0]
        Q = [w for w in cand if tiers[w] == 1]
        E = [w for w in cand if tiers[w] == 2]
        assert len(F) == min(k_f, len(cand))
        assert len(Q) == min(k_q, len(cand) - len(F))
        key = lambda w: (S[w], w)
        if F and Q:
            assert min(map(key, F)) > max(map(key, Q))
        if Q and E:
            assert min(map(key, Q)) > max(map(key, E))
        assert evicted <= {w for w in range(nw) if tiers[w] == 2}
        evicted |= set(E)
        for w in range(nw):
            if not o.is_aged(w):
                assert tiers[w] == 0
        # candidates of the next event: F and Q of this one plus newly aged windows
        prev_cand = set(F) | set(Q)
    assert evicted


def test_ledger_is_written_once_from_the_original_values():
    """§4.4 Algorithm 1: a window's codes come from its original
    full-precision values at its first demotion and are reused through every
    later promotion and demotion; a promoted window's storage is its
    reconstruction rounded to bf16, and INT2 windows are attended through
    the fp32 reconstruction."""
    rng = np.random.default_rng(25)
    L, Hq, Hkv, d, n, T = 1, 8, 2, 64, 320, 64
    K, V, q, kn, vn = _inputs(rng, L, Hq, Hkv, d, n, T, heavy=8.0)
    W = 8
    o = orc.TieredOracle(L, Hq, Hkv, d, k_f=4, k_q=12, window=W, n_sink=5, n_recent=8)
    o.prefill(K, V)
    Kfull = np.concatenate([K[0], np.moveaxis(kn[:, 0], 0, 1)], 1)
    Vfull = np.concatenate([V[0], np.moveaxis(vn[:, 0], 0, 1)], 1)
    promoted = set()
    history = {}

    def check(t):
        st = o.layers[0]
        _, tiers, ledger = o.window_state(0)
        for w in np.flatnonzero(ledger).tolist():
            sl = slice(w * W, (w + 1) * W)
            for h in range(Hkv):
                kc, ks, kz = orc.int2_quantize(Kfull[h, sl], "channel")
                vc, vs, vz = orc.int2_quantize(Vfull[h, sl], "token32")
                e = st.ledger[w][h]
                for a, b in zip(e, (kc, ks, kz, vc, vs, vz)):
                    np.testing.assert_array_equal(a, b)
                khat = orc.int2_dequantize(kc, ks, kz, "channel")
                vhat = orc.int2_dequantize(vc, vs, vz, "token32")
                if tiers[w] == 1:
                    np.testing.assert_array_equal(st.Keff[h, sl], khat)
                    np.testing.assert_array_equal(st.Veff[h, sl], vhat)
                elif tiers[w] == 0:
                    kb = torch.from_numpy(khat).to(torch.bfloat16).float().numpy()
                    vb = torch.from_numpy(vhat).to(torch.bfloat16).float().numpy()
                    np.testing.assert_array_equal(st.Keff[h, sl], kb)
                    np.testing.assert_array_equal(st.Veff[h, sl], vb)
                    promoted.add(w)
            history.setdefault(w, []).append(int(tiers[w]))

    _run(o, q, kn, vn, check)
    assert promoted, "the drifting queries should promote at least one INT2 window"
    # some window went INT2 -> full precision -> INT2 again on the reused codes
    assert any(any(a == 0 and b == 1 for a, b in zip(h, h[1:])) and 0 in h[1:] for h in history.values())


def test_int2_windows_change_the_output_by_the_reconstruction_only():
    """Replacing an INT2 window's values by its reconstruction (rounded to
    bf16 once promoted) and dropping evicted windows are the only changes
    routing makes to attention: numpy's softmax over the tiered cache built
    by hand from the original inputs reproduces every step's output."""
    rng = np.random.default_rng(26)
    L, Hq, Hkv, d, n, T = 1, 8, 2, 64, 160, 12
    K, V, q, kn, vn = _inputs(rng, L, Hq, Hkv, d, n, T)
    W = 8
    o = orc.TieredOracle(L, Hq, Hkv, d, k_f=3, k_q=5, window=W, n_sink=2, n_recent=8)
    o.prefill(K, V)
    Kfull = np.concatenate([K[0], np.moveaxis(kn[:, 0], 0, 1)], 1)
    Vfull = np.concatenate([V[0], np.moveaxis(vn[:, 0], 0, 1)], 1)
    promoted = set()
    for t in range(1, T + 1):
        _, tiers, ledger = o.window_state(0)
        out = o.decode_step(t, q[t - 1], kn[t - 1], vn[t - 1])
        npos = n + t
        Ks, Vs = [], []
        for h in range(Hkv):
            kh, vh = [], []
            for w in range(-(-npos // W)):
                sl = slice(w * W, min((w + 1) * W, npos))
                tw = tiers[w] if w < len(tiers) else 0
                quantized = w < len(ledger) and ledger[w]
                if tw == 2:
                    continue
                if quantized:
                    kc, ks, kz = orc.int2_quantize(Kfull[h, sl], "channel")
                    vc, vs, vz = orc.int2_quantize(Vfull[h, sl], "token32")
                    khat = orc.int2_dequantize(kc, ks, kz, "channel")
                    vhat = orc.int2_dequantize(vc, vs, vz, "token32")
                    if tw == 0:      # promoted: the reconstruction rounded to bf16
                        khat = torch.from_numpy(khat).to(torch.bfloat16).float().numpy()
                        vhat = torch.from_numpy(vhat).to(torch.bfloat16).float().numpy()
                    kh.append(khat)
                    vh.append(vhat)
                else:
                    kh.append(Kfull[h, sl])
                    vh.append(Vfull[h, sl])
            Ks.append(np.concatenate(kh).astype(np.float64))
            Vs.append(np.concatenate(vh).astype(np.float64))
        Hg = Hq // Hkv
        for h in range(Hkv):
            s = q[t - 1, 0, h * Hg:(h + 1) * Hg].astype(np.float64) @ Ks[h].T / math.sqrt(d)
            p = np.exp(s - s.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            np.testing.assert_allclose(out[0, h * Hg:(h + 1) * Hg], p @ Vs[h], rtol=0, atol=1e-12)
        o.route()
        _, tiers_now, ledger_now = o.window_state(0)
        promoted |= set(np.flatnonzero((tiers_now == 0) & ledger_now).tolist())
    assert promoted, "some window should be promoted back from the INT2 tier"


def test_no_routing_event_within_the_interval_is_full_attention():
    """With an interval beyond the run no routing event happens ([QEvict]
    §4.2 Eq.1: events only at t = 0 mod Omega), so even with tight
    capacities every step is softmax attention over the whole cache and
    every window stays full precision."""
    rng = np.random.default_rng(25)
    L, Hq, Hkv, d, n, T = 1, 4, 2, 32, 60, 10
    K, V, q, kn, vn = _inputs(rng, L, Hq, Hkv, d, n, T)
    o = orc.TieredOracle(L, Hq, Hkv, d, k_f=1, k_q=1, window=8, n_sink=2, n_recent=4,
                         route_interval=T + 1)
    o.prefill(K, V)
    Kall, Vall = K.astype(np.float64), V.astype(np.float64)
    for t in range(1, T + 1):
        out = o.decode_step(t, q[t - 1], kn[t - 1], vn[t - 1])
        Kall = np.concatenate([Kall, kn[t - 1][:, :, None].astype(np.float64)], 2)
        Vall = np.concatenate([Vall, vn[t - 1][:, :, None].astype(np.float64)], 2)
        qq = torch.from_numpy(q[t - 1, 0].astype(np.float64)).reshape(Hkv, Hq // Hkv, d)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, torch.from_numpy(Kall[0]), torch.from_numpy(Vall[0])).reshape(Hq, d).numpy()
        np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-12)
        assert not o.routes_after(t)
        _, tiers, ledger = o.window_state(0)
        assert (tiers == 0).all() and not ledger.any()


def test_routing_every_omega_steps():
    """Omega = 4: tiers change only after steps 4, 8, ...; at each event the
    candidates are the windows kept by the previous event plus those aged
    since (Eq.4), ranked by the score accumulated over every step (Eq.1,
    Eq.5); attention mass is conserved throughout."""
    rng = np.random.default_rng(26)
    L, Hq, Hkv, d, n, T, omega = 1, 4, 2, 32, 90, 24, 4
    K, V, q, kn, vn = _inputs(rng, L, Hq, Hkv, d, n, T, heavy=6.0)
    o = orc.TieredOracle(L, Hq, Hkv, d, k_f=2, k_q=3, window=8, n_sink=3, n_recent=8,
                         route_interval=omega)
    o.prefill(K, V)
    prev = o.window_state(0)[1].copy()
    for t in range(1, T + 1):
        o.decode_step(t, q[t - 1], kn[t - 1], vn[t - 1])
        S, tiers, _ = o.window_state(0)
        assert abs(S.sum() - t) < 1e-10
        if not o.routes_after(t):
            np.testing.assert_array_equal(tiers[:len(prev)], prev)
            assert (tiers[len(prev):] == 0).all()  # windows opened since stay full precision
            prev = tiers.copy()
            continue
        cand = [w for w in range(o.n_windows()) if o.is_aged(w) and tiers[w] != 2]
        F, Q, E = orc.route_tiers(S, cand, 2, 3)
        o.route()
        S2, tiers2, _ = o.window_state(0)
        np.testing.assert_array_equal(S2, S)
        assert sorted(np.flatnonzero(tiers2 == 1).tolist()) == Q
        routed_f = [w for w in np.flatnonzero(tiers2 == 0).tolist() if w in cand]
        assert routed_f == F
        assert all(tiers2[w] == 2 for w in E)
        prev = tiers2.copy()


def test_held_memory_stays_within_the_byte_budget():
    """§4.1 (Budget) and §4.3 Eq.3: an evicted window holds nothing, not
    even its INT2 record; after every routing event the full-precision
    windows are the pinned and local ones plus at most K_f routed ones, and
    the records held are those of the F and Q windows that were ever
    quantized, at most K_f + K_q."""
    rng = np.random.default_rng(27)
    L, Hq, Hkv, d, n, T = 1, 8, 2, 64, 320, 64
    K, V, q, kn, vn = _inputs(rng, L, Hq, Hkv, d, n, T, heavy=8.0)
    W, k_f, k_q, n_sink, n_recent = 8, 4, 12, 5, 8
    o = orc.TieredOracle(L, Hq, Hkv, d, k_f=k_f, k_q=k_q, window=W, n_sink=n_sink, n_recent=n_recent)
    o.prefill(K, V)
    ever = set()
    dropped = []

    def check(t):
        _, tiers, ledger = o.window_state(0)
        nw = len(tiers)
        routed = [w for w in range(nw) if o.is_aged(w)]
        assert not (ledger & (tiers == 2)).any(), f"step {t}: an evicted window holds a record"
        assert int(((tiers == 0) & np.isin(np.arange(nw), routed)).sum()) <= k_f
        assert int(ledger.sum()) <= k_f + k_q
        held = set(np.flatnonzero(ledger).tolist())
        dropped.extend(w for w in ever - held if tiers[w] == 2)
        ever.update(held)
        for w in range(nw):
            if w not in routed:
                assert tiers[w] == 0        # pinned and local windows stay full precision

    _run(o, q, kn, vn, check)
    assert dropped, "some quantized window should be evicted (and lose its record)"


def test_key_groups_per_token_and_32_channels():
    """The literal reading of the 131k workload's "per-32-channel-group"
    scale and zero for keys as well (key_groups="token32"): a quantized
    window's key parameters are one (scale, zero) per (token, 32-channel
    group), and keys that each such group represents exactly (every row
    of a group holds z + j*s, j in 0..3 with 0 and 3 present, z and s
    dyadic) come back exactly from the reconstruction, while a per-channel
    grouping of the same keys does not."""
    rng = np.random.default_rng(29)
    L, Hq, Hkv, d, W, n, T = 1, 8, 2, 64, 8, 160, 12
    K = np.zeros((L, Hkv, n, d), np.float32)
    for h in range(Hkv):
        for t in range(n):
            for g in range(d // 32):
                z = rng.integers(-16, 16) / 8.0
                s = rng.integers(1, 8) / 16.0
                j = rng.integers(0, 4, 32)
                j[0], j[1] = 0, 3
                K[0, h, t, 32 * g:32 * g + 32] = z + j * s
    V = rng.standard_normal((L, Hkv, n, d)).astype(np.float32)
    q = rng.standard_normal((T, L, Hq, d)).astype(np.float32)
    kn = rng.standard_normal((T, L, Hkv, d)).astype(np.float32)
    vn = rng.standard_normal((T, L, Hkv, d)).astype(np.float32)
    o = orc.TieredOracle(L, Hq, Hkv, d, k_f=2, k_q=8, window=W, n_sink=2, n_recent=8, key_groups="token32")
    o.prefill(K, V)
    _run(o, q, kn, vn)
    st = o.layers[0]
    assert st.ledger
    for w, entry in st.ledger.items():
        sl = slice(w * W, (w + 1) * W)
        for h, (kc, ks, kz, vc, vs, vz) in enumerate(entry):
            assert np.shape(ks) == (W, d // 32) and np.shape(kz) == (W, d // 32)
            # the reconstruction written out: code * scale + zero of the (token, group)
            khat = np.empty((W, d), np.float32)
            for t in range(W):
                for c in range(d):
                    khat[t, c] = np.float32(np.float32(kc[t, c]) * np.float32(ks[t, c // 32])) + np.float32(kz[t, c // 32])
            if w * W + W <= n:  # a prefill window: the grid keys come back exactly
                np.testing.assert_array_equal(khat, K[0, h, sl])
                c2, s2, z2 = orc.int2_quantize(K[0, h, sl], "channel")
                per_channel = orc.int2_dequantize(c2, s2, z2, "channel")
                assert not np.array_equal(per_channel, K[0, h, sl])
