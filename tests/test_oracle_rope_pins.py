"""Pins of the rotary stage of the two-tier oracle ("QEvict" review, §4.4,
"Positional handling for promoted keys": keys quantized before the rotation
and rotated again at their original positions on promotion).

The pages give no formula for the rotation, so ``oracle.rope`` is pinned by
an independent formulation (complex multiplication by a unit phasor), by
values the standard library computes, and by the group properties any
position rotation must have: the identity at position 0, composition,
inversion, norm preservation, and logits that depend only on the distance
between the query's and the key's positions.  The tier oracle's rotary mode
is pinned end to end with keys that the INT2 quantizer represents exactly:
then a window that is quantized and promoted must come back as exactly the
rotated keys it was stored with.
"""
import math

import numpy as np
import torch

import oracle as orc


def _phasor_rope(x, positions, theta):
    """The same rotation written as complex arithmetic: channel pair
    (i, i + d/2) is the complex number x_i + j x_{i+d/2}, multiplied by
    exp(j * position * theta**(-2i/d))."""
    x = np.asarray(x, np.float64)
    h = x.shape[1] // 2
    z = x[:, :h] + 1j * x[:, h:]
    f = np.array([theta ** (-2.0 * i / x.shape[1]) for i in range(h)])
    z = z * np.exp(1j * np.outer(np.asarray(positions, np.float64), f))
    return np.concatenate([z.real, z.imag], axis=1)


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def test_rope_equals_the_complex_phasor_rotation():
    rng = np.random.default_rng(70)
    x = rng.standard_normal((37, 128))
    pos = rng.integers(0, 131072, 37)
    np.testing.assert_allclose(orc.rope(x, pos, 500000.0), _phasor_rope(x, pos, 500000.0), rtol=0, atol=1e-9)


def test_rope_of_one_channel_pair_is_cos_sin():
    """d = 2: the only frequency is theta**0 = 1, so e_0 turns into
    (cos p, sin p) and e_1 into (-sin p, cos p)."""
    for p in (0, 1, 7, 1000, 123457):
        np.testing.assert_allclose(orc.rope(np.array([[1.0, 0.0]]), [p], 10000.0)[0],
                                   [math.cos(p), math.sin(p)], rtol=0, atol=1e-12)
        np.testing.assert_allclose(orc.rope(np.array([[0.0, 1.0]]), [p], 10000.0)[0],
                                   [-math.sin(p), math.cos(p)], rtol=0, atol=1e-12)


def test_rope_group_properties():
    rng = np.random.default_rng(71)
    x = rng.standard_normal((16, 64))
    a = rng.integers(0, 40000, 16)
    b = rng.integers(0, 40000, 16)
    th = 500000.0
    np.testing.assert_array_equal(orc.rope(x, np.zeros(16), th), x)                  # position 0
    np.testing.assert_allclose(orc.rope(orc.rope(x, a, th), b, th), orc.rope(x, a + b, th), atol=1e-9)
    np.testing.assert_allclose(orc.rope(orc.rope(x, a, th), -a, th), x, atol=1e-10)  # inverse
    y = orc.rope(x, a, th)
    np.testing.assert_allclose(y[:, :32] ** 2 + y[:, 32:] ** 2, x[:, :32] ** 2 + x[:, 32:] ** 2, rtol=1e-12)


def test_rotated_logits_depend_only_on_the_distance():
    rng = np.random.default_rng(72)
    q = rng.standard_normal((1, 128))
    k = rng.standard_normal((1, 128))
    for m, n, shift in ((100, 3, 77), (5000, 4999, 12345), (0, 131071, 9)):
        base = (orc.rope(q, [m], 5e5) @ orc.rope(k, [n], 5e5).T).item()
        moved = (orc.rope(q, [m + shift], 5e5) @ orc.rope(k, [n + shift], 5e5).T).item()
        assert abs(base - moved) <= 1e-9 * max(1.0, abs(base))


def _grid_keys(rng, Hkv, n, d, W):
    """Keys that the per-channel INT2 quantizer of a W-token window
    represents exactly: every (window, channel) column takes values
    z + j*s, j in 0..3 with 0 and 3 present, z and s small dyadic numbers
    (exact in fp16, and every z + j*s exact in bf16)."""
    K = np.zeros((Hkv, n, d), np.float32)
    for h in range(Hkv):
        for w in range(n // W):
            z = rng.integers(-16, 16, d) / 8.0
            s = rng.integers(1, 8, d) / 16.0
            j = rng.integers(0, 4, (W, d))
            j[0], j[1] = 0, 3
            K[h, w * W:(w + 1) * W] = (z + j * s).astype(np.float32)
    return K


def test_promotion_reapplies_the_rotation_at_the_original_positions():
    """A window quantized from keys the quantizer represents exactly, then
    promoted, stores bf16(rope(code*scale + zero, positions)) =
    bf16(rope(k, positions)): exactly the rotated keys it held before its
    demotion.  While it is INT2 (exact reconstruction) attention reads the
    unrounded rotation rope(k, positions)."""
    rng = np.random.default_rng(73)
    L, Hq, Hkv, d, W, n = 1, 8, 2, 64, 8, 96
    K = _grid_keys(rng, Hkv, n, d, W)[None]
    V = rng.standard_normal((L, Hkv, n, d)).astype(np.float32)
    o = orc.TieredOracle(L, Hq, Hkv, d, k_f=1, k_q=1, window=W, n_sink=2, n_recent=8, rope_theta=5e5)
    o.prefill(K, V)
    st = o.layers[0]
    stored = st.K[:, :n].copy()
    pos = np.arange(n)
    for h in range(Hkv):      # storage holds the rotated keys rounded to bf16
        np.testing.assert_array_equal(stored[h], _bf16(_phasor_rope(K[0, h], pos, 5e5)))
    q = rng.standard_normal((L, Hq, d)).astype(np.float32)
    kn = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    vn = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    o.decode_step(1, q, kn, vn)
    cand = [w for w in range(o.n_windows()) if o.is_aged(w)]
    a, b = cand[3], cand[5]
    for w in cand:            # window a to F, window b to INT2, the rest evicted
        st.S[w] = {a: 2.0, b: 1.0}.get(w, 0.0)
    o.route()
    _, tiers, _ = o.window_state(0)
    assert tiers[a] == 0 and tiers[b] == 1
    sl = slice(b * W, (b + 1) * W)
    for h in range(Hkv):
        np.testing.assert_allclose(st.Keff[h, sl], _phasor_rope(K[0, h, sl], pos[sl], 5e5), rtol=0, atol=1e-9)
    st.S[b] = 3.0             # promote b
    o.route()
    _, tiers, _ = o.window_state(0)
    assert tiers[b] == 0
    np.testing.assert_array_equal(st.K[:, sl], stored[:, sl])
    np.testing.assert_array_equal(st.Keff[:, sl], stored[:, sl])


def test_rotary_attention_rotates_queries_at_the_new_position():
    """Nothing routed away: the step's output is softmax attention of
    bf16(rope(q, p)) over bf16(rope(k, position)) for every cached key,
    p the new token's position, written with the phasor rotation."""
    rng = np.random.default_rng(74)
    L, Hq, Hkv, d, n = 1, 8, 2, 64, 40
    K = rng.standard_normal((L, Hkv, n, d)).astype(np.float32)
    V = rng.standard_normal((L, Hkv, n, d)).astype(np.float32)
    o = orc.TieredOracle(L, Hq, Hkv, d, k_f=100, k_q=0, window=8, n_sink=0, n_recent=0, rope_theta=1e4)
    o.prefill(K, V)
    q = rng.standard_normal((L, Hq, d)).astype(np.float32)
    kn = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    vn = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    out = o.decode_step(1, q, kn, vn)
    Hg = Hq // Hkv
    for h in range(Hkv):
        keys = np.concatenate([K[0, h], kn[0, h][None]])
        vals = np.concatenate([V[0, h], vn[0, h][None]]).astype(np.float64)
        kr = _bf16(_phasor_rope(keys, np.arange(n + 1), 1e4)).astype(np.float64)
        qr = _bf16(_phasor_rope(q[0, h * Hg:(h + 1) * Hg], np.full(Hg, n), 1e4)).astype(np.float64)
        s = qr @ kr.T / math.sqrt(d)
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        np.testing.assert_allclose(out[0, h * Hg:(h + 1) * Hg], p @ vals, rtol=0, atol=1e-12)


def test_bf16_reconstruction_is_what_promotion_stores():
    """With reconstruct_bf16 an INT2 window is attended through
    bf16(rope(code*scale + zero)), which also replaces its stored keys, so a
    later promotion leaves storage unchanged."""
    rng = np.random.default_rng(75)
    L, Hq, Hkv, d, W, n = 1, 8, 2, 64, 8, 96
    K = rng.standard_normal((L, Hkv, n, d)).astype(np.float32)
    V = rng.standard_normal((L, Hkv, n, d)).astype(np.float32)
    o = orc.TieredOracle(L, Hq, Hkv, d, k_f=1, k_q=2, window=W, n_sink=2, n_recent=8, rope_theta=5e5,
                         reconstruct_bf16=True)
    o.prefill(K, V)
    st = o.layers[0]
    q = rng.standard_normal((L, Hq, d)).astype(np.float32)
    kn = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    vn = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    o.decode_step(1, q, kn, vn)
    cand = [w for w in range(o.n_windows()) if o.is_aged(w)]
    b = cand[2]
    for w in cand:
        st.S[w] = {cand[0]: 5.0, b: 1.0, cand[1]: 0.5}.get(w, 0.0)
    o.route()
    sl = slice(b * W, (b + 1) * W)
    kc, ks, kz, vc, vs, vz = st.ledger[b][1]
    khat = orc.int2_dequantize(kc, ks, kz, "channel")
    want = _bf16(_phasor_rope(khat, np.arange(b * W, (b + 1) * W), 5e5))
    np.testing.assert_array_equal(st.Keff[1, sl], want)
    np.testing.assert_array_equal(st.K[1, sl], want)
    np.testing.assert_array_equal(st.V[1, sl], _bf16(orc.int2_dequantize(vc, vs, vz, "token32")))
    kept = st.K[:, sl].copy()
    st.S[b] = 9.0
    o.route()
    np.testing.assert_array_equal(st.K[:, sl], kept)
