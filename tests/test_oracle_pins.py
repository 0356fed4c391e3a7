"""Pins of the CPU oracle against closed forms, invariants, independent
library routines and brute force on tiny inputs (no GPU).

Each test is chosen so that a plausible slip in the oracle (dropped term,
wrong sign or index, transposed operand, wrong head mapping, append after
instead of before attention, missing residual) fails at least one of them.
"""
import math
from dataclasses import replace

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
import synth

RNG = np.random.default_rng(1234)


def f32(a):
    return np.asarray(a, dtype=np.float32)


# ----------------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_vector_closed_form():
    # x = c * 1, unit gain: y_i = c / sqrt(c^2 + eps)
    for c in (0.5, -3.0, 1e-3):
        for eps in (1e-6, 0.25):
            y = oracle.rmsnorm(np.full(64, c, np.float32), np.ones(64, np.float32), eps)
            want = c / math.sqrt(c * c + eps)
            np.testing.assert_allclose(y, want, rtol=1e-6)


def test_rmsnorm_scale_invariance_and_unit_rms():
    x = f32(RNG.normal(size=512) * 7.0)
    g = np.ones(512, np.float32)
    y1 = oracle.rmsnorm(x, g, 0.0)
    y2 = oracle.rmsnorm(x * 3.5, g, 0.0)
    np.testing.assert_allclose(y1, y2, rtol=2e-7, atol=1e-7)
    # with eps = 0 the output has unit root-mean-square
    assert abs(math.sqrt(np.mean(y1.astype(np.float64) ** 2)) - 1.0) < 1e-6


def test_rmsnorm_gain_is_elementwise_and_bf16_gain():
    x = f32(RNG.normal(size=128))
    g = np.zeros(128, np.float32)
    g[17] = 2.0
    y = oracle.rmsnorm(x, g, 1e-6)
    assert np.count_nonzero(y) == 1 and y[17] != 0
    # bf16 gain of value 2.0 (0x4000) equals fp32 gain of 2.0
    yb = oracle.rmsnorm(x, np.full(128, 0x4000, np.uint16), 1e-6)
    yf = oracle.rmsnorm(x, np.full(128, 2.0, np.float32), 1e-6)
    np.testing.assert_array_equal(yb, yf)


# ----------------------------------------------------------------- matvec

def test_matvec_hand_example_and_orientation():
    W = f32([[1, 2], [3, 4], [5, 6]])  # [rows=3, cols=2]: y_r = sum_c W[r,c] x[c]
    y = oracle.matvec(W, f32([1, -1]))
    np.testing.assert_array_equal(y, f32([-1, -1, -1]))
    y = oracle.matvec(W, f32([2, 0.5]))
    np.testing.assert_array_equal(y, f32([3, 8, 13]))


def test_matvec_identity_and_numpy_float64():
    n = 96
    x = f32(RNG.normal(size=n))
    np.testing.assert_array_equal(oracle.matvec(np.eye(n, dtype=np.float32), x), x)
    W = f32(RNG.normal(size=(37, 300)))
    x = f32(RNG.normal(size=300))
    ref = W.astype(np.float64) @ x.astype(np.float64)
    np.testing.assert_allclose(oracle.matvec(W, x), ref.astype(np.float32), rtol=1e-6, atol=1e-6)


def test_matvec_bf16_weights_widen_exactly():
    Wf = f32(RNG.normal(size=(20, 64)))
    Wb = synth.f32_to_bf16(Wf)
    x = f32(RNG.normal(size=64))
    ref = synth.bf16_to_f32(Wb).astype(np.float64) @ x.astype(np.float64)
    np.testing.assert_allclose(oracle.matvec(Wb, x), ref.astype(np.float32), rtol=1e-6, atol=1e-6)


# ----------------------------------------------------------------- RoPE

def test_rope_position_zero_is_identity():
    v = f32(RNG.normal(size=128))
    np.testing.assert_array_equal(oracle.rope(v, 0), v)


def test_rope_pairs_and_first_frequency():
    D = 64
    for i in (0, 5, D // 2 - 1):
        e = np.zeros(D, np.float32)
        e[i] = 1.0
        r = oracle.rope(e, 3)
        nz = set(np.flatnonzero(np.abs(r) > 0))
        assert nz <= {i, i + D // 2}
    # pair 0 turns by exactly pos radians (frequency base^0 = 1)
    e = np.zeros(D, np.float32)
    e[0] = 1.0
    r = oracle.rope(e, 3)
    assert abs(r[0] - math.cos(3.0)) < 1e-7 and abs(r[D // 2] - math.sin(3.0)) < 1e-7


def test_rope_frequencies_geometric_in_base():
    # angle of pair i at pos 1, recovered with atan2, is base^(-2i/D)
    D, base = 16, 10000.0
    ang = []
    for i in range(D // 2):
        e = np.zeros(D, np.float32)
        e[i] = 1.0
        r = oracle.rope(e, 1, base)
        ang.append(math.atan2(float(r[i + D // 2]), float(r[i])))
    ratios = np.array(ang[1:]) / np.array(ang[:-1])
    np.testing.assert_allclose(ratios, base ** (-2.0 / D), rtol=1e-5)


def test_rope_norm_preserved_and_relative_position():
    D = 128
    q = f32(RNG.normal(size=D))
    k = f32(RNG.normal(size=D))
    for p in (1, 17, 1000):
        r = oracle.rope(q, p)
        a = q[: D // 2].astype(np.float64) ** 2 + q[D // 2:].astype(np.float64) ** 2
        b = r[: D // 2].astype(np.float64) ** 2 + r[D // 2:].astype(np.float64) ** 2
        np.testing.assert_allclose(a, b, rtol=1e-5, atol=1e-6)
    # <R(m) q, R(n) k> = <R(m - n) q, k>
    for m, n in ((9, 4), (300, 100), (7, 7)):
        lhs = float(np.dot(oracle.rope(q, m).astype(np.float64), oracle.rope(k, n).astype(np.float64)))
        rhs = float(np.dot(oracle.rope(q, m - n).astype(np.float64), k.astype(np.float64)))
        assert abs(lhs - rhs) < 1e-4 * (1 + abs(rhs))


# ----------------------------------------------------------------- attention

def test_attention_single_key_returns_v():
    D = 64
    q = f32(RNG.normal(size=D))
    K = f32(RNG.normal(size=(1, D)))
    V = f32(RNG.normal(size=(1, D)))
    out, p = oracle.attention_head(q, K, V, return_probs=True)
    np.testing.assert_array_equal(out, V[0])
    assert p[0] == 1.0


def test_attention_probs_sum_to_one_and_numpy():
    D, n = 32, 57
    q = f32(RNG.normal(size=D))
    K = f32(RNG.normal(size=(n, D)))
    V = f32(RNG.normal(size=(n, D)))
    out, p = oracle.attention_head(q, K, V, return_probs=True)
    assert abs(p.sum() - 1.0) < 1e-12
    s = K.astype(np.float64) @ q.astype(np.float64) / math.sqrt(D)
    ref = softmax(s) @ V.astype(np.float64)
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(p, softmax(s), rtol=1e-12)


def test_attention_two_key_closed_form():
    # D = 2, q = (1, 0): scores (0, ln 3) give weights (1/4, 3/4)
    a = math.sqrt(2.0) * math.log(3.0)
    q = f32([1, 0])
    K = f32([[0, 0], [a, 0]])
    V = f32([[4, 8], [0, -4]])
    out = oracle.attention_head(q, K, V)
    np.testing.assert_allclose(out, [1.0, -1.0], rtol=1e-6, atol=1e-6)


def test_attention_equal_keys_mean_dominant_and_permutation():
    D, n = 16, 9
    q = f32(RNG.normal(size=D))
    V = f32(RNG.normal(size=(n, D)))
    K = np.tile(f32(RNG.normal(size=D)), (n, 1))
    np.testing.assert_allclose(oracle.attention_head(q, K, V), V.astype(np.float64).mean(0), rtol=1e-6, atol=1e-6)
    K = f32(RNG.normal(size=(n, D)) * 0.01)
    K[4] = q * 100.0
    np.testing.assert_allclose(oracle.attention_head(q, K, V), V[4], rtol=1e-6, atol=1e-6)
    K = f32(RNG.normal(size=(n, D)))
    perm = RNG.permutation(n)
    a = oracle.attention_head(q, K, V)
    b = oracle.attention_head(q, np.ascontiguousarray(K[perm]), np.ascontiguousarray(V[perm]))
    np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-7)


# ----------------------------------------------------------------- SwiGLU

def test_swiglu_closed_form():
    g = f32([0.0, 1.0, -1.0, 30.0, -30.0, 0.5])
    u = f32([5.0, 2.0, 3.0, 1.0, 1.0, -4.0])
    out = oracle.swiglu(g, u)
    ref = g.astype(np.float64) * expit(g.astype(np.float64)) * u
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-12)
    assert out[0] == 0.0


# ----------------------------------------------------------------- layer / model

def _tiny_shape(**kw):
    base = synth.ModelShape(n_layers=1, hidden=64, n_heads=4, n_kv_heads=2, head_dim=16, ffn=96, vocab=50,
                            qk_norm=True, wdtype="f32", kv_dtype="f32")
    return replace(base, **kw)


def _weights(shape, seed=7):
    return synth.model_weights(shape, seed=seed, std=0.2)


def _cache(shape, cap, length, seed=8):
    return synth.kv_contents(shape, np.array([length]), cap, seed=seed)[0]


def test_layer_identity_when_output_projections_zero():
    # W_o = W_d = 0: the layer returns x unchanged; logits = W_lm . RMSNorm(E[tok])
    shape = _tiny_shape(n_layers=2)
    w = _weights(shape)
    for lw in w["layers"]:
        lw["wo"][:] = 0
        lw["w_down"][:] = 0
    o = oracle.Oracle(shape, w)
    cache = _cache(shape, 8, 3)
    tok = 11
    logits = o.model_forward(cache, tok, 3)
    x = w["embed"][tok].astype(np.float64)
    xn = x / np.sqrt(np.mean(x * x) + shape.eps)
    ref = w["lm_head"].astype(np.float64) @ xn
    np.testing.assert_allclose(logits, ref, rtol=1e-5, atol=1e-6)


def test_layer_append_before_attention_at_position_zero():
    # At pos 0 attention sees only the new key, so every q head of group g
    # returns v_g rounded to the cache type; with W_d = 0 the layer output is
    # x + W_o [v_{g(h)}]_h. bf16 cache: the rounded value is what counts.
    shape = _tiny_shape(kv_dtype="bf16", qk_norm=False)
    w = _weights(shape)
    lw = w["layers"][0]
    lw["w_down"][:] = 0
    o = oracle.Oracle(shape, w)
    cache = _cache(shape, 4, 0)
    x = f32(RNG.normal(size=shape.hidden))
    y = o.layer_forward(0, cache, 0, x)
    xd = x.astype(np.float64)
    xn = xd / np.sqrt(np.mean(xd * xd) + shape.eps)
    v = (lw["wv"].astype(np.float64) @ xn).astype(np.float32)
    vb = synth.bf16_to_f32(synth.f32_to_bf16(v)).reshape(shape.n_kv_heads, shape.head_dim)
    # appended row equals the rounded projection (1 bf16 ulp slack for fp64-vs-fp32 ties)
    got_v = synth.bf16_to_f32(cache["v"][0, :, 0, :])
    np.testing.assert_allclose(got_v, vb, rtol=2 ** -7, atol=1e-6)
    G = shape.n_heads // shape.n_kv_heads
    att = np.concatenate([got_v[h // G] for h in range(shape.n_heads)]).astype(np.float64)
    ref = xd + lw["wo"].astype(np.float64) @ att
    np.testing.assert_allclose(y, ref, rtol=1e-5, atol=1e-6)
    # positions other than 0 untouched
    assert not np.any(cache["v"][0, :, 1:, :])


def test_gqa_equals_mha_with_duplicated_kv_heads():
    # consecutive query heads share a KV head: h -> floor(h * Hkv / Hq)
    shape_g = _tiny_shape(n_heads=4, n_kv_heads=2)
    shape_m = replace(shape_g, n_kv_heads=4)
    wg = _weights(shape_g)
    wm = {"layers": [dict(wg["layers"][0])]}
    D = shape_g.head_dim
    dup = np.concatenate([np.arange(0, D), np.arange(0, D), np.arange(D, 2 * D), np.arange(D, 2 * D)])
    wm["layers"][0]["wk"] = np.ascontiguousarray(wg["layers"][0]["wk"][dup])
    wm["layers"][0]["wv"] = np.ascontiguousarray(wg["layers"][0]["wv"][dup])
    cg = _cache(shape_g, 12, 9)
    cm = {k: np.ascontiguousarray(cg[k][:, [0, 0, 1, 1]]) for k in ("k", "v")}
    x = f32(RNG.normal(size=shape_g.hidden))
    yg = oracle.Oracle(shape_g, wg).layer_forward(0, cg, 9, x)
    ym = oracle.Oracle(shape_m, wm).layer_forward(0, cm, 9, x)
    np.testing.assert_array_equal(yg, ym)
    # an interleaved mapping (h mod Hkv) would differ
    cm2 = {k: np.ascontiguousarray(cg[k][:, [0, 1, 0, 1]]) for k in ("k", "v")}
    wm2 = {"layers": [dict(wg["layers"][0])]}
    dup2 = np.concatenate([np.arange(0, D), np.arange(D, 2 * D), np.arange(0, D), np.arange(D, 2 * D)])
    wm2["layers"][0]["wk"] = np.ascontiguousarray(wg["layers"][0]["wk"][dup2])
    wm2["layers"][0]["wv"] = np.ascontiguousarray(wg["layers"][0]["wv"][dup2])
    ym2 = oracle.Oracle(shape_m, wm2).layer_forward(0, cm2, 9, x)
    assert not np.array_equal(yg, ym2)


def test_layer_matches_float64_composition_of_pinned_primitives():
    # the layer equals the composition of the individually pinned primitives
    shape = _tiny_shape()
    w = _weights(shape)
    lw = w["layers"][0]
    o = oracle.Oracle(shape, w)
    pos = 5
    cache = _cache(shape, 8, pos)
    cache_ref = {k: cache[k].copy() for k in cache}
    x = f32(RNG.normal(size=shape.hidden))
    y = o.layer_forward(0, cache, pos, x)
    # reference in float64 numpy + scipy, independently of the oracle's loops
    D, Hq, Hkv = shape.head_dim, shape.n_heads, shape.n_kv_heads
    xd = x.astype(np.float64)

    def rms(v, g):
        return v / np.sqrt(np.mean(v * v) + shape.eps) * g

    def rot(v, p):
        h = D // 2
        th = p * shape.rope_base ** (-2.0 * np.arange(h) / D)
        a, b = v[:h], v[h:]
        return np.concatenate([a * np.cos(th) - b * np.sin(th), b * np.cos(th) + a * np.sin(th)])

    xn = rms(xd, 1.0)
    q = (lw["wq"].astype(np.float64) @ xn).reshape(Hq, D)
    k = (lw["wk"].astype(np.float64) @ xn).reshape(Hkv, D)
    v = (lw["wv"].astype(np.float64) @ xn).reshape(Hkv, D)
    q = np.stack([rot(rms(q[h], 1.0), pos) for h in range(Hq)])
    k = np.stack([rot(rms(k[h], 1.0), pos) for h in range(Hkv)])
    K = cache_ref["k"][0].astype(np.float64)
    V = cache_ref["v"][0].astype(np.float64)
    K[:, pos] = k
    V[:, pos] = v
    att = []
    for h in range(Hq):
        g = h * Hkv // Hq
        s = K[g, : pos + 1] @ q[h] / math.sqrt(D)
        att.append(softmax(s) @ V[g, : pos + 1])
    x1 = xd + lw["wo"].astype(np.float64) @ np.concatenate(att)
    xn = rms(x1, 1.0)
    gt = lw["w_gate"].astype(np.float64) @ xn
    up = lw["w_up"].astype(np.float64) @ xn
    x2 = x1 + lw["w_down"].astype(np.float64) @ (gt * expit(gt) * up)
    np.testing.assert_allclose(y, x2, rtol=2e-5, atol=2e-5)


# ----------------------------------------------------------------- norm gains: routing and order
# With unit gains a swap of two gain vectors, or QK-norm applied after RoPE
# (RoPE keeps a head's RMS), changes nothing. The pins below use seeded
# non-unit gains, different for every vector, or gains that are zero
# except where a closed form needs them.

def _f64_layer(shape, lw, cache_ref, x, pos, order="norm_then_rope"):
    """float64 decoder layer in numpy; `order` chooses where QK-norm sits."""
    D, Hq, Hkv = shape.head_dim, shape.n_heads, shape.n_kv_heads
    xd = x.astype(np.float64)

    def g(name):
        return lw[name].astype(np.float64)

    def rms(v, gain):
        return v / np.sqrt(np.mean(v * v) + shape.eps) * gain

    def rot(v, p):
        h = D // 2
        th = p * shape.rope_base ** (-2.0 * np.arange(h) / D)
        a, b = v[:h], v[h:]
        return np.concatenate([a * np.cos(th) - b * np.sin(th), b * np.cos(th) + a * np.sin(th)])

    def head(v, gain):
        if order == "norm_then_rope":
            return rot(rms(v, gain), pos)
        return rms(rot(v, pos), gain)

    xn = rms(xd, g("attn_norm"))
    q = (g("wq") @ xn).reshape(Hq, D)
    k = (g("wk") @ xn).reshape(Hkv, D)
    v = (g("wv") @ xn).reshape(Hkv, D)
    q = np.stack([head(q[h], g("q_norm")) for h in range(Hq)])
    k = np.stack([head(k[h], g("k_norm")) for h in range(Hkv)])
    K = cache_ref["k"][0].astype(np.float64)
    V = cache_ref["v"][0].astype(np.float64)
    K[:, pos] = k
    V[:, pos] = v
    att = []
    for h in range(Hq):
        grp = h * Hkv // Hq
        s = K[grp, : pos + 1] @ q[h] / math.sqrt(D)
        att.append(softmax(s) @ V[grp, : pos + 1])
    x1 = xd + g("wo") @ np.concatenate(att)
    xn = rms(x1, g("mlp_norm"))
    gt = g("w_gate") @ xn
    up = g("w_up") @ xn
    return x1 + g("w_down") @ (gt * expit(gt) * up), k


def test_random_gains_are_distinct_per_vector_and_layer():
    # the seeded gain draws differ between vectors and layers (else a swap
    # of two of them could not be seen)
    shape = _tiny_shape(n_layers=2)
    w = synth.model_weights(shape, seed=7, gains="random")
    vecs = [w["final_norm"]] + [lw[n] for lw in w["layers"] for n in ("attn_norm", "mlp_norm", "q_norm", "k_norm")]
    for i in range(len(vecs)):
        assert np.all(np.isfinite(vecs[i])) and abs(float(np.std(vecs[i])) - synth.GAIN_STD) < 0.12
        for j in range(i):
            n = min(vecs[i].size, vecs[j].size)
            assert not np.array_equal(vecs[i][:n], vecs[j][:n])


def test_layer_with_distinct_gains_matches_float64_composition_and_rejects_planted_mistakes():
    # the layer with different non-unit gains everywhere equals the float64
    # composition with R3's order (QK-norm, then RoPE); the same composition
    # with the two norms' places exchanged, and the oracle fed swapped gain
    # vectors, both land far outside the tolerance
    shape = _tiny_shape()
    w = synth.model_weights(shape, seed=7, std=0.2, gains="random")
    lw = w["layers"][0]
    pos = 5
    cache = _cache(shape, 8, pos)
    ref_cache = {k: cache[k].copy() for k in cache}
    x = f32(RNG.normal(size=shape.hidden))
    y = oracle.Oracle(shape, w).layer_forward(0, cache, pos, x)
    want, k_new = _f64_layer(shape, lw, ref_cache, x, pos)
    scale = float(np.abs(want - x).max())
    np.testing.assert_allclose(y, want, rtol=2e-5, atol=2e-5)
    np.testing.assert_allclose(cache["k"][0, :, pos], k_new, rtol=2e-5, atol=2e-6)
    # norm after RoPE: the appended keys and the layer output change
    wrong, k_wrong = _f64_layer(shape, lw, ref_cache, x, pos, order="rope_then_norm")
    assert float(np.abs(cache["k"][0, :, pos] - k_wrong).max()) > 1e-2
    assert float(np.abs(y - wrong).max()) > 1e-3 * scale
    # planted in the oracle's inputs: swapped q/k gains, swapped attn/mlp gains
    for a, b in (("q_norm", "k_norm"), ("attn_norm", "mlp_norm")):
        wp = {"layers": [dict(lw)]}
        wp["layers"][0][a], wp["layers"][0][b] = lw[b], lw[a]
        c2 = {k: ref_cache[k].copy() for k in ref_cache}
        yp = oracle.Oracle(shape, wp).layer_forward(0, c2, pos, x)
        assert float(np.abs(yp - want).max()) > 1e-3 * scale, (a, b)


def test_appended_key_is_normed_then_rotated():
    # k at position p equals R(p) applied to k at position 0 (RoPE at 0 is
    # the identity), with the same x and weights. That holds when QK-norm
    # comes before RoPE; with a non-uniform k gain, norm after RoPE breaks it.
    shape = _tiny_shape()
    w = synth.model_weights(shape, seed=9, std=0.2, gains="random")
    o = oracle.Oracle(shape, w)
    x = f32(RNG.normal(size=shape.hidden))
    c0 = _cache(shape, 16, 0)
    o.layer_forward(0, c0, 0, x)
    for p in (1, 7, 13):
        cp = _cache(shape, 16, p)
        o.layer_forward(0, cp, p, x)
        for g in range(shape.n_kv_heads):
            want = oracle.rope(c0["k"][0, g, 0], p, shape.rope_base)
            np.testing.assert_allclose(cp["k"][0, g, p], want, rtol=1e-5, atol=1e-6)
            # the value row is not rotated
            np.testing.assert_array_equal(cp["v"][0, g, p], c0["v"][0, g, 0])
    # and at p = 0 the key row is the closed form g_k * a / rms(a), a = W_k xn
    xd = x.astype(np.float64)
    xn = xd / np.sqrt(np.mean(xd * xd) + shape.eps) * w["layers"][0]["attn_norm"]
    a = (w["layers"][0]["wk"].astype(np.float64) @ xn).reshape(shape.n_kv_heads, shape.head_dim)
    gk = w["layers"][0]["k_norm"].astype(np.float64)
    want0 = gk * a / np.sqrt(np.mean(a * a, axis=1, keepdims=True) + shape.eps)
    np.testing.assert_allclose(c0["k"][0, :, 0], want0, rtol=1e-5, atol=1e-6)


def test_attention_gain_feeds_qkv_and_mlp_gain_feeds_the_mlp():
    # zero gains give closed forms that a swap of the two vectors breaks:
    #  (1) mlp gain 0 and W_o = 0: attention adds nothing, the MLP sees a zero
    #      vector and adds silu(0) * 0 = 0, so the layer is the identity;
    #  (2) attention gain 0 except one channel c: the appended value row is
    #      column c of W_v times g_c x_c / rms(x)
    shape = _tiny_shape(qk_norm=False)
    w = synth.model_weights(shape, seed=11, std=0.2, gains="random")
    lw = w["layers"][0]
    x = f32(RNG.normal(size=shape.hidden))
    pos = 4
    w1 = {"layers": [dict(lw)]}
    w1["layers"][0]["mlp_norm"] = np.zeros_like(lw["mlp_norm"])
    w1["layers"][0]["wo"] = np.zeros_like(lw["wo"])
    y = oracle.Oracle(shape, w1).layer_forward(0, _cache(shape, 8, pos), pos, x)
    np.testing.assert_array_equal(y, x)
    w1s = {"layers": [dict(w1["layers"][0])]}
    w1s["layers"][0]["attn_norm"], w1s["layers"][0]["mlp_norm"] = w1["layers"][0]["mlp_norm"], lw["attn_norm"]
    ys = oracle.Oracle(shape, w1s).layer_forward(0, _cache(shape, 8, pos), pos, x)
    assert not np.array_equal(ys, x)
    c = 13
    w2 = {"layers": [dict(lw)]}
    ga = np.zeros_like(lw["attn_norm"])
    ga[c] = lw["attn_norm"][c]
    w2["layers"][0]["attn_norm"] = ga
    cache = _cache(shape, 8, pos)
    oracle.Oracle(shape, w2).layer_forward(0, cache, pos, x)
    xd = x.astype(np.float64)
    s = float(ga[c]) * xd[c] / math.sqrt(np.mean(xd * xd) + shape.eps)
    want = (lw["wv"][:, c].astype(np.float64) * s).reshape(shape.n_kv_heads, shape.head_dim)
    np.testing.assert_allclose(cache["v"][0, :, pos], want, rtol=1e-6, atol=1e-7)


def test_zero_q_gain_gives_uniform_attention_and_zero_k_gain_a_zero_key():
    # H = Hq * D, so W_o = I and W_d = 0 expose the attention output: y = x + att.
    #  (1) q gain 0: every score is 0, each head returns the mean of its group's
    #      value rows 0..pos (the appended row included);
    #  (2) k gain 0: the appended key row is exactly zero.
    # Swapping the q and k gain vectors breaks both.
    shape = _tiny_shape()
    H = shape.hidden
    assert shape.n_heads * shape.head_dim == H
    w = synth.model_weights(shape, seed=13, std=0.2, gains="random")
    lw = dict(w["layers"][0])
    lw["wo"] = np.eye(H, dtype=np.float32)
    lw["w_down"] = np.zeros_like(lw["w_down"])
    lw["q_norm"] = np.zeros_like(lw["q_norm"])
    pos = 6
    x = f32(RNG.normal(size=H) * 0.1)
    cache = _cache(shape, 8, pos)
    y = oracle.Oracle(shape, {"layers": [lw]}).layer_forward(0, cache, pos, x)
    G = shape.n_heads // shape.n_kv_heads
    V = cache["v"][0].astype(np.float64)
    want = np.concatenate([V[h // G, : pos + 1].mean(axis=0) for h in range(shape.n_heads)])
    np.testing.assert_allclose(y, x.astype(np.float64) + want, rtol=1e-5, atol=1e-6)
    lk = dict(w["layers"][0])
    lk["k_norm"] = np.zeros_like(lk["k_norm"])
    ck = _cache(shape, 8, pos)
    oracle.Oracle(shape, {"layers": [lk]}).layer_forward(0, ck, pos, x)
    assert not np.any(ck["k"][0, :, pos])
    ls = dict(lk)
    ls["q_norm"], ls["k_norm"] = lk["k_norm"], lk["q_norm"]  # swapped: the key gets the nonzero gain
    cs = _cache(shape, 8, pos)
    oracle.Oracle(shape, {"layers": [ls]}).layer_forward(0, cs, pos, x)
    assert np.any(cs["k"][0, :, pos])


def test_final_gain_closed_form_with_one_channel():
    # W_o = W_d = 0 keep x = E[tok]; a final gain that is zero except channel c
    # gives logits = W_lm[:, c] * g_c * x_c / rms(x)
    shape = _tiny_shape(n_layers=2)
    w = synth.model_weights(shape, seed=17, std=0.2, gains="random")
    for lw in w["layers"]:
        lw["wo"][:] = 0
        lw["w_down"][:] = 0
    c = 21
    gf = np.zeros_like(w["final_norm"])
    gf[c] = w["final_norm"][c]
    w["final_norm"] = gf
    tok = 17
    logits = oracle.Oracle(shape, w).model_forward(_cache(shape, 8, 3), tok, 3)
    x = w["embed"][tok].astype(np.float64)
    s = float(gf[c]) * x[c] / math.sqrt(np.mean(x * x) + shape.eps)
    np.testing.assert_allclose(logits, w["lm_head"][:, c].astype(np.float64) * s, rtol=1e-6, atol=1e-7)


# ----------------------------------------------------------------- 4-bit weights (W4A16)
# Format: codes in row order, two per byte, low nibble first; from byte
# rows * cols / 2 rounded up to 256, one bf16 scale per 128 inputs of a row;
# the weight is (code - 8) * scale.

def _w4_buffer(codes, scales):
    rows, cols = codes.shape
    off = synth.w4_scale_offset(rows, cols)
    buf = np.zeros(off + scales.size * 2, dtype=np.uint8)
    flat = codes.reshape(-1).astype(np.uint8)
    buf[: rows * cols // 2] = flat[0::2] | (flat[1::2] << 4)
    buf[off:] = synth.f32_to_bf16(scales.astype(np.float32).reshape(-1)).view(np.uint8)
    return buf


def test_w4_matvec_hand_example_nibble_order_and_groups():
    # row 0: all codes 9 (weight +scale) with scale 0.5 in group 0, 0.25 in group 1
    # row 1: codes alternate 0, 15 (weights -8s, +7s), scale 2 everywhere
    # row 2: only column 0 nonzero (code 15 in the low nibble of byte 0)
    rows, cols = 3, 256
    codes = np.full((rows, cols), 8)
    codes[0, :] = 9
    codes[1, 0::2] = 0
    codes[1, 1::2] = 15
    codes[2, 0] = 15
    scales = np.array([[0.5, 0.25], [2.0, 2.0], [1.0, 1.0]])
    x = f32(RNG.normal(size=cols))
    y = oracle.matvec(_w4_buffer(codes, scales), x, w4_shape=(rows, cols))
    xd = x.astype(np.float64)
    want = [0.5 * xd[:128].sum() + 0.25 * xd[128:].sum(),
            2.0 * (-8.0 * xd[0::2].sum() + 7.0 * xd[1::2].sum()),
            7.0 * xd[0]]
    np.testing.assert_allclose(y, np.array(want, dtype=np.float32), rtol=1e-6, atol=1e-6)


def test_w4_matvec_equals_float64_of_the_dequantised_matrix():
    rows, cols = 40, 1024
    buf = synth.w4_matrix(3, 9, rows, cols)
    x = f32(RNG.normal(size=cols))
    ref = synth.w4_dequant(buf, rows, cols) @ x.astype(np.float64)
    np.testing.assert_allclose(oracle.matvec(buf, x, w4_shape=(rows, cols)), ref.astype(np.float32), rtol=1e-6,
                               atol=1e-7)


def test_w4_layer_equals_layer_on_dequantised_matrices():
    # (code - 8) * bf16 scale is exact in fp32, so the layer with W4 matrices
    # equals, bit for bit, the layer given the dequantised fp32 matrices and
    # the same (bf16-valued) gains in fp32
    shape = _tiny_shape(hidden=1024, n_heads=8, n_kv_heads=2, head_dim=128, ffn=1024, wdtype="w4", kv_dtype="bf16")
    w = synth.model_weights(shape, seed=21, gains="random")
    lw = w["layers"][0]
    dims = {"wq": (1024, 1024), "wk": (256, 1024), "wv": (256, 1024), "wo": (1024, 1024), "w_gate": (1024, 1024),
            "w_up": (1024, 1024), "w_down": (1024, 1024)}
    f_shape = replace(shape, wdtype="f32")
    lf = {k: (f32(synth.w4_dequant(v, *dims[k])) if k in dims else synth.bf16_to_f32(v)) for k, v in lw.items()}
    pos = 7
    ca = _cache(shape, 10, pos)
    cb = {k: v.copy() for k, v in ca.items()}
    x = f32(RNG.normal(size=shape.hidden))
    ya = oracle.Oracle(shape, {"layers": [lw]}).layer_forward(0, ca, pos, x)
    yb = oracle.Oracle(f_shape, {"layers": [lf]}).layer_forward(0, cb, pos, x)  # same bf16 cache
    np.testing.assert_array_equal(ya, yb)
    np.testing.assert_array_equal(ca["k"], cb["k"])
