"""Pins of the CPU oracle to things other than itself: brute force on tiny
inputs, closed forms, invariants the pages fix, and special cases that reduce
to library routines.  CPU only."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

RNG = np.random.default_rng(1234)


class Spec:
    """A small layer description with the fields the oracle reads."""

    def __init__(self, **kw):
        self.n_heads, self.n_kv_heads, self.head_dim = 4, 2, 8
        self.d_model, self.d_ff = 32, 48
        self.rms_eps, self.rope_theta, self.rope_layout = 1e-5, 1e4, "neox"
        self.softcap, self.gated, self.qkv_bias, self.qk_norm = 0.0, False, False, False
        self.__dict__.update(kw)


def rand_layer(spec, scale=0.2, rng=RNG):
    qw, kw = spec.n_heads * spec.head_dim, spec.n_kv_heads * spec.head_dim
    d, f = spec.d_model, spec.d_ff
    w = {
        "g_attn": 1 + 0.1 * rng.standard_normal(d),
        "wq": scale * rng.standard_normal(((2 if spec.gated else 1) * qw, d)),
        "wk": scale * rng.standard_normal((kw, d)),
        "wv": scale * rng.standard_normal((kw, d)),
        "wo": scale * rng.standard_normal((d, qw)),
        "g_ffn": 1 + 0.1 * rng.standard_normal(d),
        "wg": scale * rng.standard_normal((f, d)),
        "wu": scale * rng.standard_normal((f, d)),
        "wd": scale * rng.standard_normal((d, f)),
    }
    if spec.qkv_bias:
        w.update(bq=0.3 * rng.standard_normal(qw), bk=0.3 * rng.standard_normal(kw),
                 bv=0.3 * rng.standard_normal(kw))
    if spec.qk_norm:
        w.update(q_norm=1 + 0.2 * rng.standard_normal(spec.head_dim),
                 k_norm=1 + 0.2 * rng.standard_normal(spec.head_dim))
    return w


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(b))


# ---------------------------------------------------------------------------
# brute-force attention: per token, per head, per key scalar loops in fp64


def brute_attention(q, k_all, v_all, start_pos, softcap=0.0, gate=None, window=0):
    B, Hq, hd = q.shape
    Hkv = k_all.shape[1]
    per_group = Hq // Hkv
    out = np.zeros((B, Hq, hd))
    for b in range(B):
        last = start_pos + b
        first = max(0, last - window + 1) if window else 0
        for h in range(Hq):
            g = h // per_group
            scores = []
            for j in range(first, last + 1):
                s = 0.0
                for c in range(hd):
                    s += float(q[b, h, c]) * float(k_all[j, g, c])
                s = s / math.sqrt(hd)
                if softcap:
                    s = softcap * math.tanh(s / softcap)
                scores.append(s)
            m = max(scores)
            e = [math.exp(s - m) for s in scores]
            z = sum(e)
            for c in range(hd):
                acc = 0.0
                for i, j in enumerate(range(first, last + 1)):
                    acc += e[i] / z * float(v_all[j, g, c])
                if gate is not None:
                    acc *= 1.0 / (1.0 + math.exp(-float(gate[b, h, c])))
                out[b, h, c] = acc
    return out


@pytest.mark.parametrize("B,S", [(2, 0), (3, 0), (4, 0), (2, 3), (4, 5)])
@pytest.mark.parametrize("softcap", [0.0, 1.0])
@pytest.mark.parametrize("gated", [False, True])
def test_attention_matches_brute_force(B, S, softcap, gated):
    Hq, Hkv, hd = 4, 2, 8
    q = 2.0 * RNG.standard_normal((B, Hq, hd))
    k_all = 2.0 * RNG.standard_normal((S + B, Hkv, hd))
    v_all = RNG.standard_normal((S + B, Hkv, hd))
    gate = RNG.standard_normal((B, Hq, hd)) if gated else None
    got = oracle.causal_gqa_attention(q, k_all, v_all, S, softcap, gate)
    want = brute_attention(q, k_all, v_all, S, softcap, gate)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("B,S,window", [(4, 0, 2), (3, 5, 3), (4, 6, 1), (2, 3, 9)])
def test_windowed_attention_matches_brute_force(B, S, window):
    Hq, Hkv, hd = 4, 2, 8
    q = 2.0 * RNG.standard_normal((B, Hq, hd))
    k_all = 2.0 * RNG.standard_normal((S + B, Hkv, hd))
    v_all = RNG.standard_normal((S + B, Hkv, hd))
    got = oracle.causal_gqa_attention(q, k_all, v_all, S, 1.0, None, window)
    want = brute_attention(q, k_all, v_all, S, 1.0, None, window)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_window_special_cases():
    B, S, Hq, Hkv, hd = 4, 3, 4, 2, 8
    q = RNG.standard_normal((B, Hq, hd))
    k_all = RNG.standard_normal((S + B, Hkv, hd))
    v_all = RNG.standard_normal((S + B, Hkv, hd))
    # a window as long as every key is no window at all
    np.testing.assert_array_equal(oracle.causal_gqa_attention(q, k_all, v_all, S, 0.0, None, S + B),
                                  oracle.causal_gqa_attention(q, k_all, v_all, S))
    # a window of one key: each token returns its own value row exactly
    o = oracle.causal_gqa_attention(q, k_all, v_all, S, 0.0, None, 1)
    for b in range(B):
        for h in range(Hq):
            assert np.array_equal(o[b, h], v_all[S + b, h // 2])


def test_attention_single_key_returns_its_value():
    # token 0 with no prefix sees only itself: output is v of its KV head, exactly
    Hq, Hkv, hd = 6, 3, 4
    q = RNG.standard_normal((1, Hq, hd))
    k = RNG.standard_normal((1, Hkv, hd))
    v = RNG.standard_normal((1, Hkv, hd))
    o = oracle.causal_gqa_attention(q, k, v, 0)
    for h in range(Hq):
        assert np.array_equal(o[0, h], v[0, h // 2])


def test_attention_equal_keys_average_values():
    B, S, Hq, Hkv, hd = 3, 4, 2, 1, 8
    q = RNG.standard_normal((B, Hq, hd))
    k_all = np.repeat(RNG.standard_normal((1, Hkv, hd)), S + B, axis=0)
    v_all = RNG.standard_normal((S + B, Hkv, hd))
    o = oracle.causal_gqa_attention(q, k_all, v_all, S)
    for b in range(B):
        want = v_all[: S + b + 1, 0].mean(axis=0)
        for h in range(Hq):
            np.testing.assert_allclose(o[b, h], want, rtol=1e-12, atol=1e-14)


def test_gqa_head_map_one_hot():
    # value of KV head g is the one-hot e_g, so head h must return e_{h // group}
    B, S, Hq, Hkv, hd = 3, 2, 8, 4, 8
    q = RNG.standard_normal((B, Hq, hd))
    k_all = RNG.standard_normal((S + B, Hkv, hd))
    v_all = np.zeros((S + B, Hkv, hd))
    for g in range(Hkv):
        v_all[:, g, g] = 1.0
    o = oracle.causal_gqa_attention(q, k_all, v_all, S)
    for h in range(Hq):
        want = np.zeros(hd)
        want[h // (Hq // Hkv)] = 1.0
        np.testing.assert_allclose(o[:, h], np.broadcast_to(want, (B, hd)), atol=1e-14)
    assert [oracle.kv_head_of(h, 24, 8) for h in range(24)] == [h // 3 for h in range(24)]


def test_gqa_equals_mha_with_repeated_kv():
    B, S, Hq, Hkv, hd = 4, 3, 6, 2, 8
    q = RNG.standard_normal((B, Hq, hd))
    k_all = RNG.standard_normal((S + B, Hkv, hd))
    v_all = RNG.standard_normal((S + B, Hkv, hd))
    gqa = oracle.causal_gqa_attention(q, k_all, v_all, S)
    mha = oracle.causal_gqa_attention(q, np.repeat(k_all, Hq // Hkv, axis=1),
                                      np.repeat(v_all, Hq // Hkv, axis=1), S)
    np.testing.assert_allclose(gqa, mha, rtol=1e-13, atol=1e-14)


def test_softcap_limits_and_gate_limits():
    B, S, Hq, Hkv, hd = 3, 2, 4, 2, 8
    q = 3 * RNG.standard_normal((B, Hq, hd))
    k_all = 3 * RNG.standard_normal((S + B, Hkv, hd))
    v_all = RNG.standard_normal((S + B, Hkv, hd))
    plain = oracle.causal_gqa_attention(q, k_all, v_all, S)
    np.testing.assert_allclose(oracle.causal_gqa_attention(q, k_all, v_all, S, 1e9), plain,
                               rtol=1e-10)
    assert rel(oracle.causal_gqa_attention(q, k_all, v_all, S, 0.5), plain) > 1e-3
    big = np.full((B, Hq, hd), 60.0)
    np.testing.assert_allclose(oracle.causal_gqa_attention(q, k_all, v_all, S, 0, big), plain,
                               rtol=1e-12)
    zero = np.zeros((B, Hq, hd))
    np.testing.assert_allclose(oracle.causal_gqa_attention(q, k_all, v_all, S, 0, zero),
                               plain / 2, rtol=1e-14)


def test_softcap_squashes_each_score():
    # with a cap c, a single huge score behaves like c: two keys with scores
    # +inf-ish and 0 give weights e^c/(e^c+1) and 1/(e^c+1)
    hd, c = 4, 2.0
    q = np.zeros((2, 1, hd)); q[1, 0, 0] = 1e4
    k = np.zeros((2, 1, hd)); k[0, 0, 0] = 1.0
    v = np.zeros((2, 1, hd)); v[0, 0, 1] = 1.0; v[1, 0, 2] = 1.0
    o = oracle.causal_gqa_attention(q, k, v, 0, softcap=c)
    w0 = math.exp(c) / (math.exp(c) + 1.0)
    np.testing.assert_allclose(o[1, 0], [0, w0, 1 - w0, 0], rtol=1e-12, atol=1e-15)


def test_attention_matches_torch_sdpa():
    B, Hq, Hkv, hd = 7, 6, 2, 16
    q = RNG.standard_normal((B, Hq, hd))
    k = RNG.standard_normal((B, Hkv, hd))
    v = RNG.standard_normal((B, Hkv, hd))
    got = oracle.causal_gqa_attention(q, k, v, 0)
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2)[None]
    want = F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True, enable_gqa=True)
    np.testing.assert_allclose(got, want[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# RMSNorm, SwiGLU


def test_rms_norm_constant_row_closed_form():
    c, eps = 0.37, 1e-5
    g = 1 + 0.1 * RNG.standard_normal(16)
    got = oracle.rms_norm(np.full((1, 16), c), g, eps)
    np.testing.assert_allclose(got[0], g * c / math.sqrt(c * c + eps), rtol=1e-15)


def test_rms_norm_scale_invariant_without_eps_and_matches_torch():
    x = RNG.standard_normal((5, 32))
    g = 1 + 0.1 * RNG.standard_normal(32)
    np.testing.assert_allclose(oracle.rms_norm(7.5 * x, g, 0.0), oracle.rms_norm(x, g, 0.0),
                               rtol=1e-13)
    want = F.rms_norm(torch.from_numpy(x), (32,), torch.from_numpy(g), eps=1e-5).numpy()
    np.testing.assert_allclose(oracle.rms_norm(x, g, 1e-5), want, rtol=1e-13)


def test_swiglu_matches_torch():
    h = RNG.standard_normal((3, 12))
    wg, wu, wd = (RNG.standard_normal(s) for s in [(20, 12), (20, 12), (12, 20)])
    th = torch.from_numpy(h)
    want = (F.silu(th @ torch.from_numpy(wg).T) * (th @ torch.from_numpy(wu).T)) \
        @ torch.from_numpy(wd).T
    np.testing.assert_allclose(oracle.swiglu_ffn(h, wg, wu, wd), want.numpy(), rtol=1e-12)
    np.testing.assert_allclose(oracle.silu(np.array([0.0, 1.0, -2.0])),
                               [0.0, 1 / (1 + math.exp(-1)), -2 / (1 + math.exp(2))], rtol=1e-15)


def test_gelu_matches_torch_and_normal_cdf():
    z = np.array([0.0, 1.0, -1.0, 3.5, -6.0, 0.25])
    want = F.gelu(torch.from_numpy(z), approximate="none").numpy()
    np.testing.assert_allclose(oracle.gelu(z), want, rtol=1e-14, atol=1e-300)
    # Phi(1) = 0.8413447460685429 (standard normal table)
    assert abs(oracle.gelu(np.array([1.0]))[0] - 0.8413447460685429) < 1e-15
    h = RNG.standard_normal((3, 12))
    wg, wu, wd = (RNG.standard_normal(s) for s in [(20, 12), (20, 12), (12, 20)])
    th = torch.from_numpy(h)
    ref = (F.gelu(th @ torch.from_numpy(wg).T) * (th @ torch.from_numpy(wu).T)) @ torch.from_numpy(wd).T
    np.testing.assert_allclose(oracle.swiglu_ffn(h, wg, wu, wd, "geglu"), ref.numpy(), rtol=1e-12)


# ---------------------------------------------------------------------------
# RoPE


def test_rope_hand_example_neox_and_norm():
    x = np.zeros((1, 1, 4)); x[0, 0, 0] = 1.0
    neox = oracle.apply_rope(x, [1], 1e4, "neox")[0, 0]
    norm = oracle.apply_rope(x, [1], 1e4, "norm")[0, 0]
    np.testing.assert_allclose(neox, [math.cos(1), 0, math.sin(1), 0], atol=1e-16)
    np.testing.assert_allclose(norm, [math.cos(1), math.sin(1), 0, 0], atol=1e-16)
    # the second pair turns at theta^(-2/4) = 1/100 rad per position
    x = np.zeros((1, 1, 4)); x[0, 0, 1] = 1.0
    np.testing.assert_allclose(oracle.apply_rope(x, [3], 1e4, "neox")[0, 0],
                               [0, math.cos(0.03), 0, math.sin(0.03)], atol=1e-16)


def test_rope_position_zero_is_identity_and_pairs_keep_norm():
    x = RNG.standard_normal((5, 3, 16))
    assert np.array_equal(oracle.apply_rope(x[:1], [0], 5e5), x[:1])
    y = oracle.apply_rope(x, np.arange(5) * 37, 5e5)
    pair = lambda a: a[..., :8] ** 2 + a[..., 8:] ** 2
    np.testing.assert_allclose(pair(y), pair(x), rtol=1e-13)


def test_rope_matches_complex_rotation():
    # neox pairs (i, i+hd/2) as the complex number x_i + 1j*x_{i+hd/2}
    hd, pos = 16, np.array([0, 1, 7, 4095])
    x = RNG.standard_normal((4, 2, hd))
    z = x[..., : hd // 2] + 1j * x[..., hd // 2:]
    freqs = np.array([5e5 ** (-2 * i / hd) for i in range(hd // 2)])
    zr = z * np.exp(1j * pos[:, None, None] * freqs[None, None, :])
    y = oracle.apply_rope(x, pos, 5e5, "neox")
    np.testing.assert_allclose(y[..., : hd // 2], zr.real, atol=1e-12)
    np.testing.assert_allclose(y[..., hd // 2:], zr.imag, atol=1e-12)


def test_rope_relative_position_property():
    hd = 32
    q, k = RNG.standard_normal((1, 1, hd)), RNG.standard_normal((1, 1, hd))
    def logit(pq, pk):
        return float(np.sum(oracle.apply_rope(q, [pq], 1e4) * oracle.apply_rope(k, [pk], 1e4)))
    for delta in (1, 100, 3000):
        assert abs(logit(10 + delta, 3 + delta) - logit(10, 3)) < 1e-9


def test_rope_options_freq_factors_partial_and_mscale():
    hd, pos = 8, [5]
    x = RNG.standard_normal((1, 1, hd))
    # frequency factors of 2 halve every angle: position 5 turns like 2.5
    half = oracle.apply_rope(x, pos, 1e4, freq_factors=np.full(4, 2.0))
    np.testing.assert_allclose(half, oracle.apply_rope(x, [2.5], 1e4), atol=1e-14)
    # a partial rotated width leaves the tail channels alone
    part = oracle.apply_rope(x, pos, 1e4, rot_dim=4)
    assert np.array_equal(part[..., 4:], x[..., 4:])
    np.testing.assert_allclose(part[..., :4], oracle.apply_rope(x[..., :4], pos, 1e4), atol=1e-15)
    # the attention factor scales the rotated channels only
    ms = oracle.apply_rope(x, pos, 1e4, rot_dim=4, mscale=0.5)
    np.testing.assert_allclose(ms[..., :4], 0.5 * part[..., :4], atol=1e-15)
    assert np.array_equal(ms[..., 4:], x[..., 4:])


def test_rope_options_hand_example():
    # rot_dim 2 of 4 channels, position 1, attention factor 0.5: only the first
    # pair turns (by 1 rad) and is halved; Norm and Neox pair the same channels
    x = np.array([[[1.0, 0.0, 5.0, 7.0]]])
    want = [0.5 * math.cos(1), 0.5 * math.sin(1), 5.0, 7.0]
    for lay in ("norm", "neox"):
        np.testing.assert_allclose(oracle.apply_rope(x, [1], 1e4, lay, rot_dim=2, mscale=0.5)[0, 0],
                                   want, atol=1e-16)
    # frequency factors divide each pair's frequency: factor 2 on pair 0
    e0 = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    np.testing.assert_allclose(oracle.apply_rope(e0, [1], 1e4, "neox", freq_factors=[2.0, 1.0])[0, 0],
                               [math.cos(0.5), 0.0, math.sin(0.5), 0.0], atol=1e-16)


@pytest.mark.parametrize("layout", ["norm", "neox"])
def test_projection_applies_every_rope_option(layout):
    # one-hot k rows reveal the angle, factor and pairing the projection step
    # applies: hd 8, rotated width 4, factors (1, 4), attention factor 2, position 3
    spec = Spec(n_heads=2, n_kv_heads=1, head_dim=8, d_model=8, rope_theta=1e4,
                rope_layout=layout, rope_rot_dim=4, rope_freq_factors=(1.0, 4.0), rope_mscale=2.0)
    w = rand_layer(spec)
    w["wk"] = np.eye(8)
    h = np.eye(8)                       # token c's k is e_c
    _, _, k, _ = oracle.project_qkv(h, w, spec, np.full(8, 3))
    k = k[:, 0, :]
    a0, a1 = 3.0, 3.0 * 1e4 ** (-2.0 / 4) / 4.0     # pair 0 and pair 1 angles
    p0, p1 = ((0, 1), (2, 3)) if layout == "norm" else ((0, 2), (1, 3))
    for (c0, c1), a in ((p0, a0), (p1, a1)):
        np.testing.assert_allclose(k[c0][[c0, c1]], [2 * math.cos(a), 2 * math.sin(a)], atol=1e-15)
        np.testing.assert_allclose(k[c1][[c0, c1]], [-2 * math.sin(a), 2 * math.cos(a)], atol=1e-15)
    for c in (4, 5, 6, 7):              # past the rotated width: untouched, unscaled
        np.testing.assert_array_equal(k[c], np.eye(8)[c])


# ---------------------------------------------------------------------------
# projections, positions, the layer


def test_projection_orientation_one_hot_input():
    spec = Spec(rope_theta=None)
    w = rand_layer(spec)
    j = 5
    h = np.zeros((1, spec.d_model)); h[0, j] = 1.0
    q, gate, k, v = oracle.project_qkv(h, w, spec, [0])
    np.testing.assert_array_equal(q.reshape(-1), w["wq"][:, j])
    np.testing.assert_array_equal(k.reshape(-1), w["wk"][:, j])
    np.testing.assert_array_equal(v.reshape(-1), w["wv"][:, j])
    assert gate is None


def test_gated_wq_split_first_half_q_second_half_gate():
    spec = Spec(gated=True, rope_theta=None)
    w = rand_layer(spec)
    h = RNG.standard_normal((2, spec.d_model))
    q, gate, _, _ = oracle.project_qkv(h, w, spec, [0, 1])
    qw = spec.n_heads * spec.head_dim
    np.testing.assert_allclose(q.reshape(2, -1), h @ w["wq"][:qw].T, rtol=1e-13)
    np.testing.assert_allclose(gate.reshape(2, -1), h @ w["wq"][qw:].T, rtol=1e-13)


def test_bias_then_qk_norm_then_rope_order():
    spec = Spec(qkv_bias=True, qk_norm=True)
    w = rand_layer(spec)
    w["wk"][:] = 0.0                      # k before the norm is the bias alone
    h = RNG.standard_normal((3, spec.d_model))
    S = 4
    _, _, k, _ = oracle.project_qkv(h, w, spec, S + np.arange(3))
    kb = w["bk"].reshape(spec.n_kv_heads, spec.head_dim)
    normed = kb / np.sqrt(np.mean(kb ** 2, axis=-1, keepdims=True) + spec.rms_eps) * w["k_norm"]
    want = oracle.apply_rope(np.broadcast_to(normed, (3,) + normed.shape), S + np.arange(3), 1e4)
    np.testing.assert_allclose(k, want, rtol=1e-13)


def test_positions_from_one_hot_key_rows():
    # k of head 0 before RoPE is e_0, so its row reveals the angle start_pos + b
    spec = Spec(n_heads=2, n_kv_heads=1, head_dim=4, d_model=8, rope_theta=1e4)
    w = rand_layer(spec)
    w["wk"][:] = 0.0
    w["wk"][0, :] = 1.0
    x = np.ones((6, spec.d_model))        # rms_norm(ones) * g has positive mean
    S = 9
    h = oracle.rms_norm(x, w["g_attn"], spec.rms_eps)
    amp = float(h[0].sum())
    _, k_rows, _ = oracle.dense_layer(x, w, spec, S, np.zeros((S, 4)), np.zeros((S, 4)))
    for b in range(6):
        np.testing.assert_allclose(k_rows[b] / amp, [math.cos(S + b), 0, math.sin(S + b), 0],
                                   atol=1e-12)


def test_layer_residual_structure():
    spec = Spec()
    w = rand_layer(spec)
    x = RNG.standard_normal((3, spec.d_model))
    z = dict(w, wo=np.zeros_like(w["wo"]), wd=np.zeros_like(w["wd"]))
    out, _, _ = oracle.dense_layer(x, z, spec, 0)
    assert np.array_equal(out, x)
    # one token and no prefix: attention returns v, so the layer has a closed form
    spec1 = Spec(qkv_bias=True)
    w = rand_layer(spec1)
    x = RNG.standard_normal((1, spec1.d_model))
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    h = F.rms_norm(t(x), (spec1.d_model,), t(w["g_attn"]), eps=spec1.rms_eps)
    v = h @ t(w["wv"]).T + t(w["bv"])
    o = v.reshape(1, spec1.n_kv_heads, spec1.head_dim).repeat_interleave(2, dim=1).reshape(1, -1)
    x1 = t(x) + o @ t(w["wo"]).T
    h2 = F.rms_norm(x1, (spec1.d_model,), t(w["g_ffn"]), eps=spec1.rms_eps)
    want = x1 + (F.silu(h2 @ t(w["wg"]).T) * (h2 @ t(w["wu"]).T)) @ t(w["wd"]).T
    got, _, v_rows = oracle.dense_layer(x, w, spec1, 0)
    # absolute floor: fp64 rounding of O(1) sums, for entries that land near zero
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(v_rows, v.numpy(), rtol=1e-13)


def one_token_layer_torch(x, w, spec):
    """A layer over one new token and an empty cache, in torch library calls:
    its only key is its own, so the attention returns v (repeated over each
    KV head's query group), and RoPE at position 0 is the identity.
    Returns (out, k_row, v_row)."""
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    n = lambda a, g: F.rms_norm(a, (spec.d_model,), t(g), eps=spec.rms_eps)
    h = n(t(x), w["g_attn"])
    k, v = h @ t(w["wk"]).T, h @ t(w["wv"]).T
    group = spec.n_heads // spec.n_kv_heads
    o = v.reshape(1, spec.n_kv_heads, spec.head_dim).repeat_interleave(group, dim=1).reshape(1, -1)
    x1 = t(x) + o @ t(w["wo"]).T
    h2 = n(x1, w["g_ffn"])
    out = x1 + (F.silu(h2 @ t(w["wg"]).T) * (h2 @ t(w["wu"]).T)) @ t(w["wd"]).T
    return out.numpy(), k.numpy(), v.numpy()


def test_stack_chains_layers_and_returns_each_layers_rows():
    # two different layers over one token: layer 1 must see layer 0's output
    # (not the input), and the rows of layer l must be layer l's projections
    # of its own input; both orders, plus an identity layer (wo = wd = 0)
    spec = Spec()
    a, b = rand_layer(spec), rand_layer(spec)
    ident = dict(rand_layer(spec), wo=np.zeros((spec.d_model, spec.n_heads * spec.head_dim)),
                 wd=np.zeros((spec.d_model, spec.d_ff)))
    x = RNG.standard_normal((1, spec.d_model))
    for first, second in ((a, b), (b, a), (ident, a), (a, ident)):
        y, k0, v0 = one_token_layer_torch(x, first, spec)
        z, k1, v1 = one_token_layer_torch(y, second, spec)
        out, ks, vs = oracle.prefill_dense_stack(x, [first, second], spec, 0)
        assert len(ks) == len(vs) == 2
        np.testing.assert_allclose(out, z, rtol=1e-12, atol=1e-13)
        for got, want in ((ks[0], k0), (vs[0], v0), (ks[1], k1), (vs[1], v1)):
            np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    # the identity layer passes its input through exactly, wherever it sits
    out, _, _ = oracle.prefill_dense_stack(x, [ident, ident], spec, 0)
    assert np.array_equal(out, x)


def test_sandwich_norms_closed_form_and_scale_invariance():
    # one token, no prefix: attention returns v, so a sandwich-norm layer has
    # a closed form in library calls
    spec = Spec(rope_theta=None)
    w = rand_layer(spec)
    w.update(g_post_attn=1 + 0.1 * RNG.standard_normal(spec.d_model),
             g_post_ffn=1 + 0.1 * RNG.standard_normal(spec.d_model))
    x = RNG.standard_normal((1, spec.d_model))
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    n = lambda a, g: F.rms_norm(a, (spec.d_model,), t(g), eps=spec.rms_eps)
    h = n(t(x), w["g_attn"])
    v = h @ t(w["wv"]).T
    o = v.reshape(1, spec.n_kv_heads, spec.head_dim).repeat_interleave(2, dim=1).reshape(1, -1)
    x1 = t(x) + n(o @ t(w["wo"]).T, w["g_post_attn"])
    h2 = n(x1, w["g_ffn"])
    want = x1 + n((F.silu(h2 @ t(w["wg"]).T) * (h2 @ t(w["wu"]).T)) @ t(w["wd"]).T, w["g_post_ffn"])
    got, _, _ = oracle.dense_layer(x, w, spec, 0)
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-13)
    # with eps 0 each branch's scale is normalised away: scaling wo and wd
    # leaves a 3-token output unchanged
    spec0 = Spec(rms_eps=0.0)
    x3 = RNG.standard_normal((3, spec.d_model))
    a, _, _ = oracle.dense_layer(x3, w, spec0, 0)
    b, _, _ = oracle.dense_layer(x3, dict(w, wo=7.0 * w["wo"], wd=0.01 * w["wd"]), spec0, 0)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


def test_returned_rows_are_rotated_k_and_v():
    spec = Spec(qk_norm=True, qkv_bias=True)
    w = rand_layer(spec)
    x = RNG.standard_normal((5, spec.d_model))
    S = 3
    pk, pv = RNG.standard_normal((S, 16)), RNG.standard_normal((S, 16))
    _, k_rows, v_rows = oracle.dense_layer(x, w, spec, S, pk, pv)
    h = oracle.rms_norm(x, w["g_attn"], spec.rms_eps)
    k = (h @ w["wk"].T + w["bk"]).reshape(5, 2, 8)
    k = k / np.sqrt(np.mean(k * k, -1, keepdims=True) + spec.rms_eps) * w["k_norm"]
    z = (k[..., :4] + 1j * k[..., 4:]) * np.exp(
        1j * (S + np.arange(5))[:, None, None] * (1e4 ** (-np.arange(4) / 4))[None, None, :])
    np.testing.assert_allclose(k_rows.reshape(5, 2, 8), np.concatenate([z.real, z.imag], -1),
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(v_rows, h @ w["wv"].T + w["bv"], rtol=1e-13)


# ---------------------------------------------------------------------------
# invariants of the stack


def _stack(spec, n_layers, rng=RNG):
    return [rand_layer(spec, rng=rng) for _ in range(n_layers)]


@pytest.mark.parametrize("extras", [dict(), dict(qkv_bias=True, qk_norm=True, softcap=3.0,
                                                  gated=True)])
def test_prefill_equals_single_token_steps(extras):
    spec = Spec(**extras)
    layers = _stack(spec, 3)
    N = 6
    x = RNG.standard_normal((N, spec.d_model))
    full, fk, fv = oracle.prefill_dense_stack(x, layers, spec, 0)
    ck = [np.zeros((0, 16)) for _ in layers]
    cv = [np.zeros((0, 16)) for _ in layers]
    for t in range(N):
        out, k, v = oracle.prefill_dense_stack(x[t:t + 1], layers, spec, t, ck, cv)
        np.testing.assert_allclose(out[0], full[t], rtol=1e-12, atol=1e-12)
        ck = [np.concatenate([a, b]) for a, b in zip(ck, k)]
        cv = [np.concatenate([a, b]) for a, b in zip(cv, v)]
    for l in range(3):
        np.testing.assert_allclose(ck[l], fk[l], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(cv[l], fv[l], rtol=1e-12, atol=1e-13)


def test_chunked_prefill_equals_whole():
    spec = Spec(qk_norm=True)
    layers = _stack(spec, 2)
    x = RNG.standard_normal((7, spec.d_model))
    full, fk, fv = oracle.prefill_dense_stack(x, layers, spec, 0)
    a, ak, av = oracle.prefill_dense_stack(x[:3], layers, spec, 0)
    b, bk, bv = oracle.prefill_dense_stack(x[3:], layers, spec, 3, ak, av)
    np.testing.assert_allclose(np.concatenate([a, b]), full, rtol=1e-12, atol=1e-12)
    for l in range(2):
        np.testing.assert_allclose(np.concatenate([ak[l], bk[l]]), fk[l], rtol=1e-12, atol=1e-13)


def test_causality_later_tokens_do_not_change_earlier():
    spec = Spec()
    layers = _stack(spec, 2)
    x = RNG.standard_normal((6, spec.d_model))
    y = x.copy(); y[4:] += 5.0
    a, ak, _ = oracle.prefill_dense_stack(x, layers, spec, 0)
    b, bk, _ = oracle.prefill_dense_stack(y, layers, spec, 0)
    assert np.array_equal(a[:4], b[:4]) and np.array_equal(ak[1][:4], bk[1][:4])
    assert not np.allclose(a[4:], b[4:])


def test_decode_attn_layer_equals_prefill_of_one_token():
    spec = Spec(gated=True, softcap=4.0, qk_norm=True)
    w = rand_layer(spec)
    R = 5
    ck, cv = RNG.standard_normal((R, 16)), RNG.standard_normal((R, 16))
    x = RNG.standard_normal((1, spec.d_model))
    want, k_row, v_row = oracle.dense_layer(x, w, spec, R, ck, cv)
    h = oracle.rms_norm(x, w["g_attn"], spec.rms_eps)
    q, gate, k, v = oracle.project_qkv(h, w, spec, [R])
    np.testing.assert_allclose(k.reshape(-1), k_row[0], rtol=1e-14)
    # the mirror may be bigger than the rows in use: only `rows` are read
    big_k = np.concatenate([ck, RNG.standard_normal((3, 16))])
    big_v = np.concatenate([cv, RNG.standard_normal((3, 16))])
    got = oracle.attn_layer(q.reshape(-1), k.reshape(-1), v.reshape(-1), gate.reshape(-1),
                            big_k, big_v, R, w, spec, x[0])
    np.testing.assert_allclose(got, want[0], rtol=1e-12)


# ---------------------------------------------------------------------------
# the input encoder


@pytest.mark.parametrize("opts", [dict(), dict(qkv_bias=True, qk_norm=True, gated=True, softcap=3.0,
                                             rope_layout="norm", rope_rot_dim=6,
                                             rope_freq_factors=(1.0, 2.0, 8.0), rope_mscale=0.8,
                                             ffn_act="geglu")])
def test_decode_layer_equals_one_token_prefill(opts):
    # the device-side decode layer (head + attention + tail) at position R is
    # the prefill of one token over the R cached rows
    spec = Spec(**opts)
    w = rand_layer(spec)
    R = 6
    ck = RNG.standard_normal((R, spec.n_kv_heads * spec.head_dim))
    cv = RNG.standard_normal((R, spec.n_kv_heads * spec.head_dim))
    x = RNG.standard_normal(spec.d_model)
    out, k_row, v_row = oracle.decode_layer(x, w, spec, ck, cv, R)
    want, wk, wv = oracle.dense_layer(x[None], w, spec, R, ck, cv)
    np.testing.assert_allclose(out, want[0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(k_row, wk[0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(v_row, wv[0], rtol=1e-13, atol=1e-14)


def test_bf16_encoder_matches_torch_rne():
    x = (RNG.standard_normal(100000) * 0.02).astype(np.float32)
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 0.0]   # exact ties round to even
    bits = synth.to_bf16_bits(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, want)
    assert np.array_equal(synth.bf16_bits_to_f32(bits),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_synthetic_draws_are_keyed_and_repeatable():
    cfg = synth.STACK_CONFIGS["tiny"]
    a = synth.layer_weights(cfg, 1)
    b = synth.layer_weights(cfg, 1)
    assert all(np.array_equal(a[n], b[n]) for n in a)
    c = synth.layer_weights(cfg, 0)
    assert not np.array_equal(a["wq"], c["wq"])
    assert a["wq"].shape == (256, 256) and a["wg"].shape == (704, 256)
    assert abs(float(np.std(a["wg"])) - 0.02) < 1e-3
    assert abs(float(np.mean(a["g_attn"])) - 1.0) < 1e-2


def test_tiny_stack_matches_committed_sample():
    """Regression pin: the oracle still gives the committed tiny-stack sample."""
    import importlib.util
    import json
    import os
    here = os.path.join(os.path.dirname(__file__), "golden")
    with open(os.path.join(here, "tiny_stack_sample.json")) as f:
        want = json.load(f)
    spec = importlib.util.spec_from_file_location("mk", os.path.join(here, "make_tiny_golden.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    got = mk.sample()
    for key in ("hidden_out", "k_rows_layer1", "v_rows_layer0"):
        np.testing.assert_allclose(got[key], want[key], rtol=1e-12, atol=1e-14)
