"""Pins of the CPU oracle against closed forms, invariants and brute force.

Each test checks one operator of the decode step listed in section 2 of the
page "Flint Inference on Apple Silicon: rec Megakernel and Tempo9 Compared"
against something other than the oracle's own formula: a closed-form value,
an invariant of the mathematics, a brute-force search, or a library routine
(numpy) on a special case that reduces to it.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ------------------------------------------------------------------ RMSNorm

def test_rmsnorm_constant_vector_closed_form():
    rng = np.random.default_rng(1)
    for c in (0.5, -3.0, 1e-3, 7.25):
        n, eps = 2048, 1e-6
        g = rng.normal(size=n).astype(np.float32)
        y = oracle.rmsnorm(np.full(n, c), g, eps)
        np.testing.assert_allclose(y, c / math.sqrt(c * c + eps) * g.astype(np.float64), rtol=1e-13, atol=0)


def test_rmsnorm_scale_invariance_and_unit_rms():
    rng = np.random.default_rng(2)
    x = rng.normal(size=2048) * 3.0
    g = np.ones(2048, np.float32)
    y1 = oracle.rmsnorm(x, g, 0.0)
    y2 = oracle.rmsnorm(x * 17.0, g, 0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-12)
    assert abs(np.sqrt(np.mean(y1 ** 2)) - 1.0) < 1e-12


def test_rmsnorm_bf16_output_is_representable():
    rng = np.random.default_rng(3)
    y = oracle.rmsnorm(rng.normal(size=256), np.ones(256, np.float32), 1e-6, round_bf16_out=True)
    bits = y.astype(np.float32).view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)


def test_round_bf16_ties_to_even():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: even mantissa (1.0) wins
    assert oracle.round_bf16(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert oracle.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert oracle.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -20) == 1.0 + 2.0 ** -7


# ------------------------------------------------------------------ softmax

def test_softmax_sums_to_one_shift_invariant_equal_scores():
    rng = np.random.default_rng(4)
    z = rng.normal(size=64) * 5
    p = oracle.softmax(z)
    assert abs(p.sum() - 1.0) < 1e-14
    np.testing.assert_allclose(oracle.softmax(z + 123.0), p, rtol=1e-12)
    np.testing.assert_allclose(oracle.softmax(np.full(7, 3.3)), np.full(7, 1 / 7), rtol=1e-15)
    # two logits: logistic function
    d = 0.731
    np.testing.assert_allclose(oracle.softmax([d, 0.0])[0], 1.0 / (1.0 + math.exp(-d)), rtol=1e-15)
    # large logits do not overflow (max subtracted)
    assert np.isfinite(oracle.softmax([1000.0, 999.0])).all()


# ------------------------------------------------------------------ attention

def test_attention_single_position_returns_v():
    rng = np.random.default_rng(5)
    d = 128
    q, k, v = rng.normal(size=d), rng.normal(size=(1, d)), rng.normal(size=(1, d))
    np.testing.assert_array_equal(oracle.attention_head(q, k, v), v[0].astype(np.float32).astype(np.float64))


def test_attention_equal_keys_gives_mean_of_v():
    rng = np.random.default_rng(6)
    T, d = 37, 64
    k = np.tile(rng.normal(size=d), (T, 1))
    v = rng.normal(size=(T, d)).astype(np.float32)
    out = oracle.attention_head(rng.normal(size=d), k, v)
    np.testing.assert_allclose(out, v.astype(np.float64).mean(0), rtol=1e-12, atol=1e-14)


def test_attention_dominant_score_selects_its_value():
    rng = np.random.default_rng(7)
    T, d = 16, 64
    k = np.zeros((T, d), np.float32)
    k[9, 0] = 1.0
    v = rng.normal(size=(T, d)).astype(np.float32)
    q = np.zeros(d)
    q[0] = 1e4
    np.testing.assert_allclose(oracle.attention_head(q, k, v), v[9], rtol=1e-12, atol=1e-12)


def test_attention_scale_is_inverse_sqrt_head_dim():
    # two keys, scores alpha/sqrt(d) and 0: weight of key 0 is the logistic of alpha/sqrt(d)
    rng = np.random.default_rng(8)
    for d in (64, 128):
        alpha = 3.0
        k = np.zeros((2, d), np.float32)
        k[0, 5] = 1.0
        q = np.zeros(d)
        q[5] = alpha
        v = rng.normal(size=(2, d)).astype(np.float32)
        p0 = 1.0 / (1.0 + math.exp(-alpha / math.sqrt(d)))
        vd = v.astype(np.float64)
        np.testing.assert_allclose(oracle.attention_head(q, k, v), p0 * vd[0] + (1 - p0) * vd[1], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------ RoPE

def test_rope_position_zero_is_identity():
    rng = np.random.default_rng(9)
    v = rng.normal(size=128)
    np.testing.assert_array_equal(oracle.rope(v, 0, 1e4), v)


def test_rope_preserves_pair_norms():
    rng = np.random.default_rng(10)
    d = 128
    v = rng.normal(size=d)
    r = oracle.rope(v, 8022, 1e4)
    np.testing.assert_allclose(r[: d // 2] ** 2 + r[d // 2:] ** 2, v[: d // 2] ** 2 + v[d // 2:] ** 2, rtol=1e-12)


def test_rope_rotate_half_pairing_and_direction():
    # basis vector e_i at position p goes to cos(phi) e_i + sin(phi) e_{i+d/2}, phi = p * base^(-2i/d)
    d, base = 64, 1e4
    for i in (0, 1, 17, 31):
        for p in (1, 5, 1000):
            e = np.zeros(d)
            e[i] = 1.0
            r = oracle.rope(e, p, base)
            phi = p * base ** (-2.0 * i / d)
            expect = np.zeros(d)
            expect[i], expect[i + d // 2] = math.cos(phi), math.sin(phi)
            np.testing.assert_allclose(r, expect, atol=1e-12)


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(11)
    d = 128
    q, k = rng.normal(size=d), rng.normal(size=d)
    ref = np.dot(oracle.rope(q, 10, 1e4), oracle.rope(k, 3, 1e4))
    for m, n in ((107, 100), (8029, 8022), (7, 0)):
        assert abs(np.dot(oracle.rope(q, m, 1e4), oracle.rope(k, n, 1e4)) - ref) < 1e-9 * max(1, abs(ref))
    # and with e_i the score is cos((m - n) * base^(-2i/d))
    i = 9
    e = np.zeros(d)
    e[i] = 1.0
    assert abs(np.dot(oracle.rope(e, 50, 1e4), oracle.rope(e, 20, 1e4)) - math.cos(30 * 1e4 ** (-2 * i / d))) < 1e-12


# ------------------------------------------------------------------ weights / GEMV

def _pack_int4(q):
    u = (np.asarray(q) + 8).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def test_int4_dequant_hand_built_group():
    rows, cols = 3, 128
    q = np.tile(np.arange(-8, 8), (rows, cols // 16))        # codes -8..7 repeating
    codes = _pack_int4(q)
    # scales: 0.5 (0x3F00), 2.0 (0x4000), 0.0
    scales = np.array([[0x3F00, 0x4000], [0x4000, 0x3F00], [0x0000, 0x3F00]], np.uint16)
    m = {"w": codes, "s": scales}
    s = np.array([[0.5, 2.0], [2.0, 0.5], [0.0, 0.5]])
    for r in range(rows):
        for c in (0, 1, 2, 15, 63, 64, 65, 127):
            assert oracle.weight(m, oracle.INT4G64, r, c) == s[r, c // 64] * q[r, c]
    # one-hot activation extracts a dequantised column (even column = low nibble)
    for c in (0, 1, 64, 127):
        x = np.zeros(cols)
        x[c] = 1.0
        np.testing.assert_array_equal(oracle.linear(m, oracle.INT4G64, x), s[:, c // 64] * q[:, c])


def test_linear_matches_numpy_matvec_fp32_and_bf16():
    rng = np.random.default_rng(12)
    w = rng.normal(size=(96, 200)).astype(np.float32)
    x = rng.normal(size=200)
    np.testing.assert_allclose(oracle.linear({"w": w}, oracle.F32, x), w.astype(np.float64) @ x, rtol=1e-12, atol=1e-12)
    wb = (w.view(np.uint32) >> 16).astype(np.uint16)
    wf = oracle.bf16_bits_to_f32(wb).astype(np.float64)
    np.testing.assert_allclose(oracle.linear({"w": wb}, oracle.BF16, x), wf @ x, rtol=1e-12, atol=1e-12)


def test_generator_int4_quantisation_recipe():
    # the synthetic int4 weights follow the stated recipe: scale = bf16(absmax/7),
    # |dequant - w| <= scale/2, and the element of largest magnitude maps to code +-7
    codes, scales = synth.int4g64(synth.tensor_id(synth.EGATE, 3, 1), 8, 256, 0.02)
    w = synth.normal_f32(synth.tensor_id(synth.EGATE, 3, 1), 8 * 256, 0.02).reshape(8, 256)
    m = {"w": codes, "s": scales}
    for r in range(8):
        for g in range(4):
            grp = w[r, g * 64:(g + 1) * 64].astype(np.float64)
            s = oracle.bf16_bits_to_f32(scales[r, g:g + 1])[0]
            assert abs(s - np.abs(grp).max() / 7) <= abs(s) * 2 ** -8
            deq = np.array([oracle.weight(m, oracle.INT4G64, r, g * 64 + j) for j in range(64)])
            assert np.all(np.abs(deq - grp) <= s / 2 * (1 + 1e-6) + 1e-12)
            j = np.argmax(np.abs(grp))
            assert abs(round(deq[j] / s)) == 7


# ------------------------------------------------------------------ top-k / argmax

def test_topk_brute_force_over_all_subsets():
    rng = np.random.default_rng(13)
    for n, k in ((8, 2), (10, 3), (64, 6)):
        for _ in range(20 if n < 64 else 3):
            z = rng.normal(size=n)
            sel = oracle.topk(z, k)
            assert len(set(sel)) == k
            assert list(sel) == sorted(sel, key=lambda i: -z[i])
            if n <= 10:
                best = max(itertools.combinations(range(n), k), key=lambda s: sum(z[i] for i in s))
                assert set(sel) == set(best)
            else:
                assert min(z[sel]) >= max(np.delete(z, sel))


def test_topk_ties_prefer_lower_index():
    np.testing.assert_array_equal(oracle.topk(np.zeros(64), 6), np.arange(6))
    z = np.array([1.0, 3.0, 3.0, 2.0, 3.0])
    np.testing.assert_array_equal(oracle.topk(z, 2), [1, 2])


def test_argmax_ties_lowest_id():
    z = np.array([0.5, 2.0, -1.0, 2.0, 2.0])
    assert oracle.argmax(z) == 1
    assert oracle.argmax(np.zeros(1024)) == 0


# ------------------------------------------------------------------ layers and the model

def _tiny(**kw):
    return synth.CONFIGS["tiny"].replace(**kw)


def _zero(m):
    return {k: np.zeros_like(v) for k, v in m.items()}


def _model(cfg):
    layers = [synth.layer(cfg, l) for l in range(cfg.n_layers)]
    return layers, synth.head(cfg)


def test_swiglu_zero_gate_leaves_residual_unchanged():
    # silu(0) = 0: with the MLP gate weights zero the MLP half adds nothing
    cfg = _tiny(n_layers=1, n_dense_layers=1)
    layers, hw = _model(cfg)
    layers[0]["dense_gate"] = _zero(layers[0]["dense_gate"])
    o1 = oracle.Oracle(cfg, lambda l: layers[l], hw, cap=8)
    layers2 = [dict(layers[0])]
    layers2[0]["dense_down"] = _zero(layers[0]["dense_down"])
    o2 = oracle.Oracle(cfg, lambda l: layers2[l], hw, cap=8)
    t = synth.tokens(cfg, 3)
    np.testing.assert_array_equal(o1.forward(0, t)["x"], o2.forward(0, t)["x"])


def test_whole_model_with_zero_outputs_is_norm_then_lm_head():
    # o_proj and every down projection zero: the residual stays E[t], so the
    # logits are lm_head . rmsnorm(E[t]) (numpy matvec) and the id their argmax
    cfg = _tiny()
    layers, hw = _model(cfg)
    for L in layers:
        L["o"] = _zero(L["o"])
        for name in ("dense_down", "exp_down"):
            if name in L:
                L[name] = _zero(L[name])
    o = oracle.Oracle(cfg, lambda l: layers[l], hw, cap=16)
    t = synth.tokens(cfg, 5, stream=3)
    r = o.forward(0, t)
    E = hw["embed"].astype(np.float64)
    for i, tok in enumerate(t):
        x = E[tok]
        f = x / np.sqrt(np.mean(x * x) + cfg.rms_eps)
        expect = hw["lm_head"].astype(np.float64) @ f
        np.testing.assert_allclose(r["logits"][i], expect, rtol=1e-5, atol=1e-7)
        assert r["ids"][i] == int(np.argmax(expect))


def test_first_token_attention_output_is_its_value_and_gqa_mapping():
    # Position 0 attends only to itself, so o_h = v_{h // (n_q / n_kv)}.  With the
    # embedding row constant the normed input is the constant k = 1/sqrt(1 + eps),
    # so v_j = k * (row sums of W_v), and with W_o = I the residual gains exactly o.
    cfg = _tiny(n_layers=1, n_dense_layers=1)
    layers, hw = _model(cfg)
    L = layers[0]
    H, d, nq, nkv = cfg.hidden, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    assert nq * d == H
    L["o"] = {"w": np.eye(H, dtype=np.float32)}
    L["dense_down"] = _zero(L["dense_down"])
    hw = dict(hw)
    hw["embed"] = hw["embed"].copy()
    hw["embed"][7] = 1.0
    o = oracle.Oracle(cfg, lambda l: layers[l], hw, cap=4)
    x = o.forward(0, np.array([7], np.int32))["x"][0]
    k = 1.0 / math.sqrt(1.0 + cfg.rms_eps)
    wv = L["qkv"]["w"][(nq + nkv) * d:].astype(np.float64)
    v = (k * wv.sum(1).reshape(nkv, d)).astype(np.float32).astype(np.float64)   # the fp32 model caches fp32 V
    group = nq // nkv
    expect = 1.0 + np.concatenate([v[h // group] for h in range(nq)])
    np.testing.assert_allclose(x, expect, rtol=1e-12, atol=1e-12)


def test_kv_append_is_roped_key_at_current_position():
    # the cached key of position p is RoPE(k, p) of the token's projection
    cfg = _tiny(n_layers=1, n_dense_layers=1)
    layers, hw = _model(cfg)
    hw = dict(hw)
    hw["embed"] = hw["embed"].copy()
    hw["embed"][3] = 1.0
    o = oracle.Oracle(cfg, lambda l: layers[l], hw, cap=16)
    o.len[0] = 11                       # resident positions 0..10 (zeros)
    o.forward(0, np.array([3], np.int32))
    H, d, nq, nkv = cfg.hidden, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    k = 1.0 / math.sqrt(1.0 + cfg.rms_eps)
    wk = layers[0]["qkv"]["w"][nq * d:(nq + nkv) * d].astype(np.float64)
    kv = k * wk.sum(1).reshape(nkv, d)
    for j in range(nkv):
        # rotate by hand: pairs (i, i + d/2) by 11 * base^(-2i/d)
        ang = 11 * 1e4 ** (-2.0 * np.arange(d // 2) / d)
        a, b = kv[j, : d // 2], kv[j, d // 2:]
        expect = np.concatenate([a * np.cos(ang) - b * np.sin(ang), b * np.cos(ang) + a * np.sin(ang)])
        np.testing.assert_allclose(o.K[0][0][j, 11], expect, rtol=1e-5, atol=1e-7)
        assert not o.K[0][0][j, 12].any()


def test_moe_with_identical_experts_and_renorm_equals_dense_mlp():
    # renormalised weights sum to 1, so identical experts collapse to one MLP
    base = _tiny(n_layers=1, n_dense_layers=0, router_renorm=1)
    layers, hw = _model(base)
    L = layers[0]
    E = base.n_experts
    for name in ("exp_gate", "exp_up", "exp_down"):
        L[name] = {"w": np.repeat(L[name]["w"][:1], E, axis=0)}
    dense_cfg = base.replace(n_dense_layers=1, dense_inter=base.expert_inter)
    Ld = {k: v for k, v in L.items() if not k.startswith("exp_") and k != "router"}
    Ld["dense_gate"] = {"w": L["exp_gate"]["w"][0]}
    Ld["dense_up"] = {"w": L["exp_up"]["w"][0]}
    Ld["dense_down"] = {"w": L["exp_down"]["w"][0]}
    t = synth.tokens(base, 4)
    a = oracle.Oracle(base, lambda l: L, hw, cap=8).forward(0, t)
    b = oracle.Oracle(dense_cfg, lambda l: Ld, hw, cap=8).forward(0, t)
    np.testing.assert_allclose(a["x"], b["x"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a["route_w"][:, 0].sum(1), 1.0, rtol=1e-6)


def test_zero_router_selects_first_experts_with_uniform_weight():
    cfg = _tiny(n_layers=1, n_dense_layers=0)
    layers, hw = _model(cfg)
    layers[0]["router"] = _zero(layers[0]["router"])
    r = oracle.Oracle(cfg, lambda l: layers[l], hw, cap=8).forward(0, synth.tokens(cfg, 2))
    np.testing.assert_array_equal(r["routes"][:, 0], [[0, 1], [0, 1]])
    np.testing.assert_allclose(r["route_w"][:, 0], 1.0 / cfg.n_experts, rtol=1e-7)
    r2 = oracle.Oracle(cfg.replace(router_renorm=1), lambda l: layers[l], hw, cap=8).forward(0, synth.tokens(cfg, 2))
    np.testing.assert_allclose(r2["route_w"][:, 0], 1.0 / cfg.top_k, rtol=1e-7)


def test_router_weights_are_softmax_probabilities_of_selected():
    cfg = _tiny(n_layers=1, n_dense_layers=0)
    layers, hw = _model(cfg)
    hw = dict(hw)
    hw["embed"] = hw["embed"].copy()
    hw["embed"][5] = 2.0
    # router rows constant per expert: z_e = c_e * sum(b) with b = 2/sqrt(4+eps) * ones
    c = np.array([0.1, 0.7, -0.2, 0.5, 0.3, 0.0, 0.65, -1.0])
    layers[0]["router"] = {"w": np.repeat(c[:, None], cfg.hidden, 1).astype(np.float32)}
    layers[0]["o"] = _zero(layers[0]["o"])
    r = oracle.Oracle(cfg, lambda l: layers[l], hw, cap=4).forward(0, np.array([5], np.int32))
    cf = c.astype(np.float32).astype(np.float64)
    z = cf * cfg.hidden * 2.0 / math.sqrt(4.0 + cfg.rms_eps)
    p = np.exp(z - z.max())
    p /= p.sum()
    np.testing.assert_array_equal(r["routes"][0, 0], [1, 6])
    np.testing.assert_allclose(r["route_w"][0, 0], p[[1, 6]], rtol=1e-6)


def test_block_pass_equals_token_by_token_decode():
    # layer-major over a block == one decode step per position (causality, positions)
    cfg = synth.CONFIGS["tiny"]
    layers, hw = _model(cfg)
    t = synth.tokens(cfg, 9, stream=5)
    a = oracle.Oracle(cfg, lambda l: layers[l], hw, cap=16)
    ra = a.forward(0, t)
    b = oracle.Oracle(cfg, lambda l: layers[l], hw, cap=16)
    logits = [b.forward(0, t[i:i + 1])["logits"][0] for i in range(len(t))]
    np.testing.assert_allclose(ra["logits"], np.stack(logits), rtol=1e-6, atol=1e-7)


def test_route_tie_adoption_rules():
    # experts 2 and 3 tie exactly behind expert 0: the oracle picks {0, 2} (lower
    # index), accepts {0, 3} as a valid top-2 (flag 1) and rejects {6, 7} (flag 2)
    cfg = _tiny(n_layers=1, n_dense_layers=0)
    layers, hw = _model(cfg)
    hw = dict(hw)
    hw["embed"] = hw["embed"].copy()
    hw["embed"][11] = 1.0
    w = layers[0]["router"]["w"].copy()
    w[0], w[2], w[3] = 0.02, 0.01, 0.01
    layers[0]["router"] = {"w": w}
    t = np.array([11], np.int32)
    own = oracle.Oracle(cfg, lambda l: layers[l], hw, cap=4).forward(0, t)
    np.testing.assert_array_equal(own["routes"][0, 0], [0, 2])
    assert own["route_gap"][0, 0] == 0.0
    ref = own["routes"].copy()
    ref[0, 0] = [3, 0]
    r = oracle.Oracle(cfg, lambda l: layers[l], hw, cap=4).forward(0, t, ref_routes=ref, route_margin=1e-3)
    assert r["route_flags"][0, 0] == 1 and set(r["routes"][0, 0]) == {0, 3}
    bad = own["routes"].copy()
    bad[0, 0] = [6, 7]
    r = oracle.Oracle(cfg, lambda l: layers[l], hw, cap=4).forward(0, t, ref_routes=bad, route_margin=1e-3)
    assert r["route_flags"][0, 0] == 2
    np.testing.assert_array_equal(r["routes"][0, 0], [0, 2])
    # with no margin at all an exactly tied set is still a valid top-2 (min in = max out)
    r = oracle.Oracle(cfg, lambda l: layers[l], hw, cap=4).forward(0, t, ref_routes=ref, route_margin=0.0)
    assert r["route_flags"][0, 0] == 1


def test_route_adoption_needs_a_gap_below_the_margin():
    # expert 3's logit 2 % (of max|z|) below expert 2's: swapping them is accepted at a 3 % margin, not at 1 %
    cfg = _tiny(n_layers=1, n_dense_layers=0)
    layers, hw = _model(cfg)
    hw = dict(hw)
    hw["embed"] = hw["embed"].copy()
    hw["embed"][11] = 1.0
    c = np.zeros(cfg.n_experts)
    c[0], c[2], c[3] = 1.0, 0.5, 0.48
    layers[0]["router"] = {"w": np.repeat(c[:, None], cfg.hidden, 1).astype(np.float32)}
    t = np.array([11], np.int32)
    own = oracle.Oracle(cfg, lambda l: layers[l], hw, cap=4).forward(0, t)
    np.testing.assert_array_equal(own["routes"][0, 0], [0, 2])
    assert abs(own["route_gap"][0, 0] - 0.02) < 1e-6
    ref = own["routes"].copy()
    ref[0, 0] = [0, 3]
    for margin, flag in ((0.03, 1), (0.01, 2)):
        r = oracle.Oracle(cfg, lambda l: layers[l], hw, cap=4).forward(0, t, ref_routes=ref, route_margin=margin)
        assert r["route_flags"][0, 0] == flag


# ------------------------------------------------------------------ closed forms of whole layers
# (fp32 models: no bf16 rounding, so each case below is exact up to double rounding)

def _silu(t):
    # the SiLU of the SwiGLU MLP: t * logistic(t), the logistic from scipy
    from scipy.special import expit
    return t * expit(t)


def _one_hot_swiglu(L, I, H, alpha, beta, out_row, prefix="dense_"):
    """gate row 0 = alpha e_0, up row 0 = beta e_1, every other gate/up row 0; down column 0 = e_out_row."""
    g = np.zeros((I, H), np.float32)
    u = np.zeros((I, H), np.float32)
    d = np.zeros((H, I), np.float32)
    g[0, 0], u[0, 1], d[out_row, 0] = alpha, beta, 1.0
    L[prefix + "gate"], L[prefix + "up"], L[prefix + "down"] = {"w": g}, {"w": u}, {"w": d}


def test_swiglu_is_silu_of_gate_times_up():
    # one dense layer, o_proj zero, a constant embedding row c: the post-attention norm output is
    # b = k g (k = c / sqrt(c^2 + eps), g the norm weights).  With gate = alpha e_0 and up = beta e_1 the
    # MLP adds silu(alpha b_0) * beta b_1 to coordinate 5 and nothing elsewhere.  Distinct alpha and beta,
    # both signs of the gate input: swapping gate and up or flipping SiLU's exponent fails this.
    cfg = _tiny(n_layers=1, n_dense_layers=1, norm_sigma=0.1)
    layers, hw = _model(cfg)
    L = layers[0]
    L["o"] = _zero(L["o"])
    H, I = cfg.hidden, cfg.dense_inter
    hw = dict(hw)
    hw["embed"] = hw["embed"].copy()
    c = 0.5
    hw["embed"][9] = c
    g = L["post_norm"].astype(np.float64)
    k = c / math.sqrt(c * c + cfg.rms_eps)
    for alpha, beta in ((3.0, -0.75), (-2.0, 1.25)):
        _one_hot_swiglu(L, I, H, alpha, beta, 5)
        x = oracle.Oracle(cfg, lambda l: layers[l], hw, cap=4).forward(0, np.array([9], np.int32))["x"][0]
        expect = np.full(H, c)
        expect[5] += _silu(alpha * k * g[0]) * beta * k * g[1]
        np.testing.assert_allclose(x, expect, rtol=1e-12, atol=1e-14)


def test_moe_output_is_router_weighted_sum_of_distinct_experts():
    # one MoE layer (8 experts, top-2), o_proj zero, constant embedding row c, norm weights g: b = k g.
    # Router row e = r_e e_0, so z_e = r_e b_0.  Expert e: gate = alpha e_0, up = beta_e e_0, down writes
    # coordinate 10 + e, so its output is y_e = silu(alpha b_0) beta_e b_0 on coordinate 10 + e alone.
    # The layer must add w_e y_e for the two largest z (w = scipy softmax over all 8 logits): a plain
    # average of the experts, or weights renormalised over the pair, fails this.
    cfg = _tiny(n_layers=1, n_dense_layers=0, norm_sigma=0.1)
    layers, hw = _model(cfg)
    L = layers[0]
    L["o"] = _zero(L["o"])
    H, E, I = cfg.hidden, cfg.n_experts, cfg.expert_inter
    r = np.array([0.3, 1.9, -0.4, 0.8, 2.6, 0.1, -1.2, 1.1])
    beta = np.array([0.9, -1.4, 0.6, 1.7, 0.5, -0.8, 1.2, 2.0])
    alpha = 1.5
    L["router"] = {"w": np.zeros((E, H), np.float32)}
    L["router"]["w"][:, 0] = r
    gt, ut, dt = np.zeros((E, I, H), np.float32), np.zeros((E, I, H), np.float32), np.zeros((E, H, I), np.float32)
    for e in range(E):
        gt[e, 0, 0], ut[e, 0, 0], dt[e, 10 + e, 0] = alpha, beta[e], 1.0
    L["exp_gate"], L["exp_up"], L["exp_down"] = {"w": gt}, {"w": ut}, {"w": dt}
    hw = dict(hw)
    hw["embed"] = hw["embed"].copy()
    c = -0.75
    hw["embed"][4] = c
    k = c / math.sqrt(c * c + cfg.rms_eps)
    b0 = k * float(L["post_norm"][0])
    from scipy.special import softmax
    z = r.astype(np.float32).astype(np.float64) * b0
    w = softmax(z)
    top = np.argsort(-z)[:2]
    res = oracle.Oracle(cfg, lambda l: layers[l], hw, cap=4).forward(0, np.array([4], np.int32))
    assert set(res["routes"][0, 0]) == set(top)
    expect = np.full(H, c)
    for e in top:
        expect[10 + e] += w[e] * _silu(alpha * b0) * float(np.float32(beta[e])) * b0
    np.testing.assert_allclose(res["x"][0], expect, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(res["route_w"][0, 0], w[res["routes"][0, 0]], rtol=1e-6)


def test_attention_after_cached_positions_includes_the_new_token():
    # position 5 after five cached positions whose keys are zero (score 0) and whose values are random.
    # The new token's query and key are parallel with q.k / sqrt(d) = 60 (RoPE turns both by the same
    # angles at the same position, so the product is kept): its own value gets all but e^-60 of the weight,
    # so with W_o = I the residual gains exactly v.  Attention over positions 0..4 only would give the
    # mean of the cached values instead.
    cfg = _tiny(n_layers=1, n_dense_layers=1)
    layers, hw = _model(cfg)
    L = layers[0]
    H, d, nq, nkv = cfg.hidden, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    assert nq * d == H
    c = 1.0
    k = c / math.sqrt(c * c + cfg.rms_eps)       # the normed input is k * ones (norm weights 1)
    rng = np.random.default_rng(17)
    t = rng.normal(size=d)
    t *= math.sqrt(60.0 * math.sqrt(d)) / np.linalg.norm(t) / k   # (k t).(k t) / sqrt(d) = 60
    wv = rng.normal(size=(nkv * d,)) * 0.3
    qkv = np.zeros(((nq + 2 * nkv) * d, H), np.float32)
    for h in range(nq):
        qkv[h * d:(h + 1) * d] = np.repeat((t / H)[:, None], H, 1)
    for j in range(nkv):
        qkv[(nq + j) * d:(nq + j + 1) * d] = np.repeat((t / H)[:, None], H, 1)
    qkv[(nq + nkv) * d:] = np.repeat((wv / H)[:, None], H, 1)
    L["qkv"] = {"w": qkv}
    L["o"] = {"w": np.eye(H, dtype=np.float32)}
    L["dense_down"] = _zero(L["dense_down"])
    hw = dict(hw)
    hw["embed"] = hw["embed"].copy()
    hw["embed"][2] = c
    o = oracle.Oracle(cfg, lambda l: layers[l], hw, cap=8)
    cached_v = rng.normal(size=(nkv, 5, d)).astype(np.float32)
    o.set_resident(0, 0, np.zeros((nkv, 5, d), np.float32), cached_v)
    o.len[0] = 5
    x = o.forward(0, np.array([2], np.int32))["x"][0]
    v = (k * qkv[(nq + nkv) * d:].astype(np.float64).sum(1)).reshape(nkv, d).astype(np.float32).astype(np.float64)
    group = nq // nkv
    expect = c + np.concatenate([v[h // group] for h in range(nq)])
    np.testing.assert_allclose(x, expect, rtol=1e-9, atol=1e-9)


def test_norm_weights_layer_by_layer():
    # two dense layers with distinct norm weights (1 + N(0, 0.1) each), a constant embedding row c.
    # Layer 0 adds nothing (o_proj and down zero), so both layers see x = c ones and the input norm output
    # is k g_in,l: the key each layer caches at position 0 (RoPE is the identity there) is W_k,l (k g_in,l),
    # a numpy matvec.  Layer 1's MLP is the one-hot SwiGLU on b = k g_post,1.  The logits are
    # lm_head . (x / rms(x) * g_final).  Taking another layer's or another norm's weights fails this.
    cfg = _tiny(n_layers=2, n_dense_layers=2, norm_sigma=0.1)
    layers, hw = _model(cfg)
    H, I, d, nq, nkv = cfg.hidden, cfg.dense_inter, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    assert not np.array_equal(layers[0]["attn_norm"], layers[1]["attn_norm"])
    for L in layers:
        L["o"] = _zero(L["o"])
    layers[0]["dense_down"] = _zero(layers[0]["dense_down"])
    _one_hot_swiglu(layers[1], I, H, 2.5, -1.125, 3)
    hw = dict(hw)
    hw["embed"] = hw["embed"].copy()
    c = 0.75
    hw["embed"][1] = c
    o = oracle.Oracle(cfg, lambda l: layers[l], hw, cap=4)
    r = o.forward(0, np.array([1], np.int32))
    k = c / math.sqrt(c * c + cfg.rms_eps)
    for l in range(2):
        wk = layers[l]["qkv"]["w"][nq * d:(nq + nkv) * d].astype(np.float64)
        key = (wk @ (k * layers[l]["attn_norm"].astype(np.float64))).astype(np.float32).reshape(nkv, d)
        np.testing.assert_allclose(o.K[l][0][:, 0], key, rtol=1e-6, atol=1e-7)
    g1 = layers[1]["post_norm"].astype(np.float64)
    x = np.full(H, c)
    x[3] += _silu(2.5 * k * g1[0]) * -1.125 * k * g1[1]
    np.testing.assert_allclose(r["x"][0], x, rtol=1e-12, atol=1e-14)
    f = x / np.sqrt(np.mean(x * x) + cfg.rms_eps) * hw["final_norm"].astype(np.float64)
    np.testing.assert_allclose(r["logits"][0], hw["lm_head"].astype(np.float64) @ f, rtol=1e-5, atol=1e-7)
