"""Pins of the oracle's operators against values fixed by the pages and by mathematics.

Nothing here compares the oracle with itself: every check is a hand-worked
value (tests/golden/glm_hand.json), a pure-Python brute force on tiny
inputs, a closed form, a property stated on the pages, or a special case
that reduces to a library routine (torch CPU).
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import ops

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "glm_hand.json")))


# ---------------------------------------------------------------- GLM linear


@pytest.mark.parametrize("case", ["linear_1x1", "linear_2_1_to_1_2"])
def test_glm_linear_hand_values(case):
    g = GOLD[case]
    x = np.array(g["x_r"] + g["x_c"], dtype=float)[None, :]
    y = ops.glm_linear(x, np.array(g["W"], float), np.array(g["b"], float), g["d_in_r"], g["d_out_r"])
    assert y[0, : g["d_out_r"]].tolist() == g["y_r"]
    assert y[0, g["d_out_r"]:].tolist() == g["y_c"]


def _brute_linear(x, W, b, d_in_r, d_out_r):
    n, d_in = x.shape
    d_out = len(W)
    y = [[0.0] * d_out for _ in range(n)]
    for i in range(n):
        for o in range(d_out):
            s = float(b[o])
            for j in range(d_in):
                out_group = 0 if o < d_out_r else 1
                in_group = 0 if j < d_in_r else 1
                if in_group <= out_group:  # M_ij = 1{j <= i}
                    s += float(W[o][j]) * float(x[i][j])
            y[i][o] = s
    return np.array(y)


def test_glm_linear_brute_force():
    rng = np.random.default_rng(1)
    for d_in_r, d_in_c, d_out_r, d_out_c in [(3, 2, 2, 4), (1, 5, 3, 1), (4, 4, 0, 1), (2, 3, 2, 0)]:
        x = rng.standard_normal((5, d_in_r + d_in_c))
        W = rng.standard_normal((d_out_r + d_out_c, d_in_r + d_in_c))
        b = rng.standard_normal(d_out_r + d_out_c)
        got = ops.glm_linear(x, W, b, d_in_r, d_out_r)
        ref = _brute_linear(x, W, b, d_in_r, d_out_r)
        assert np.max(np.abs(got - ref)) <= 1e-12


def test_glm_linear_request_outputs_ignore_candidate_inputs():
    # [R] §2.1 two-group form: f(x_R, x_C) = (f_R(x_R), f_C(x_R, x_C)).
    rng = np.random.default_rng(2)
    d_in_r, d_in_c, d_out_r, d_out_c = 6, 5, 4, 3
    W = rng.standard_normal((d_out_r + d_out_c, d_in_r + d_in_c))
    b = rng.standard_normal(d_out_r + d_out_c)
    x = rng.standard_normal((7, d_in_r + d_in_c))
    x2 = x.copy()
    x2[:, d_in_r:] = rng.standard_normal((7, d_in_c)) * 1e6
    y1 = ops.glm_linear(x, W, b, d_in_r, d_out_r)
    y2 = ops.glm_linear(x2, W, b, d_in_r, d_out_r)
    assert np.array_equal(y1[:, :d_out_r], y2[:, :d_out_r])
    assert not np.allclose(y1[:, d_out_r:], y2[:, d_out_r:])


def test_glm_linear_planted_unmasked_weight_is_caught():
    # Planted mistake: skip the mask.  The invariance check above must fail.
    rng = np.random.default_rng(3)
    W = rng.standard_normal((5, 6))
    x = rng.standard_normal((4, 6))
    x2 = x.copy()
    x2[:, 3:] += 1.0
    y1 = ops.glm_linear(x, W, None, 3, 2, mask=False)
    y2 = ops.glm_linear(x2, W, None, 3, 2, mask=False)
    assert not np.array_equal(y1[:, :2], y2[:, :2])


def test_glm_linear_two_tower_special_case():
    # W_CR = 0 leaves two independent maps (two-tower case, [R] §1).
    rng = np.random.default_rng(4)
    W = rng.standard_normal((7, 9))
    W[3:, :4] = 0.0
    x = rng.standard_normal((6, 9))
    y = ops.glm_linear(x, W, None, 4, 3)
    assert np.allclose(y[:, :3], x[:, :4] @ W[:3, :4].T, atol=1e-12)
    assert np.allclose(y[:, 3:], x[:, 4:] @ W[3:, 4:].T, atol=1e-12)


def test_decomposed_form_equals_dense_masked_form():
    # [R] §2.4: Y_C[i] = Z[m_i] + W_CC X_C[i] equals the dense masked layer on the broadcast input.
    rng = np.random.default_rng(5)
    B, counts = 4, [3, 0, 5, 1]
    cand2req = np.repeat(np.arange(B), counts)
    d_in_r, d_in_c, d_out_r, d_out_c = 5, 3, 4, 6
    W = rng.standard_normal((d_out_r + d_out_c, d_in_r + d_in_c))
    b = rng.standard_normal(d_out_r + d_out_c)
    x_r = rng.standard_normal((B, d_in_r))
    x_c = rng.standard_normal((len(cand2req), d_in_c))
    y_r, y_c = ops.decomposed_linear(x_r, x_c, cand2req, W, b, d_in_r, d_out_r)
    dense = ops.glm_linear(np.concatenate([x_r[cand2req], x_c], 1), W, b, d_in_r, d_out_r)
    assert np.max(np.abs(dense[:, d_out_r:] - y_c)) <= 1e-12
    assert np.max(np.abs(dense[:, :d_out_r] - y_r[cand2req])) <= 1e-12


# ---------------------------------------------------------------- group norm


def test_layernorm_hand_values():
    g = GOLD["layernorm"]
    y = ops.group_norm(np.array([g["x"]], float), g["widths"], "layer", g["eps"])
    assert np.max(np.abs(y[0] - np.array(g["y"]))) <= 1e-15


def test_rmsnorm_hand_values():
    g = GOLD["rmsnorm"]
    y = ops.group_norm(np.array([g["x"]], float), g["widths"], "rms", g["eps"])
    assert np.max(np.abs(y[0] - np.array(g["y"]))) <= 1e-15


def test_group_norm_closed_form_moments():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((8, 5 + 11)) * 3 + 1
    eps = 0.37
    y = ops.group_norm(x, [5, 11], "layer", eps)
    for sl in (slice(0, 5), slice(5, 16)):
        xs, ys = x[:, sl], y[:, sl]
        var = xs.var(axis=1)
        assert np.allclose(ys.mean(axis=1), 0, atol=1e-13)
        assert np.allclose(ys.var(axis=1), var / (var + eps), rtol=1e-12)
    y = ops.group_norm(x, [5, 11], "rms", eps)
    for sl in (slice(0, 5), slice(5, 16)):
        ms = (x[:, sl] ** 2).mean(axis=1)
        assert np.allclose((y[:, sl] ** 2).mean(axis=1), ms / (ms + eps), rtol=1e-12)
    # constant row -> zero under LayerNorm
    c = np.full((1, 7), 4.25)
    assert np.array_equal(ops.group_norm(c, [7], "layer", 1e-5), np.zeros((1, 7)))


def test_group_norm_matches_torch_per_slice():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    x = rng.standard_normal((9, 12 + 20))
    gam = [rng.standard_normal(12), rng.standard_normal(20)]
    bet = [rng.standard_normal(12), rng.standard_normal(20)]
    y = ops.group_norm(x, [12, 20], "layer", 1e-5, gam, bet)
    t = torch.from_numpy(x)
    ref0 = torch.nn.functional.layer_norm(t[:, :12], (12,), torch.from_numpy(gam[0]), torch.from_numpy(bet[0]), 1e-5)
    ref1 = torch.nn.functional.layer_norm(t[:, 12:], (20,), torch.from_numpy(gam[1]), torch.from_numpy(bet[1]), 1e-5)
    assert np.max(np.abs(y - torch.cat([ref0, ref1], 1).numpy())) <= 1e-12
    y = ops.group_norm(x, [12, 20], "rms", 1e-5, gam, None)
    r0 = torch.nn.functional.rms_norm(t[:, :12], (12,), torch.from_numpy(gam[0]), 1e-5)
    r1 = torch.nn.functional.rms_norm(t[:, 12:], (20,), torch.from_numpy(gam[1]), 1e-5)
    assert np.max(np.abs(y - torch.cat([r0, r1], 1).numpy())) <= 1e-12


def test_group_norm_is_group_local():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((4, 10))
    x2 = x.copy()
    x2[:, 6:] *= 50.0
    y1 = ops.group_norm(x, [6, 4], "layer")
    y2 = ops.group_norm(x2, [6, 4], "layer")
    assert np.array_equal(y1[:, :6], y2[:, :6])


# ---------------------------------------------------------------- masked FM


def test_fm_hand_values():
    g = GOLD["fm"]
    X = np.array([g["X_r"] + g["X_c"]], float)
    f_r, f_c = ops.masked_fm(X, g["n_r"])
    assert f_r[0].tolist() == g["f_r"]
    assert f_c[0].tolist() == g["f_c"]


def test_fm_brute_force_and_properties():
    rng = np.random.default_rng(9)
    n_r, n_c, D = 3, 2, 4
    X = rng.standard_normal((3, n_r + n_c, D))
    f_r, f_c = ops.masked_fm(X, n_r)
    for i in range(3):
        for a in range(n_r):
            for b in range(n_r):
                assert abs(f_r[i, a * n_r + b] - sum(X[i, a, e] * X[i, b, e] for e in range(D))) <= 1e-12
        for a in range(n_c):
            for b in range(n_r + n_c):
                ref = sum(X[i, n_r + a, e] * X[i, b, e] for e in range(D))
                assert abs(f_c[i, a * (n_r + n_c) + b] - ref) <= 1e-12
    # request block is symmetric
    Fr = f_r.reshape(3, n_r, n_r)
    assert np.array_equal(Fr, Fr.transpose(0, 2, 1))
    # no candidate tokens: plain X X^T
    f_r0, f_c0 = ops.masked_fm(X[:, :n_r], n_r)
    assert f_c0.shape == (3, 0)
    assert np.allclose(f_r0.reshape(3, n_r, n_r), np.einsum("nad,nbd->nab", X[:, :n_r], X[:, :n_r]), atol=1e-12)
    # request outputs ignore candidate tokens
    X2 = X.copy()
    X2[:, n_r:] += 7.0
    assert np.array_equal(ops.masked_fm(X2, n_r)[0], f_r)


# ---------------------------------------------------------------- token LCB


def test_token_lcb_hand_values():
    g = GOLD["token_lcb"]
    X = np.array([g["X_r"] + g["X_c"]], float)
    t_r, t_c = ops.token_lcb(X, np.array(g["W"], float), g["n_r"], g["t_r"])
    assert t_r[0].tolist() == g["T_r"]
    assert t_c[0].tolist() == g["T_c"]


def test_token_lcb_brute_force():
    rng = np.random.default_rng(10)
    n_r, n_c, t_r, t_c, D = 3, 2, 2, 4, 5
    X = rng.standard_normal((2, n_r + n_c, D))
    W = rng.standard_normal((t_r + t_c, n_r + n_c))
    T_r, T_c = ops.token_lcb(X, W, n_r, t_r)
    for i in range(2):
        for t in range(t_r + t_c):
            for e in range(D):
                s = 0.0
                for a in range(n_r + n_c):
                    if (a < n_r) or (t >= t_r):
                        s += W[t, a] * X[i, a, e]
                got = T_r[i, t * D + e] if t < t_r else T_c[i, (t - t_r) * D + e]
                assert abs(got - s) <= 1e-12


# ---------------------------------------------------------------- attention


def test_attention_single_key_returns_value():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((3, 4, 8))
    K = rng.standard_normal((3, 1, 8))
    V = rng.standard_normal((3, 1, 8))
    a = ops.attention(q, K, V, n_heads=2)
    assert np.allclose(a, np.broadcast_to(V, a.shape), atol=1e-15)


def test_attention_equal_scores_give_mean_value():
    rng = np.random.default_rng(12)
    V = rng.standard_normal((2, 5, 8))
    K = np.broadcast_to(rng.standard_normal((2, 1, 8)), (2, 5, 8)).copy()
    q = rng.standard_normal((2, 3, 8))
    a = ops.attention(q, K, V, n_heads=2)
    assert np.allclose(a, np.broadcast_to(V.mean(axis=1, keepdims=True), a.shape), atol=1e-13)
    a0 = ops.attention(np.zeros_like(q), rng.standard_normal((2, 5, 8)), V, n_heads=2)
    assert np.allclose(a0, np.broadcast_to(V.mean(axis=1, keepdims=True), a0.shape), atol=1e-13)


def test_attention_dominant_key():
    rng = np.random.default_rng(13)
    K = rng.standard_normal((1, 6, 4)) * 0.01
    K[0, 4] = [100.0, 0, 0, 0]
    V = rng.standard_normal((1, 6, 4))
    q = np.array([[[100.0, 0, 0, 0]]])
    a = ops.attention(q, K, V, n_heads=1)
    assert np.allclose(a[0, 0], V[0, 4], atol=1e-12)


def test_attention_brute_force_and_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(14)
    n, Lq, Lk, H, dh = 2, 3, 7, 2, 4
    q = rng.standard_normal((n, Lq, H * dh))
    K = rng.standard_normal((n, Lk, H * dh))
    V = rng.standard_normal((n, Lk, H * dh))
    a = ops.attention(q, K, V, n_heads=H)
    for i in range(n):
        for t in range(Lq):
            for h in range(H):
                s = [sum(q[i, t, h * dh + e] * K[i, k, h * dh + e] for e in range(dh)) / math.sqrt(dh) for k in range(Lk)]
                mx = max(s)
                p = [math.exp(v - mx) for v in s]
                z = sum(p)
                for e in range(dh):
                    ref = sum(p[k] / z * V[i, k, h * dh + e] for k in range(Lk))
                    assert abs(a[i, t, h * dh + e] - ref) <= 1e-12
    tq = torch.from_numpy(q).view(n, Lq, H, dh).transpose(1, 2)
    tk = torch.from_numpy(K).view(n, Lk, H, dh).transpose(1, 2)
    tv = torch.from_numpy(V).view(n, Lk, H, dh).transpose(1, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).transpose(1, 2).reshape(n, Lq, H * dh)
    assert np.max(np.abs(a - ref.numpy())) <= 1e-12


# ---------------------------------------------------------------- encoder


def test_encoder_layer_matches_torch_transformer_layer():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(15)
    d, H, f, L, n = 16, 4, 32, 9, 2
    p = {
        "w_qkv": rng.standard_normal((3 * d, d)) / 4, "b_qkv": rng.standard_normal(3 * d) * 0.1,
        "w_o": rng.standard_normal((d, d)) / 4, "b_o": rng.standard_normal(d) * 0.1,
        "w_1": rng.standard_normal((f, d)) / 4, "b_1": rng.standard_normal(f) * 0.1,
        "w_2": rng.standard_normal((d, f)) / 6, "b_2": rng.standard_normal(d) * 0.1,
    }
    S = rng.standard_normal((n, L, d))
    got = ops.encoder_layer(S, p, H, eps=1e-5)
    layer = torch.nn.TransformerEncoderLayer(d, H, f, dropout=0.0, activation="relu", batch_first=True,
                                             norm_first=False, layer_norm_eps=1e-5, dtype=torch.float64)
    layer.eval()
    with torch.no_grad():
        layer.self_attn.in_proj_weight.copy_(torch.from_numpy(p["w_qkv"]))
        layer.self_attn.in_proj_bias.copy_(torch.from_numpy(p["b_qkv"]))
        layer.self_attn.out_proj.weight.copy_(torch.from_numpy(p["w_o"]))
        layer.self_attn.out_proj.bias.copy_(torch.from_numpy(p["b_o"]))
        layer.linear1.weight.copy_(torch.from_numpy(p["w_1"]))
        layer.linear1.bias.copy_(torch.from_numpy(p["b_1"]))
        layer.linear2.weight.copy_(torch.from_numpy(p["w_2"]))
        layer.linear2.bias.copy_(torch.from_numpy(p["b_2"]))
        ref = layer(torch.from_numpy(S)).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-10
