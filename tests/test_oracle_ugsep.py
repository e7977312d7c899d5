"""Pins of the UG-Separation TokenMixer oracle (CPU only).

Citation: "Compute Only Once: UG-Separation for Efficient Large
Recommendation Models" (xllm-io review), §3 core formulas and separation
mask.  Each pin checks the oracle against something other than itself: a
numpy or torch library route, hand-worked values, a closed form, an
invariant, or a pure-Python scalar brute force written from the
definitions.
"""

import math

import numpy as np
import pytest

import rocs_synth as S
from oracle import ugsep as U


def _rng(seed=0):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ Mixup

@pytest.mark.parametrize("T,c", [(2, 3), (4, 2), (5, 4)])
def test_unmasked_mixup_is_the_chunk_grid_transpose(T, c):
    X = _rng(T).standard_normal((3, T, T * c))
    grid = X.reshape(3, T, T, c).swapaxes(1, 2).reshape(3, T, T * c)
    np.testing.assert_array_equal(U.mixup(X, 0), grid)  # no U tokens: nothing masked
    np.testing.assert_array_equal(U.mixup(X, T), grid)  # no G tokens: nothing masked


def test_unmasked_mixup_is_an_involution():
    X = _rng(1).standard_normal((2, 6, 18))
    np.testing.assert_array_equal(U.mixup(U.mixup(X, 0), 0), X)


def test_mixup_hand_values():
    X = np.array([[1.0, 2.0], [3.0, 4.0]])  # token 0 = U, token 1 = G, chunk width 1
    np.testing.assert_array_equal(U.mixup(X, 0), [[1, 3], [2, 4]])
    np.testing.assert_array_equal(U.mixup(X, 1), [[1, 0], [2, 4]])
    np.testing.assert_array_equal(U.mixup(X, 1, mask=False), [[1, 3], [2, 4]])


def test_mixup_mask_zeroes_exactly_the_g_chunks_of_u_outputs():
    n_u, n_g, c = 3, 2, 4
    T = n_u + n_g
    X = _rng(2).standard_normal((T, T * c)) + 10.0  # no accidental zeros
    out = U.mixup(X, n_u)
    full = U.mixup(X, n_u, mask=False)
    for h in range(T):
        for t in range(T):
            blk = out[h, t * c:(t + 1) * c]
            if h < n_u and t >= n_u:
                assert np.all(blk == 0.0)
            else:
                np.testing.assert_array_equal(blk, full[h, t * c:(t + 1) * c])


# ------------------------------------------------------------------ compensation

def test_compensation_hand_values():
    X = np.array([[1.0, 2.0], [10.0, 20.0]])
    np.testing.assert_array_equal(U.compensate(X, 1, np.array([[2.0]])), [[1, 2], [12, 24]])
    X = np.array([[1.0, 2.0], [3.0, 5.0], [0.0, 0.0]])
    np.testing.assert_array_equal(U.compensate(X, 2, np.array([[1.0, -1.0]])), [[1, 2], [3, 5], [-2, -3]])


def test_compensation_special_cases():
    r = _rng(3)
    X = r.standard_normal((4, 5, 10))
    P = r.standard_normal((3, 2))
    np.testing.assert_array_equal(U.compensate(X, 2, None), X)
    np.testing.assert_array_equal(U.compensate(X, 2, np.zeros((3, 2))), X)
    X0 = X.copy()
    X0[:, :2] = 0.0
    np.testing.assert_array_equal(U.compensate(X0, 2, P), X0)  # no U information, nothing added
    np.testing.assert_array_equal(U.compensate(X, 2, P)[:, :2], X[:, :2])  # U tokens untouched


# ------------------------------------------------------------------ whole layer

def _tiny_params(rng, T, n_u, D, H, comp=True):
    return {
        "comp": rng.standard_normal((T - n_u, n_u)) if comp else None,
        "ln1_g": 1 + 0.1 * rng.standard_normal(D), "ln1_b": 0.1 * rng.standard_normal(D),
        "w1": rng.standard_normal((T, H, D)), "b1": rng.standard_normal((T, H)),
        "w2": rng.standard_normal((T, D, H)), "b2": rng.standard_normal((T, D)),
        "ln2_g": 1 + 0.1 * rng.standard_normal(D), "ln2_b": 0.1 * rng.standard_normal(D),
    }


def _brute_layer(X, p, n_u, eps):
    """Scalar loops straight from the definitions (no numpy arithmetic)."""
    T, D = len(X), len(X[0])
    c, H = D // T, len(p["b1"][0])
    Xc = [[float(v) for v in row] for row in X]
    if p["comp"] is not None:
        for g in range(T - n_u):
            for e in range(D):
                s = 0.0
                for u in range(n_u):
                    s += float(p["comp"][g][u]) * float(X[u][e])
                Xc[n_u + g][e] = float(X[n_u + g][e]) + s
    mixed = [[0.0] * D for _ in range(T)]
    for h in range(T):
        for e in range(D):
            t, o = divmod(e, c)
            mixed[h][e] = 0.0 if (h < n_u <= t) else Xc[t][h * c + o]

    def ln(row, g, b):
        mu = sum(row) / len(row)
        var = sum((v - mu) ** 2 for v in row) / len(row)
        return [(v - mu) / math.sqrt(var + eps) * float(g[k]) + float(b[k]) for k, v in enumerate(row)]

    P = [ln(mixed[h], p["ln1_g"], p["ln1_b"]) for h in range(T)]
    out = []
    for t in range(T):
        hid = [max(0.0, sum(float(p["w1"][t][j][k]) * P[t][k] for k in range(D)) + float(p["b1"][t][j])) for j in range(H)]
        f = [sum(float(p["w2"][t][e][j]) * hid[j] for j in range(H)) + float(p["b2"][t][e]) for e in range(D)]
        out.append(ln([f[e] + Xc[t][e] for e in range(D)], p["ln2_g"], p["ln2_b"]))
    return np.array(out)


@pytest.mark.parametrize("n_u,n_g,c,H,comp", [(1, 2, 2, 4, True), (2, 1, 1, 3, True), (2, 2, 2, 5, False), (0, 3, 1, 2, False)])
def test_layer_matches_scalar_brute_force(n_u, n_g, c, H, comp):
    r = _rng(10 + n_u * 7 + n_g)
    T = n_u + n_g
    D = T * c
    p = _tiny_params(r, T, n_u, D, H, comp and n_u > 0)
    X = r.standard_normal((T, D))
    got = U.tokenmixer_layer(X, p, n_u, 1e-5)
    np.testing.assert_allclose(got, _brute_layer(X, p, n_u, 1e-5), rtol=0, atol=1e-11)


def test_residual_only_layer_is_torch_layer_norm():
    torch = pytest.importorskip("torch")
    r = _rng(4)
    T, n_u, D, H = 4, 2, 8, 6
    p = _tiny_params(r, T, n_u, D, H, comp=False)
    p["w2"] = np.zeros_like(p["w2"])
    p["b2"] = np.zeros_like(p["b2"])
    X = r.standard_normal((3, T, D))
    ref = torch.nn.functional.layer_norm(torch.tensor(X), (D,), torch.tensor(p["ln2_g"]), torch.tensor(p["ln2_b"]), 1e-5)
    np.testing.assert_allclose(U.tokenmixer_layer(X, p, n_u, 1e-5), ref.numpy(), rtol=0, atol=1e-12)


def test_pffn_uses_each_tokens_own_weights():
    r = _rng(5)
    T, D, H = 3, 6, 4
    Pm = r.standard_normal((2, T, D))
    w1, b1 = r.standard_normal((T, H, D)), r.standard_normal((T, H))
    w2, b2 = r.standard_normal((T, D, H)), r.standard_normal((T, D))
    out = U.pffn(Pm, w1, b1, w2, b2)
    for t in range(T):
        ref = np.maximum(Pm[:, t] @ w1[t].T + b1[t], 0.0) @ w2[t].T + b2[t]
        np.testing.assert_allclose(out[:, t], ref, rtol=0, atol=1e-12)
    perm = [2, 0, 1]  # permuting tokens and their weights together permutes the outputs
    out_p = U.pffn(Pm[:, perm], w1[perm], b1[perm], w2[perm], b2[perm])
    np.testing.assert_allclose(out_p, out[:, perm], rtol=0, atol=1e-12)


# ------------------------------------------------------------------ separation invariance

def test_u_outputs_do_not_depend_on_g_inputs():
    r = _rng(6)
    n_u, n_g, c, H = 2, 3, 2, 4
    T, D = n_u + n_g, (n_u + n_g) * c
    layers = [_tiny_params(r, T, n_u, D, H) for _ in range(3)]
    X = r.standard_normal((4, T, D))
    X2 = X.copy()
    X2[:, n_u:] = r.standard_normal((4, n_g, D)) * 3.0
    a, b = U.tokenmixer(X, layers, n_u, 1e-5), U.tokenmixer(X2, layers, n_u, 1e-5)
    np.testing.assert_array_equal(a[:, :n_u], b[:, :n_u])
    assert np.max(np.abs(a[:, n_u:] - b[:, n_u:])) > 1e-3
    # planted control: the unmasked mixing lets G reach U, and the check sees it
    a, b = U.tokenmixer(X, layers, n_u, 1e-5, mask=False), U.tokenmixer(X2, layers, n_u, 1e-5, mask=False)
    assert np.max(np.abs(a[:, :n_u] - b[:, :n_u])) > 1e-3


def test_forward_request_outputs_agree_with_every_candidate():
    inp = S.make_ugsep_inputs(S.ugsep_config("small", "f32"), seed=5)
    out = U.ugsep_forward(inp)
    np.testing.assert_allclose(out["y_g_u"], out["y_u"][inp["cand2req"]], rtol=0, atol=1e-12)
    assert out["y_g"].shape == (len(inp["cand2req"]), 5, 64)


def test_forward_subsets_match_the_whole_batch():
    inp = S.make_ugsep_inputs(S.ugsep_config("tiny", "f32"), seed=6)
    full = U.ugsep_forward(inp)
    cand, req = [3, 0, 7], [2, 1]
    part = U.ugsep_forward(inp, candidates=cand, requests=req)
    np.testing.assert_array_equal(part["y_g"], full["y_g"][cand])
    np.testing.assert_array_equal(part["y_u"], full["y_u"][req])


# ------------------------------------------------------------------ U side on 8-bit weights

def test_u_w8a16_substitution_with_hand_decoded_codes():
    """with_u_w8a16 against weights written out by hand from the E4M3
    format: 0x38 = +1 (exponent field 7 = bias, mantissa 0), 0xB8 = -1,
    0x40 = +2, 0x30 = +0.5, 0x01 = 2^-9 (smallest subnormal).  The U tokens
    take scale x those values; the G tokens keep their weights."""
    cfg = S.UgsepConfig("w8pin", 2, ("fixed", 2), 2, 2, 8, 6, 1, True, "f32")
    inp = S.make_ugsep_inputs(cfg, seed=31)
    rng = _rng(5)
    table = {0x38: 1.0, 0xB8: -1.0, 0x40: 2.0, 0x30: 0.5, 0x01: 2.0 ** -9}
    keys = np.array(list(table), dtype=np.uint8)
    q1 = keys[rng.integers(0, len(keys), (2, 6, 8))]
    q2 = keys[rng.integers(0, len(keys), (2, 8, 6))]
    s1, s2 = rng.uniform(0.5, 1.5, (2, 6)), rng.uniform(0.5, 1.5, (2, 8))
    quant = [dict(w1_q=q1, w1_scale=s1, w2_q=q2, w2_scale=s2)]
    lay = U.with_u_w8a16(inp["layers"], quant, 2)[0]
    hand1 = np.vectorize(table.get)(q1) * s1[:, :, None]
    hand2 = np.vectorize(table.get)(q2) * s2[:, :, None]
    np.testing.assert_array_equal(lay["w1"][:2], hand1)
    np.testing.assert_array_equal(lay["w2"][:2], hand2)
    np.testing.assert_array_equal(lay["w1"][2:], inp["layers"][0]["w1"][2:])
    np.testing.assert_array_equal(lay["w2"][2:], inp["layers"][0]["w2"][2:])
    for k in ("b1", "b2", "ln1_g", "ln2_b", "comp"):
        np.testing.assert_array_equal(lay[k], inp["layers"][0][k])
    # and the layer with them is the layer with the hand weights
    hand = dict(inp["layers"][0])
    hand["w1"] = np.concatenate([hand1, inp["layers"][0]["w1"][2:]])
    hand["w2"] = np.concatenate([hand2, inp["layers"][0]["w2"][2:]])
    a = U.ugsep_forward(dict(inp, layers=[lay]))
    b = U.ugsep_forward(dict(inp, layers=[hand]))
    np.testing.assert_array_equal(a["y_g"], b["y_g"])
    np.testing.assert_array_equal(a["y_u"], b["y_u"])
