"""Oracle for the UG-Separation TokenMixer layer, float64 numpy.

TEST INFRASTRUCTURE ONLY (same rule as the rest of this package): only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.

Citation: [U] "Compute Only Once: UG-Separation for Efficient Large
Recommendation Models" (xllm-io paper review), §3 technical architecture:
the framework tree, the core formulas (TokenMixer layer, token
concatenation, separation mask, information compensation) and the mask
picture.

What it computes, sample by sample and with nothing shared: one sample is
the token matrix X = [x_u0 .. x_u(n_u-1), x_g0 .. x_g(n_g-1)] of T = n_u +
n_g tokens of width D.  For a candidate i of request m_i the U tokens are
the request's and the G tokens the candidate's ([U] §3 token concatenation:
U tokens are purely user-side, G tokens mix user and item).  A layer is

    X'  = X with G replaced by G + P U                (compensation, U3)
    Pm  = LN1(Mixup_UG(X'))                           (U2, U4)
    X_k = LN2(PFFN(Pm) + X')                          (U5, U6)

Readings of the page (where it is silent or contradicts itself):

U1  Mask direction.  The framework tree blocks G -> U (a group token may not
    affect a user token); the mask formula zeroes the pair (i in G, j in U),
    read as source i, destination j, which says the same.  The mask
    picture's caption ("U can attend to all, G cannot attend to U") would
    make U depend on candidates and defeat the reuse the page is about, so
    it is read with the tree: U outputs read U inputs only, G outputs read
    everything.
U2  Mixup is multi-head token mixing with as many heads as tokens: each
    token is cut into T chunks of width c = D / T, and output token h is the
    concatenation over input tokens t (in order) of chunk h of token t.  The
    UG mask zeroes, in U outputs, the chunks that come from G tokens.  A
    G input's chunks h < n_u are therefore read by no output.
U3  Compensation G_comp = G + Proj(U) is taken as a learned token-axis map
    P in R^{n_g x n_u}: G slot g receives sum_u P[g, u] U_u.  It depends on
    the request only.  It replaces G in the layer input, so the Mixup and
    the residual both see G_comp.  It is optional (P = None).
U4  LN is LayerNorm over the D features of one token (biased variance, eps
    inside the root), gamma and beta shared by all tokens of a layer.
U5  PFFN has per-token weights: F_t = W2_t act(W1_t Pm_t + b1_t) + b2_t.
    The activation is not stated; ReLU is taken.
U6  Separated residual: output token h adds input token h, so the U side's
    residual never reads a G token.

Pins (tests/test_oracle_ugsep.py): Mixup against numpy's reshape-transpose
of the chunk grid (unmasked, and all-U), the involution of the unmasked
Mixup, hand-worked masked values, a pure-Python scalar brute force of the
whole layer (every index from the definitions above), invariance of U
outputs to G inputs with a planted unmasked control, the compensation's
hand values and special cases, the residual-only closed form against
torch's CPU layer_norm, and request outputs that agree across all of a
request's candidates.
"""

from __future__ import annotations

from typing import Any, Dict, Optional, Sequence

import numpy as np

from . import ops

F64 = np.float64


def ug_reads(n_u: int, n_g: int) -> np.ndarray:
    """A[h, t] = 1 when output token h may read input token t (U1).

    Only U outputs reading G inputs are blocked.
    """
    T = n_u + n_g
    A = np.ones((T, T), dtype=F64)
    A[:n_u, n_u:] = 0.0
    return A


def mixup(X: np.ndarray, n_u: int, mask: bool = True) -> np.ndarray:
    """Multi-head token mixing under the UG mask (U1, U2).  X [..., T, D].

    ``mask=False`` exists so that tests can plant the unmasked mistake and
    check that the invariance test catches it.
    """
    X = np.asarray(X, dtype=F64)
    T, D = X.shape[-2], X.shape[-1]
    assert D % T == 0, "D must be a multiple of the token count"
    c = D // T
    A = ug_reads(n_u, T - n_u) if mask else np.ones((T, T), dtype=F64)
    out = np.zeros_like(X)
    for h in range(T):
        for t in range(T):
            out[..., h, t * c:(t + 1) * c] = A[h, t] * X[..., t, h * c:(h + 1) * c]
    return out


def compensation(U: np.ndarray, P) -> Optional[np.ndarray]:
    """Proj(U) = P U along the token axis (U3).  U [..., n_u, D] -> [..., n_g, D]."""
    if P is None:
        return None
    return np.matmul(np.asarray(P, dtype=F64), np.asarray(U, dtype=F64))


def compensate(X: np.ndarray, n_u: int, P) -> np.ndarray:
    """X with its G tokens replaced by G + P U (U3)."""
    X = np.array(X, dtype=F64)
    comp = compensation(X[..., :n_u, :], P)
    if comp is not None:
        X[..., n_u:, :] += comp
    return X


def layer_norm(x: np.ndarray, gamma, beta, eps: float) -> np.ndarray:
    """LayerNorm over the last axis (one token's D features, U4)."""
    return ops.group_norm(x, [np.shape(x)[-1]], "layer", eps, [gamma], [beta])


def pffn(Pm: np.ndarray, w1, b1, w2, b2) -> np.ndarray:
    """Per-token FFN (U5).  Pm [..., T, D]; w1 [T, H, D]; b1 [T, H]; w2 [T, D, H]; b2 [T, D]."""
    Pm = np.asarray(Pm, dtype=F64)
    out = np.empty_like(Pm)
    for t in range(Pm.shape[-2]):
        h = ops.relu(Pm[..., t, :] @ np.asarray(w1[t], dtype=F64).T + np.asarray(b1[t], dtype=F64))
        out[..., t, :] = h @ np.asarray(w2[t], dtype=F64).T + np.asarray(b2[t], dtype=F64)
    return out


def tokenmixer_layer(X: np.ndarray, p: Dict[str, Any], n_u: int, eps: float, mask: bool = True) -> np.ndarray:
    """One TokenMixer layer with UG separation ([U] §3 core formulas; U1-U6)."""
    Xc = compensate(X, n_u, p.get("comp"))
    Pm = layer_norm(mixup(Xc, n_u, mask), p["ln1_g"], p["ln1_b"], eps)
    return layer_norm(pffn(Pm, p["w1"], p["b1"], p["w2"], p["b2"]) + Xc, p["ln2_g"], p["ln2_b"], eps)


def tokenmixer(X: np.ndarray, layers: Sequence[Dict[str, Any]], n_u: int, eps: float, mask: bool = True) -> np.ndarray:
    for p in layers:
        X = tokenmixer_layer(X, p, n_u, eps, mask)
    return X


def with_u_w8a16(layers: Sequence[Dict[str, Any]], quant: Sequence[Dict[str, Any]], n_u: int) -> list:
    """Layers whose U tokens' FFN weights are the dequantized 8-bit weights
    ([U] §3 framework tree stage 4 and the W8A16 configuration; readings
    W1-W2 of the W8A16 oracle): token t < n_u uses
    W1_t = w1_scale[t] * fp8(w1_q[t]) and W2_t = w2_scale[t] * fp8(w2_q[t]);
    the G tokens keep their weights.  The layer itself is unchanged, so the
    result is the TokenMixer of ``tokenmixer`` with these weights."""
    from . import w8a16

    out = []
    for p, q in zip(layers, quant):
        r = dict(p)
        w1 = np.array(p["w1"], dtype=F64)
        w2 = np.array(p["w2"], dtype=F64)
        for t in range(n_u):
            w1[t] = w8a16.dequantize(q["w1_q"][t], q["w1_scale"][t])
            w2[t] = w8a16.dequantize(q["w2_q"][t], q["w2_scale"][t])
        r["w1"], r["w2"] = w1, w2
        out.append(r)
    return out


def ugsep_forward(inputs: Dict[str, Any], candidates=None, requests=None) -> Dict[str, np.ndarray]:
    """Stack outputs for the listed candidates and requests (default: all).

    Each candidate is evaluated alone on its own concatenation [U of its
    request ; its G tokens].  A request's U outputs are evaluated with zero
    G tokens: under U1 and U6 they do not depend on the G tokens, which the
    pins check on whole candidates.
    """
    n_u, n_g = int(inputs["n_u"]), int(inputs["n_g"])
    layers, eps = inputs["layers"], float(inputs["eps"])
    x_u = np.asarray(inputs["x_u"], dtype=F64)
    x_g = np.asarray(inputs["x_g"], dtype=F64)
    c2r = np.asarray(inputs["cand2req"], dtype=np.int64)
    cand = np.arange(x_g.shape[0]) if candidates is None else np.asarray(candidates, dtype=np.int64)
    req = np.arange(x_u.shape[0]) if requests is None else np.asarray(requests, dtype=np.int64)
    D = x_u.shape[-1] if n_u > 0 else x_g.shape[-1]
    Xc = np.concatenate([x_u[c2r[cand]], x_g[cand]], axis=1) if cand.size else np.zeros((0, n_u + n_g, D))
    Xr = np.concatenate([x_u[req], np.zeros((req.size, n_g, D))], axis=1)
    y_c = tokenmixer(Xc, layers, n_u, eps)
    y_r = tokenmixer(Xr, layers, n_u, eps)
    return {"y_g": y_c[:, n_u:, :], "y_u": y_r[:, :n_u, :], "y_g_u": y_c[:, :n_u, :]}
