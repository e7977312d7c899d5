"""Oracle operators, float64 numpy.  Test infrastructure only (see package header).

Each operator acts on the per-candidate *dense* state: for candidate i the
state row is the concatenation [request part ; candidate part] of one
early-fused model evaluation.  Request parts are carried per candidate (a
materialized broadcast); nothing here shares work across candidates.

Pins (tests/test_oracle_ops.py):
  glm_linear      hand-worked small-integer values, pure-Python brute force,
                  two-group invariance, planted unmasked-weight control,
                  decomposed (IKBO) identity
  group_norm      hand values, closed-form moments, torch CPU layer_norm /
                  rms_norm on each slice, group locality
  masked_fm       hand values, symmetry of the request block, n_c = 0 reduces
                  to X X^T, brute force
  token_lcb       brute force, hand values, invariance
  attention       L = 1 returns V, equal keys return mean(V), one dominant
                  key returns its value row, torch CPU SDPA, brute force
  encoder_layer   torch.nn.TransformerEncoderLayer (CPU, eval, float64)
"""

from __future__ import annotations

import numpy as np

F64 = np.float64


def glm_mask(d_in_r: int, d_in_c: int, d_out_r: int, d_out_c: int) -> np.ndarray:
    """Channel-level dependency mask of a two-group GLM linear layer.

    [R] §2.1, dependency matrix: output group i may read input group j iff
    j <= i.  Group 0 is the request, group 1 the candidate, so only the
    request-output x candidate-input block is zero.
    """
    M = np.ones((d_out_r + d_out_c, d_in_r + d_in_c), dtype=F64)
    M[:d_out_r, d_in_r:] = 0.0
    return M


def glm_linear(x: np.ndarray, W: np.ndarray, b, d_in_r: int, d_out_r: int, mask: bool = True) -> np.ndarray:
    """Masked dense linear map applied to every candidate's dense state row.

    [R] §2.1, masked-weight equation and the two-group block matrix:
    W~ = M (.) W, y = W~ x + b, so y_R = W_RR x_R + b_R and
    y_C = W_CR x_R + W_CC x_C + b_C.  The mask is applied to the weights
    before the product (masking outputs afterwards would not be
    equivalent, same section).

    ``mask=False`` exists only so tests can plant the unmasked mistake and
    check that the invariance test catches it.
    """
    x = np.asarray(x, dtype=F64)
    W = np.asarray(W, dtype=F64)
    d_out = W.shape[0]
    d_in = W.shape[1]
    assert x.shape[-1] == d_in
    Wt = W * glm_mask(d_in_r, d_in - d_in_r, d_out_r, d_out - d_out_r) if mask else W
    y = x @ Wt.T
    if b is not None:
        y = y + np.asarray(b, dtype=F64)
    return y


def decomposed_linear(x_r, x_c, cand2req, W, b, d_in_r: int, d_out_r: int):
    """The request/candidate decomposition of the same layer, for pinning only.

    [R] §2.4: on the request batch compute Y_R and Z = W_CR X_R once; each
    candidate output is Y_C[i] = Z[m_i] + W_CC X_C[i] (+ b_C).  The oracle
    itself never uses this form; tests check it equals ``glm_linear`` on
    the broadcast state, which is the identity the method relies on.
    """
    W = np.asarray(W, dtype=F64)
    x_r = np.asarray(x_r, dtype=F64)
    x_c = np.asarray(x_c, dtype=F64)
    W_rr = W[:d_out_r, :d_in_r]
    W_cr = W[d_out_r:, :d_in_r]
    W_cc = W[d_out_r:, d_in_r:]
    b = np.zeros(W.shape[0]) if b is None else np.asarray(b, dtype=F64)
    y_r = x_r @ W_rr.T + b[:d_out_r]
    z = x_r @ W_cr.T
    y_c = z[np.asarray(cand2req)] + x_c @ W_cc.T + b[d_out_r:]
    return y_r, y_c


def relu(x: np.ndarray) -> np.ndarray:
    """Elementwise ReLU; elementwise ops are group-local by construction ([R] §2.1, Figure 2(b))."""
    return np.maximum(np.asarray(x, dtype=F64), 0.0)


def _norm_rows(x: np.ndarray, kind: str, eps: float) -> np.ndarray:
    if kind == "layer":
        mu = x.mean(axis=-1, keepdims=True)
        var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)  # biased variance
        return (x - mu) / np.sqrt(var + eps)
    if kind == "rms":
        ms = (x * x).mean(axis=-1, keepdims=True)
        return x / np.sqrt(ms + eps)
    raise ValueError(kind)


def group_norm(x: np.ndarray, widths, kind: str, eps: float = 1e-5, gammas=None, betas=None) -> np.ndarray:
    """Group-local LayerNorm / RMSNorm of each row of the dense state.

    [R] §2.1, Figure 2(b): normalisation statistics are taken inside each
    group, never across groups.  ``widths`` lists the group widths in
    order (request first); statistics are over each slice of a row only.
    LayerNorm uses the biased variance; gamma/beta default to 1/0.
    """
    x = np.asarray(x, dtype=F64)
    out = np.empty_like(x)
    c0 = 0
    for g, w in enumerate(widths):
        sl = x[..., c0:c0 + w]
        y = _norm_rows(sl, kind, eps)
        if gammas is not None and gammas[g] is not None:
            y = y * np.asarray(gammas[g], dtype=F64)
        if betas is not None and betas[g] is not None:
            y = y + np.asarray(betas[g], dtype=F64)
        out[..., c0:c0 + w] = y
        c0 += w
    assert c0 == x.shape[-1]
    return out


def token_mask(n_r: int, n_c: int) -> np.ndarray:
    """Token-level dependency mask for an interaction over [request tokens ; candidate tokens].

    [R] §2.1, masked-FM equation: output group i interacts with input
    groups 0..i only, so request-token rows see request-token columns only.
    """
    M = np.ones((n_r + n_c, n_r + n_c), dtype=F64)
    M[:n_r, n_r:] = 0.0
    return M


def masked_fm(X: np.ndarray, n_r: int):
    """Masked factorization-machine interaction on one dense token matrix per candidate.

    [R] §2.1, masked-FM equation and Figure 2(c): with X~ = [X_R ; X_C]
    ((n_r + n_c) x D), P = (X~ X~^T) (.) M_tok; the request output is
    P[:n_r, :n_r] (request x request), the candidate output is P[n_r:, :]
    (candidate x [request, candidate]).  The structurally zero
    request x candidate block is not returned.  Outputs are flattened
    token-major: row a of P, then its columns.

    X: [n, n_r + n_c, D].  Returns (f_r [n, n_r*n_r], f_c [n, n_c*(n_r+n_c)]).
    """
    X = np.asarray(X, dtype=F64)
    n_tok = X.shape[1]
    P = np.einsum("nad,nbd->nab", X, X) * token_mask(n_r, n_tok - n_r)
    f_r = P[:, :n_r, :n_r].reshape(X.shape[0], -1)
    f_c = P[:, n_r:, :].reshape(X.shape[0], -1)
    return f_r, f_c


def token_lcb(X: np.ndarray, W: np.ndarray, n_r: int, t_r: int, mask: bool = True):
    """GLM linear compression along the token axis.

    [R] §2.1, masked-weight linear equation applied with tokens as the
    grouped axis ("LCB" in Figure 1(d) / Figure 2(a)): W~ = M (.) W over
    [t_r + t_c, n_r + n_c] token blocks, T = W~ X~ for each candidate's
    dense token matrix X~ = [X_R ; X_C].  Returns (T_R [n, t_r*D],
    T_C [n, t_c*D]) flattened token-major.  No bias.
    """
    X = np.asarray(X, dtype=F64)
    W = np.asarray(W, dtype=F64)
    n_tok = X.shape[1]
    t_out = W.shape[0]
    Wt = W * glm_mask(n_r, n_tok - n_r, t_r, t_out - t_r) if mask else W
    T = np.einsum("ta,nad->ntd", Wt, X)
    return T[:, :t_r, :].reshape(X.shape[0], -1), T[:, t_r:, :].reshape(X.shape[0], -1)


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, n_heads: int, scale=None) -> np.ndarray:
    """Multi-head softmax attention with no mask, one batch item at a time.

    [R] §2.2, grouped cross-attention A = Attn(Q, S W_K, S W_V).  Heads are
    contiguous head_dim slices of the feature axis; scores are
    q_h . k_h / sqrt(head_dim); softmax over keys with the max subtracted;
    output is the probability-weighted sum of values.

    q: [n, Lq, d], K, V: [n, Lk, d] (already broadcast per batch item).
    Returns [n, Lq, d].
    """
    q = np.asarray(q, dtype=F64)
    K = np.asarray(K, dtype=F64)
    V = np.asarray(V, dtype=F64)
    n, Lq, d = q.shape
    dh = d // n_heads
    scale = 1.0 / np.sqrt(dh) if scale is None else scale
    out = np.empty((n, Lq, d), dtype=F64)
    for h in range(n_heads):
        sl = slice(h * dh, (h + 1) * dh)
        s = np.einsum("nqe,nke->nqk", q[..., sl], K[..., sl]) * scale
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=-1, keepdims=True)
        out[..., sl] = np.einsum("nqk,nke->nqe", p, V[..., sl])
    return out


def mha(S: np.ndarray, w_qkv, b_qkv, w_o, b_o, n_heads: int) -> np.ndarray:
    """Multi-head self-attention with a fused [3d, d] in-projection (q, k, v row blocks) and an output projection."""
    S = np.asarray(S, dtype=F64)
    d = S.shape[-1]
    qkv = S @ np.asarray(w_qkv, F64).T + np.asarray(b_qkv, F64)
    q, k, v = qkv[..., :d], qkv[..., d:2 * d], qkv[..., 2 * d:]
    a = attention(q, k, v, n_heads)
    return a @ np.asarray(w_o, F64).T + np.asarray(b_o, F64)


def encoder_layer(S: np.ndarray, p: dict, n_heads: int, eps: float = 1e-5) -> np.ndarray:
    """One request-only sequence encoder layer S_k = Enc_k(S_{k-1}).

    [R] §2.2, first equation: the encoder reads only the request's
    sequence.  Its internal form is not given on the pages; the reading
    used is a post-LN transformer layer with a ReLU FFN and no mask:
    S' = LN(S + MHA(S)); S'' = LN(S' + W2 ReLU(W1 S' + b1) + b2).

    S: [n, L, d]; p holds w_qkv, b_qkv, w_o, b_o, w_1, b_1, w_2, b_2.
    """
    S = np.asarray(S, dtype=F64)
    d = S.shape[-1]
    a = mha(S, p["w_qkv"], p["b_qkv"], p["w_o"], p["b_o"], n_heads)
    S1 = group_norm(S + a, [d], "layer", eps)
    f = relu(S1 @ np.asarray(p["w_1"], F64).T + np.asarray(p["b_1"], F64))
    f = f @ np.asarray(p["w_2"], F64).T + np.asarray(p["b_2"], F64)
    return group_norm(S1 + f, [d], "layer", eps)
