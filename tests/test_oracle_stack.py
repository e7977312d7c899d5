"""Stack-level pins of the oracle: the properties the pages fix for a ROCSified model.

[R] §2.1: request outputs equal for every candidate of a request and equal
to F_R(X_R) (request-output equality), composition closure (Figure 2(d)),
and the two-group form.  Plus request independence, permutation
equivariance and the planted unmasked-weight control.
"""

import numpy as np
import pytest

import oracle
import rocs_synth as S
from oracle import ops


def _perturbed(inputs, scale=25.0, seed=99):
    rng = np.random.default_rng(seed)
    out = dict(inputs)
    xc = inputs["x_c"]
    out["x_c"] = (xc + rng.standard_normal(xc.shape).astype(np.float32) * scale).astype(np.float32)
    return out


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_request_outputs_independent_of_candidates(k):
    inp = S.make_inputs(S.small_config(k))
    a = oracle.oracle_forward(inp)
    b = oracle.oracle_forward(_perturbed(inp))
    assert np.array_equal(a["y_r"], b["y_r"])
    assert not np.allclose(a["y_c"], b["y_c"])


def test_planted_unmasked_weights_break_request_invariance(monkeypatch):
    inp = S.make_inputs(S.small_config(2))
    real = ops.glm_linear

    def unmasked(x, W, b, d_in_r, d_out_r, mask=True):
        return real(x, W, b, d_in_r, d_out_r, mask=False)

    monkeypatch.setattr(ops, "glm_linear", unmasked)
    with pytest.raises(AssertionError):
        # request outputs now differ across a request's candidates
        oracle.oracle_forward(inp)


@pytest.mark.parametrize("k", [2, 3, 4])
def test_request_subsets_are_independent(k):
    inp = S.make_inputs(S.small_config(k))
    full = oracle.oracle_forward(inp)
    sub = [1, 3]
    part = oracle.oracle_forward(inp, requests=sub)
    pos = {r: i for i, r in enumerate(full["rows"].tolist())}
    idx = [pos[r] for r in part["rows"].tolist()]
    assert np.max(np.abs(full["y_c"][idx] - part["y_c"])) <= 1e-12
    assert np.max(np.abs(full["y_r"][sub] - part["y_r"])) <= 1e-12


@pytest.mark.parametrize("k", [2, 5])
def test_candidate_permutation_equivariance(k):
    inp = S.make_inputs(S.small_config(k))
    full = oracle.oracle_forward(inp)
    sh = S.shuffle_candidates(inp, seed=3)
    out = oracle.oracle_forward(sh)
    # row j of the shuffled batch is row perm[j] of the original
    assert np.max(np.abs(out["y_c"] - full["y_c"][sh["perm"]])) <= 1e-12
    assert np.max(np.abs(out["y_r"] - full["y_r"])) <= 1e-12


def test_empty_request_gets_request_outputs():
    cfg = S.small_config(2)
    full = S.make_inputs(cfg, counts=[1, 3, 2, 2, 5, 1, 1, 4, 2, 1, 1, 6])
    # same draw with the candidates of requests 0, 2 and 6 removed
    keep = ~np.isin(full["cand2req"], [0, 2, 6])
    counts = full["counts"].copy()
    counts[[0, 2, 6]] = 0
    inp = dict(full)
    inp.update(S.make_batch(counts))
    inp["x_c"] = full["x_c"][keep]
    out = oracle.oracle_forward(inp)
    ref = oracle.oracle_forward(full)
    assert out["y_r"].shape == (cfg.B, cfg.d_r)
    assert np.max(np.abs(out["y_r"] - ref["y_r"])) <= 1e-12
    assert np.max(np.abs(out["y_c"] - ref["y_c"][keep])) <= 1e-12


def test_single_candidate_requests_match_per_pair_evaluation():
    # N = 1: the shared batch equals evaluating every (request, candidate) pair alone.
    cfg = S.small_config(3)
    inp = S.make_inputs(cfg, counts=[1] * cfg.B)
    joint = oracle.oracle_forward(inp)
    for b in range(cfg.B):
        alone = oracle.oracle_forward(inp, requests=[b])
        assert np.max(np.abs(alone["y_c"][0] - joint["y_c"][b])) <= 1e-12


def test_composition_closure_random_chains():
    # [R] §2.1 Figure 2(d): any composition of GLM-compliant ops is GLM-compliant.
    rng = np.random.default_rng(21)
    for trial in range(20):
        w_r, w_c = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        x = rng.standard_normal((5, w_r + w_c))
        x2 = x.copy()
        x2[:, w_r:] = rng.standard_normal((5, w_c)) * 10

        def chain(v, seed):
            r = np.random.default_rng(seed)
            cur_r, cur_c = w_r, w_c
            for _ in range(int(r.integers(2, 7))):
                op = r.integers(0, 4)
                if op == 0:
                    o_r, o_c = int(r.integers(1, 6)), int(r.integers(1, 6))
                    W = r.standard_normal((o_r + o_c, cur_r + cur_c))
                    v = ops.glm_linear(v, W, r.standard_normal(o_r + o_c), cur_r, o_r)
                    cur_r, cur_c = o_r, o_c
                elif op == 1:
                    v = ops.group_norm(v, [cur_r, cur_c], "layer" if r.integers(0, 2) else "rms")
                elif op == 2:
                    v = ops.relu(v)
                else:
                    W = r.standard_normal((cur_r + cur_c, cur_r + cur_c))
                    v = v + ops.glm_linear(v, W, None, cur_r, cur_r)  # residual add
            return v, cur_r

        y1, o_r = chain(x, 1000 + trial)
        y2, _ = chain(x2, 1000 + trial)
        assert np.array_equal(y1[:, :o_r], y2[:, :o_r])


def test_full_size_batches_match_the_workload_counts():
    # the seeded count draws are part of the workload definition
    assert len(S.make_inputs(S.config(1))["cand2req"]) == 39
    for k, bc in [(2, 73704), (4, 30231), (5, 32486)]:
        c = S.config(k)
        rng = np.random.default_rng(100 + k)
        from rocs_synth import _draw_counts
        assert int(_draw_counts(rng, c).sum()) == bc


# ---------------------------------------------------------------------------
# Closed-form pins of the compositions.  Each test replaces some weights with
# special values (zero, identity, selection) under which a composition
# reduces to library routines (torch layer_norm / rms_norm /
# TransformerEncoderLayer, numpy products) computed here independently of the
# oracle.  Every plausible slip in assembling a stack (a dropped residual,
# LayerNorm swapped for RMSNorm, ReLU on the wrong side of a norm, [G || A] or
# [vec F || vec T] in the wrong order, the wrong encoder depth, the wrong
# key/value group) changes at least one of these values.

import torch  # noqa: E402
import torch.nn.functional as TF  # noqa: E402

from oracle.stack import depth_source  # noqa: E402


def _blocks(d_in_r, d_in_c, d_out_r, d_out_c, rr=None, cr=None, cc=None, seed=0):
    """Dense GLM weight from its three live blocks; the masked block gets noise."""
    W = np.zeros((d_out_r + d_out_c, d_in_r + d_in_c))
    if rr is not None:
        W[:d_out_r, :d_in_r] = rr
    if cr is not None:
        W[d_out_r:, :d_in_r] = cr
    if cc is not None:
        W[d_out_r:, d_in_r:] = cc
    # the request-output x candidate-input block must be ignored (mask)
    W[:d_out_r, d_in_r:] = np.random.default_rng(seed).standard_normal((d_out_r, d_in_c)) * 3.0
    return W


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


def _ln(a, eps=1e-5):
    return TF.layer_norm(_t(a), (a.shape[-1],), eps=eps).numpy()


def _rms(a, eps=1e-5):
    return TF.rms_norm(_t(a), (a.shape[-1],), eps=eps).numpy()


def _torch_encoder(seq, w, cfg):
    """S_0..S_n_enc with torch's post-LN encoder layer (weights copied in)."""
    d, H, f = cfg.d_seq, cfg.n_heads, cfg.ffn
    S = [np.asarray(seq, np.float64)]
    for k in range(cfg.n_enc):
        layer = torch.nn.TransformerEncoderLayer(d, H, f, dropout=0.0, activation="relu", batch_first=True,
                                                 norm_first=False, layer_norm_eps=cfg.eps, dtype=torch.float64)
        layer.eval()
        with torch.no_grad():
            layer.self_attn.in_proj_weight.copy_(_t(w[f"enc{k}.w_qkv"]))
            layer.self_attn.in_proj_bias.copy_(_t(w[f"enc{k}.b_qkv"]))
            layer.self_attn.out_proj.weight.copy_(_t(w[f"enc{k}.w_o"]))
            layer.self_attn.out_proj.bias.copy_(_t(w[f"enc{k}.b_o"]))
            layer.linear1.weight.copy_(_t(w[f"enc{k}.w_1"]))
            layer.linear1.bias.copy_(_t(w[f"enc{k}.b_1"]))
            layer.linear2.weight.copy_(_t(w[f"enc{k}.w_2"]))
            layer.linear2.bias.copy_(_t(w[f"enc{k}.b_2"]))
            S.append(layer(_t(S[-1])).numpy())
    return S


def _close(a, b, tol=1e-10):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.max(np.abs(a - b)) <= tol * max(1.0, float(np.max(np.abs(b))))


def test_depth_source_hand_values():
    # [R] §2.2 pairs interaction depth i with encoder output i; the reading
    # for unequal depth counts spreads the encoder outputs evenly.
    assert depth_source(2, 1) == [2]
    assert depth_source(2, 2) == [1, 2]
    assert depth_source(2, 3) == [1, 2, 2]
    assert depth_source(2, 4) == [1, 1, 2, 2]
    assert depth_source(3, 3) == [1, 2, 3]
    assert depth_source(1, 3) == [1, 1, 1]
    assert depth_source(4, 2) == [2, 4]


def test_glm_tiny_identity_weights_give_relu_of_group_layernorm():
    cfg = S.small_config(1)
    inp = S.make_inputs(cfg)
    d, H = cfg.d_r, cfg.hidden
    inp["w"]["lin.W"] = _blocks(d, d, H, H, rr=np.eye(d), cc=np.eye(d))
    inp["w"]["lin.b"] = np.zeros(2 * H)
    out = oracle.oracle_forward(inp)
    xr = np.asarray(inp["x_r"], np.float64)
    xc = np.asarray(inp["x_c"], np.float64)[out["rows"]]
    _close(out["y_r"], np.maximum(_ln(xr), 0.0))
    _close(out["y_c"], np.maximum(_ln(xc), 0.0))


@pytest.mark.parametrize("r", [1, 2])
def test_glm_mlp_zero_down_projection_gives_repeated_rmsnorm_and_head_dots(r):
    # o = 0, so every block is x <- RMSNorm_g(x + 0): n_blocks nested rms_norms
    # per group; the head is then w_CR . y_R[m] + w_CC . y_C.  r = 2 widens the
    # request-side path (request-side scaling, [R] §2.3).
    cfg = S.small_config(2)
    cfg = cfg.with_(d_r=r * cfg.d_r, hidden_r=r * cfg.hidden)
    inp = S.make_inputs(cfg)
    w = inp["w"]
    for k in range(cfg.n_blocks):
        w[f"blk{k}.down.W"] = np.zeros_like(w[f"blk{k}.down.W"])
        w[f"blk{k}.down.b"] = np.zeros_like(w[f"blk{k}.down.b"])
    out = oracle.oracle_forward(inp)
    yr = np.asarray(inp["x_r"], np.float64)
    yc = np.asarray(inp["x_c"], np.float64)[out["rows"]]
    for _ in range(cfg.n_blocks):
        yr, yc = _rms(yr), _rms(yc)
    _close(out["y_r"], yr)
    _close(out["y_c"], yc)
    hw = np.asarray(w["head.W"], np.float64)[0]
    m = inp["cand2req"][out["rows"]]
    _close(out["logits"], yr[m] @ hw[:cfg.d_r] + yc @ hw[cfg.d_r:])


def test_glm_mlp_identity_blocks_pin_relu_residual_and_cross_term():
    # hidden = d, up = [[I, *], [A, I]] + b1, down = [[I, *], [0, I]] + b2:
    # h = ReLU(x W_up + b1); x <- RMSNorm_g(x + h + b2), with the candidate
    # group's h reading A x_R (the W_CR cross term).
    d = 48
    cfg = S.small_config(2).with_(B=5, counts=("uniform", 1, 6), d_r=d, d_c=d, hidden=d, n_blocks=2)
    inp = S.make_inputs(cfg)
    w = inp["w"]
    rng = np.random.default_rng(5)
    A = [rng.standard_normal((d, d)) * 0.3 for _ in range(cfg.n_blocks)]
    b1 = [rng.standard_normal(2 * d) for _ in range(cfg.n_blocks)]
    b2 = [rng.standard_normal(2 * d) for _ in range(cfg.n_blocks)]
    I = np.eye(d)
    for k in range(cfg.n_blocks):
        w[f"blk{k}.up.W"] = _blocks(d, d, d, d, rr=I, cr=A[k], cc=I, seed=k)
        w[f"blk{k}.up.b"] = b1[k]
        w[f"blk{k}.down.W"] = _blocks(d, d, d, d, rr=I, cc=I, seed=10 + k)
        w[f"blk{k}.down.b"] = b2[k]
    out = oracle.oracle_forward(inp)
    m = inp["cand2req"][out["rows"]]
    xr = np.asarray(inp["x_r"], np.float64)
    xc = np.asarray(inp["x_c"], np.float64)[out["rows"]]
    for k in range(cfg.n_blocks):
        hr = np.maximum(xr + b1[k][:d], 0.0)
        hc = np.maximum(xr[m] @ A[k].T + xc + b1[k][d:], 0.0)
        xr, xc = _rms(xr + hr + b2[k][:d]), _rms(xc + hc + b2[k][d:])
    _close(out["y_r"], xr)
    _close(out["y_c"], xc)


def test_dca_one_event_zero_query_mlp_gives_bias_then_encoded_values():
    # L = 1: attention returns the single value row whatever the query, and
    # with MLP2's weights zero G is its bias: each group's output is
    # [b || S_src . W_V] with S_src = S_2 (two encoder layers, one
    # interaction layer) from torch's encoder layer.
    cfg = S.small_config(3).with_(L=1)
    inp = S.make_inputs(cfg)
    w = inp["w"]
    d = cfg.d_seq
    b = np.random.default_rng(8).standard_normal(2 * d)
    w["int0.mlp2.W"] = np.zeros_like(w["int0.mlp2.W"])
    w["int0.mlp2.b"] = b
    out = oracle.oracle_forward(inp)
    Ss = _torch_encoder(inp["seq"], w, cfg)
    s = Ss[2][:, 0, :]
    m = inp["cand2req"][out["rows"]]
    a_r = s @ np.asarray(w["kv0.wv_r"], np.float64).T
    a_c = s[m] @ np.asarray(w["kv0.wv_c"], np.float64).T
    _close(out["y_r"], np.concatenate([np.broadcast_to(b[:d], (cfg.B, d)), a_r], axis=1))
    _close(out["y_c"], np.concatenate([np.broadcast_to(b[d:], (len(m), d)), a_c], axis=1))


def test_dca_zero_query_gives_mean_of_encoded_values():
    # q = 0: every key gets the same score, so A = mean over the L events of
    # S_src . W_V for each group.
    cfg = S.small_config(3)
    inp = S.make_inputs(cfg)
    w = inp["w"]
    d = cfg.d_seq
    w["int0.mlp2.W"] = np.zeros_like(w["int0.mlp2.W"])
    w["int0.mlp2.b"] = np.zeros_like(w["int0.mlp2.b"])
    out = oracle.oracle_forward(inp)
    Ss = _torch_encoder(inp["seq"], w, cfg)
    mean = Ss[2].mean(axis=1)
    m = inp["cand2req"][out["rows"]]
    _close(out["y_r"][:, d:], mean @ np.asarray(w["kv0.wv_r"], np.float64).T)
    _close(out["y_c"][:, d:], mean[m] @ np.asarray(w["kv0.wv_c"], np.float64).T)
    assert np.all(out["y_r"][:, :d] == 0.0) and np.all(out["y_c"][:, :d] == 0.0)


def test_dca_pass_through_chain_pins_depths_and_the_query_input():
    # Two encoder layers, two interaction layers (depths 1, 2), L = 1.  The
    # second layer's query MLP passes the A part of its input [G0 || A0]
    # through unchanged (ReLU(a) - ReLU(-a) = a): its output is then
    # [A0 || A1] = [S_1 . W_V0 || S_2 . W_V1] per group.
    cfg = S.small_config(5).with_(L=1, n_int=2)
    inp = S.make_inputs(cfg)
    w = inp["w"]
    d, H = cfg.d_seq, cfg.hidden
    assert H == 2 * d
    I = np.eye(d)
    Z = np.zeros((d, d))
    sel = np.block([[Z, I], [Z, -I]])  # [2d, 2d]: rows pick +A then -A from [G || A]
    w["int1.mlp1.W"] = _blocks(2 * d, 2 * d, H, H, rr=sel, cc=sel, seed=3)
    w["int1.mlp1.b"] = np.zeros(2 * H)
    comb = np.concatenate([I, -I], axis=1)  # [d, 2d]
    w["int1.mlp2.W"] = _blocks(H, H, d, d, rr=comb, cc=comb, seed=4)
    w["int1.mlp2.b"] = np.zeros(2 * d)
    out = oracle.oracle_forward(inp)
    Ss = _torch_encoder(inp["seq"], w, cfg)
    m = inp["cand2req"][out["rows"]]
    s1, s2 = Ss[1][:, 0, :], Ss[2][:, 0, :]
    wv = lambda nm: np.asarray(w[nm], np.float64).T  # noqa: E731
    _close(out["y_r"], np.concatenate([s1 @ wv("kv0.wv_r"), s2 @ wv("kv1.wv_r")], axis=1))
    _close(out["y_c"], np.concatenate([s1[m] @ wv("kv0.wv_c"), s2[m] @ wv("kv1.wv_c")], axis=1))
    hw = np.asarray(w["head.W"], np.float64)[0]
    _close(out["logits"], out["y_r"][np.searchsorted(out["requests"], m)] @ hw[:2 * d] + out["y_c"] @ hw[2 * d:])


def test_wukong_selection_mlp_gives_nested_layernorms_of_fm_and_token_columns():
    # mlp1 selects columns of u = [vec F || vec T] per group (W_CR = 0),
    # mlp2 is zero: h1 = LN_g(ReLU(u[:, sel])), h2 = LN_g(h1 + ReLU(0)) =
    # LN_g(h1).  F and T are recomputed here with plain products:
    # F_R = X_R X_R^T, F_C = X_C [X_R; X_C]^T, T_R = W_RR X_R,
    # T_C = W_CR X_R + W_CC X_C, each flattened row-major.
    cfg = S.small_config(4)
    inp = S.make_inputs(cfg)
    w = inp["w"]
    nr, nc, D, T, H = cfg.n_tok_r, cfg.n_tok_c, cfg.tok_dim, cfg.tok_out, cfg.hidden
    ur, uc = nr * nr + T * D, nc * (nr + nc) + T * D
    rng = np.random.default_rng(17)
    sel_r = np.concatenate([np.arange(nr * nr), nr * nr + np.sort(rng.choice(T * D, H - nr * nr, replace=False))])
    sel_c = np.concatenate([np.arange(nc * (nr + nc)),
                            nc * (nr + nc) + np.sort(rng.choice(T * D, H - nc * (nr + nc), replace=False))])
    Pr = np.zeros((H, ur))
    Pr[np.arange(H), sel_r] = 1.0
    Pc = np.zeros((H, uc))
    Pc[np.arange(H), sel_c] = 1.0
    w["mlp1.W"] = _blocks(ur, uc, H, H, rr=Pr, cc=Pc, seed=6)
    w["mlp1.b"] = np.zeros(2 * H)
    w["mlp2.W"] = np.zeros_like(w["mlp2.W"])
    w["mlp2.b"] = np.zeros_like(w["mlp2.b"])
    out = oracle.oracle_forward(inp)
    m = inp["cand2req"][out["rows"]]
    Xr = np.asarray(inp["x_r"], np.float64)
    Xc = np.asarray(inp["x_c"], np.float64)[out["rows"]]
    Wt = np.asarray(w["tok.W"], np.float64)
    fr = np.stack([x @ x.T for x in Xr]).reshape(cfg.B, -1)
    fc = np.stack([xc @ np.concatenate([Xr[b], xc]).T for xc, b in zip(Xc, m)]).reshape(len(m), -1)
    tr = np.stack([Wt[:T, :nr] @ x for x in Xr]).reshape(cfg.B, -1)
    tc = np.stack([Wt[T:, :nr] @ Xr[b] + Wt[T:, nr:] @ xc for xc, b in zip(Xc, m)]).reshape(len(m), -1)
    ur_v = np.concatenate([fr, tr], axis=1)
    uc_v = np.concatenate([fc, tc], axis=1)
    h_r = _ln(_ln(np.maximum(ur_v[:, sel_r], 0.0)))
    h_c = _ln(_ln(np.maximum(uc_v[:, sel_c], 0.0)))
    _close(out["y_r"], h_r)
    _close(out["y_c"], h_c)
    hw = np.asarray(w["head.W"], np.float64)[0]
    _close(out["logits"], h_r[m] @ hw[:H] + h_c @ hw[H:])


# Planted slips (in the oracle, on the CPU): each pin above must fail when the
# oracle makes the mistake it is there to catch.

def test_planted_wrong_depth_fails_the_pass_through_pin(monkeypatch):
    import oracle.stack as OS

    monkeypatch.setattr(OS, "depth_source", lambda n_enc, n_int: [n_enc] * n_int)
    with pytest.raises(AssertionError):
        test_dca_pass_through_chain_pins_depths_and_the_query_input()


def test_planted_norm_kind_swap_fails_the_rmsnorm_pin(monkeypatch):
    real = ops.group_norm

    def swapped(x, widths, kind, eps=1e-5, gammas=None, betas=None):
        return real(x, widths, "layer" if kind == "rms" else "rms", eps, gammas, betas)

    monkeypatch.setattr(ops, "group_norm", swapped)
    with pytest.raises(AssertionError):
        test_glm_mlp_zero_down_projection_gives_repeated_rmsnorm_and_head_dots(1)


def test_planted_attention_group_swap_fails_the_one_event_pin(monkeypatch):
    import oracle.stack as OS

    real = OS.oracle_encoder

    def swapped(inputs, requests=None):
        out = real(inputs, requests)
        out["kv"] = [(kc, vc, kr, vr) for (kr, vr, kc, vc) in out["kv"]]
        return out

    monkeypatch.setattr(OS, "oracle_encoder", swapped)
    with pytest.raises(AssertionError):
        test_dca_one_event_zero_query_mlp_gives_bias_then_encoded_values()


def test_planted_fm_token_order_swap_fails_the_selection_pin(monkeypatch):
    # the oracle assembling u as [vec T || vec F] instead of [vec F || vec T]
    import oracle.stack as OS

    real_np = OS.np

    class _SwappingNumpy:
        def __getattr__(self, k):
            return getattr(real_np, k)

        @staticmethod
        def concatenate(arrs, axis=0):
            if len(arrs) == 4 and axis == 1 and arrs[0].shape[1] < arrs[1].shape[1]:
                arrs = [arrs[1], arrs[0], arrs[3], arrs[2]]
            return real_np.concatenate(arrs, axis=axis)

    monkeypatch.setattr(OS, "np", _SwappingNumpy())
    with pytest.raises(AssertionError):
        test_wukong_selection_mlp_gives_nested_layernorms_of_fm_and_token_columns()
