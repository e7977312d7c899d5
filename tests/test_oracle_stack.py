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
