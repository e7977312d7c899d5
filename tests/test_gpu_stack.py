"""Whole-stack GPU parity (rocs_stack_forward) against the dense CPU oracle.

Small variants of all five workloads run in full; the full-size workloads
(the configuration the benchmark times) run on the GPU in full and are
compared with the oracle on a sample of requests (requests are independent,
so the oracle evaluates only the sampled requests' candidates).
"""

import numpy as np
import pytest

import oracle
import rocs_synth as S
from gpu_util import rel_err, tol

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _stack(inp, mode=0, fusion=False):
    from request_candidate_sharing_amd.stacks import DeviceStack

    st = DeviceStack(inp, mode=mode, fusion=fusion)
    st.run()
    return st, st.outputs()


def _compare(cfg, got, ref, rows=None, reqs=None):
    t = tol(cfg.dtype)
    yc = got["y_c"] if rows is None else got["y_c"][rows]
    yr = got["y_r"] if reqs is None else got["y_r"][reqs]
    assert rel_err(yc, ref["y_c"]) <= t
    assert rel_err(yr, ref["y_r"]) <= t
    if ref["logits"] is not None:
        lg = got["logits"] if rows is None else got["logits"][rows]
        assert rel_err(lg, ref["logits"]) <= t


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_small_stack_parity(k):
    cfg = S.small_config(k)
    inp = S.make_inputs(cfg)
    _, got = _stack(inp)
    ref = oracle.oracle_forward(inp)
    assert np.array_equal(ref["rows"], np.arange(len(inp["cand2req"])))
    _compare(cfg, got, ref)


@pytest.mark.parametrize("k", [2, 3, 4, 5])
def test_small_stack_request_outputs_ignore_candidates(k):
    cfg = S.small_config(k)
    inp = S.make_inputs(cfg)
    _, a = _stack(inp)
    pert = dict(inp)
    pert["x_c"] = (inp["x_c"] + 3.0 * np.random.default_rng(1).standard_normal(inp["x_c"].shape)).astype(np.float32)
    pert["x_c"] = S.round_bf16(pert["x_c"]) if cfg.dtype == "bf16" else pert["x_c"]
    _, b = _stack(pert)
    assert np.array_equal(a["y_r"], b["y_r"])


@pytest.mark.parametrize("k", [2, 3, 5])
def test_small_stack_shuffled_candidates(k):
    cfg = S.small_config(k)
    inp = S.make_inputs(cfg)
    _, a = _stack(inp)
    sh = S.shuffle_candidates(inp, seed=5)
    _, b = _stack(sh)
    p = sh["perm"]
    assert np.array_equal(b["y_c"], a["y_c"][p])
    assert np.array_equal(b["y_r"], a["y_r"])
    if a["logits"] is not None:
        assert np.array_equal(b["logits"], a["logits"][p])


@pytest.mark.parametrize("k", [2, 3, 4])
def test_dense_broadcast_mode_matches_shared(k):
    cfg = S.small_config(k)
    inp = S.make_inputs(cfg)
    _, a = _stack(inp, mode=0)
    _, b = _stack(inp, mode=1)
    if k == 3:  # attention: per-candidate tiles; same arithmetic per query
        assert rel_err(b["y_c"], a["y_c"]) <= 1e-2
    else:  # same kernels on copied rows: identical bits
        assert np.array_equal(a["y_c"], b["y_c"])
    assert np.array_equal(a["y_r"], b["y_r"])


@pytest.mark.parametrize("k", [2, 3, 5])
def test_fused_stack_parity(k):
    # ROCS_STACK_FUSE_MLP: candidate-side LINEAR -> LINEAR [-> NORM] as one kernel
    # (GLM MLP blocks of workload 2, the 256-wide interaction MLPs of the DCA stacks).
    cfg = S.small_config(k)
    inp = S.make_inputs(cfg)
    _, got = _stack(inp, fusion=True)
    _compare(cfg, got, oracle.oracle_forward(inp))


@pytest.mark.parametrize("k", [2, 3, 5])
def test_fused_mlp_block_matches_unfused_layers(k):
    # Without a fused norm (the DCA interaction MLPs) both paths reduce in the same
    # order and round once: identical bits.  With the norm fused (workload 2), the
    # unfused path rounds the pre-norm sum to bf16 first.
    from request_candidate_sharing_amd.stacks import DeviceStack

    cfg = S.small_config(k)
    inp = S.make_inputs(cfg)
    f = DeviceStack(inp, fusion=True)
    u = DeviceStack(inp, fusion=False)
    f.run()
    u.run()
    a, b = f.outputs(), u.outputs()
    assert np.array_equal(a["y_r"], b["y_r"])
    if k == 2:
        assert rel_err(a["y_c"], b["y_c"]) <= 1e-2
    else:
        assert np.array_equal(a["y_c"], b["y_c"])


def test_single_candidate_requests_match_oracle():
    cfg = S.small_config(2)
    inp = S.make_inputs(cfg, counts=[1] * cfg.B)
    _, got = _stack(inp)
    _compare(cfg, got, oracle.oracle_forward(inp))


def test_tiny_glm_full_fp32():
    cfg = S.config(1)
    inp = S.make_inputs(cfg)
    _, got = _stack(inp)
    _compare(cfg, got, oracle.oracle_forward(inp))


@pytest.mark.slow
@pytest.mark.parametrize("k,sample,fusion", [(2, [0, 77, 255], False), (2, [3, 128], True), (3, [0, 63], False),
                                            (4, [5, 100], False), (5, [0, 31], False)])
def test_full_size_stack_sampled(k, sample, fusion):
    cfg = S.config(k)
    inp = S.make_inputs(cfg)
    _, got = _stack(inp, fusion=fusion)
    assert np.all(np.isfinite(got["y_c"]))
    ref = oracle.oracle_forward(inp, requests=sample)
    _compare(cfg, got, ref, rows=ref["rows"], reqs=ref["requests"])


@pytest.mark.parametrize("k", [2, 4])
def test_head_fused_into_norm_matches_standalone_head(k):
    # The stack runs a score head that reads a norm's output inside that
    # norm's candidate pass.  Its logits equal, bit for bit, the standalone
    # head (rocs_head_forward) applied to the stack's own output rows.
    from request_candidate_sharing_amd import rocs as Rr

    cfg = S.small_config(k)
    inp = S.make_inputs(cfg)
    st, out = _stack(inp)
    if out["logits"] is None:
        pytest.skip("stack without a head")
    W = np.asarray(inp["w"]["head.W"], dtype=np.float32)
    b = float(np.asarray(inp["w"]["head.b"], dtype=np.float32).reshape(-1)[0])
    wr, wc = st.slots[1]
    w_cr = st.t(W[0, :wr])
    w_cc = st.t(W[0, wr:])
    z = torch.empty(max(st.B_r, 1), dtype=torch.float32, device="cuda")
    lg = torch.empty(max(st.B_c, 1), dtype=torch.float32, device="cuda")
    Rr.rocs_head_forward(st.batch, Rr.ROCS_BF16, st.y_r, wr, wr, st.y_c, wc, wc, w_cr, w_cc, b, z, lg,
                         Rr.cur_stream())
    torch.cuda.synchronize()
    assert np.array_equal(lg[: st.B_c].cpu().numpy(), out["logits"])
