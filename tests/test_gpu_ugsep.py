"""GPU parity of the UG-Separation TokenMixer path against the CPU oracle.

Citation: "Compute Only Once: UG-Separation for Efficient Large
Recommendation Models" (xllm-io review), §3.  Every case calls librocs
through the C ABI and compares with ``oracle/ugsep.py`` on the same seeded
inputs: max|gpu - oracle| / max|oracle| within 1e-5 (fp32) or 2e-2 (bf16
storage, fp32 accumulation).  Sizes span several GEMM tiles with ragged
tails, requests with no candidates, shuffled candidate order, padded
leading dimensions, the empty batch and sides with no tokens; the
full-size workload is checked on sampled candidates and requests.
"""

import numpy as np
import pytest

import rocs_synth as S
from oracle import ugsep as U
from gpu_util import dev, rel_err, to_np, tol

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _R():
    from request_candidate_sharing_amd import rocs as R

    return R


def _tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _rdt(R, dtype):
    return R.ROCS_BF16 if dtype == "bf16" else R.ROCS_F32


def _rows(a, ld, tdt):
    """[rows, width] array placed in storage with leading dimension ld (NaN padding)."""
    a = np.asarray(a, dtype=np.float32)
    st = torch.full((max(a.shape[0], 1), ld), float("nan"), dtype=tdt, device="cuda")
    if a.shape[0] and a.shape[1]:
        st[:a.shape[0], :a.shape[1]].copy_(torch.as_tensor(a, device="cuda").to(tdt))
    return st


def _layers(inp, tdt, quant=None):
    out = []
    for p in inp["layers"]:
        d = {k: dev(p[k], tdt) for k in ("ln1_g", "ln1_b", "w1", "b1", "w2", "b2", "ln2_g", "ln2_b")}
        d["comp"] = None if p["comp"] is None else torch.as_tensor(p["comp"], dtype=torch.float32, device="cuda")
        out.append(d)
    for d, q in zip(out, quant or ()):
        for k in ("w1_q", "w2_q"):
            d[k] = torch.as_tensor(np.ascontiguousarray(q[k]), dtype=torch.uint8, device="cuda")
        for k in ("w1_scale", "w2_scale"):
            d[k] = torch.as_tensor(q[k], dtype=torch.float32, device="cuda")
    return out


def run_forward(inp, dtype, mode=0, pad=0, quant=None):
    """Runs rocs_ugsep_forward; returns (y_u [B_r, n_u, D], y_g [B_c, n_g, D]) as numpy."""
    R = _R()
    tdt = _tdt(dtype)
    n_u, n_g, D, H = inp["n_u"], inp["n_g"], inp["dim"], inp["hidden"]
    B_r, B_c = inp["x_u"].shape[0], inp["x_g"].shape[0]
    ldu, ldg = n_u * D + pad, n_g * D + pad
    xu = _rows(inp["x_u"].reshape(B_r, n_u * D), max(ldu, 8), tdt)
    xg = _rows(inp["x_g"].reshape(B_c, n_g * D), max(ldg, 8), tdt)
    yu = torch.full((max(B_r, 1), max(ldu, 8)), float("nan"), dtype=tdt, device="cuda")
    yg = torch.full((max(B_c, 1), max(ldg, 8)), float("nan"), dtype=tdt, device="cuda")
    c2r = torch.as_tensor(inp["cand2req"], dtype=torch.int32, device="cuda")
    offs = None if inp.get("offsets") is None else torch.as_tensor(inp["offsets"], dtype=torch.int32, device="cuda")
    desc = R.ugsep_desc(n_u, n_g, D, H, inp["eps"], _layers(inp, tdt, quant))
    need = R.rocs_ugsep_workspace_size(desc, _rdt(R, dtype), B_r, B_c, mode)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    R.rocs_ugsep_forward(desc, R.batch(B_r, B_c, offs, c2r), _rdt(R, dtype), mode, xu, max(ldu, 8), xg, max(ldg, 8),
                         yu, max(ldu, 8), yg, max(ldg, 8), ws, need, R.cur_stream())
    torch.cuda.synchronize()
    y_u = to_np(yu[:B_r, :n_u * D]).reshape(B_r, n_u, D)
    y_g = to_np(yg[:B_c, :n_g * D]).reshape(B_c, n_g, D)
    if pad:  # the padding columns were never written
        assert torch.isnan(yg[:B_c, n_g * D:]).all() and torch.isnan(yu[:B_r, n_u * D:]).all()
    return y_u, y_g


# ------------------------------------------------------------------ steps

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_compensation_matches_oracle(dtype):
    R = _R()
    tdt = _tdt(dtype)
    rng = np.random.default_rng(31)
    B_r, n_u, n_g, D = 37, 3, 5, 64
    xu = S.round_bf16(rng.standard_normal((B_r, n_u, D)).astype(np.float32))
    P = rng.standard_normal((n_g, n_u)).astype(np.float32)
    uc = torch.full((B_r, n_g * D + 4), float("nan"), dtype=torch.float32, device="cuda")
    R.rocs_ugsep_compensation(_rdt(R, dtype), B_r, n_u, n_g, D, dev(xu.reshape(B_r, -1), tdt), n_u * D,
                              torch.as_tensor(P, device="cuda"), uc, n_g * D + 4, R.cur_stream())
    torch.cuda.synchronize()
    ref = U.compensation(xu, P).reshape(B_r, -1)
    assert rel_err(uc[:, :n_g * D].cpu().numpy(), ref) <= 1e-5
    assert torch.isnan(uc[:, n_g * D:]).all()


MIX_CASES = [  # n_u, n_g, dim, dtype, compensation
    (2, 2, 32, "bf16", True),
    (3, 5, 64, "bf16", True),
    (0, 4, 32, "bf16", False),
    (4, 0, 32, "bf16", False),
    (8, 8, 1280, "bf16", True),
    (2, 2, 64, "f32", True),
    (1, 3, 64, "f32", False),
]


@pytest.mark.parametrize("n_u,n_g,D,dtype,comp", MIX_CASES)
def test_mixup_norm_matches_oracle(n_u, n_g, D, dtype, comp):
    R = _R()
    tdt = _tdt(dtype)
    rng = np.random.default_rng(40 + n_u * 3 + n_g + D)
    counts = [3, 0, 70, 17, 1, 9, 40]
    bt = S.make_batch(counts)
    B_r, B_c = len(counts), int(sum(counts))
    xu = S.round_bf16(rng.standard_normal((B_r, n_u, D)).astype(np.float32))
    xg = S.round_bf16(rng.standard_normal((B_c, n_g, D)).astype(np.float32))
    gam = S.round_bf16((1 + 0.1 * rng.standard_normal(D)).astype(np.float32))
    bet = S.round_bf16((0.1 * rng.standard_normal(D)).astype(np.float32))
    P = rng.standard_normal((n_g, n_u)).astype(np.float32) if comp else None
    ldu, ldg = n_u * D + 8, n_g * D + 8
    xu_d, xg_d = _rows(xu.reshape(B_r, n_u * D), ldu, tdt), _rows(xg.reshape(B_c, n_g * D), ldg, tdt)
    uc = None
    if comp:
        uc = torch.empty(B_r, n_g * D, dtype=torch.float32, device="cuda")
        R.rocs_ugsep_compensation(_rdt(R, dtype), B_r, n_u, n_g, D, xu_d, ldu, torch.as_tensor(P, device="cuda"), uc,
                                  n_g * D, R.cur_stream())
    pu = torch.full((B_r, ldu), float("nan"), dtype=tdt, device="cuda")
    pg = torch.full((B_c, ldg), float("nan"), dtype=tdt, device="cuda")
    c2r = torch.as_tensor(bt["cand2req"], dtype=torch.int32, device="cuda")
    R.rocs_ugsep_mixup_norm(R.batch(B_r, B_c, None, c2r), _rdt(R, dtype), n_u, n_g, D, 1e-5, xu_d, ldu, xg_d, ldg, uc,
                            n_g * D, dev(gam, tdt), dev(bet, tdt), pu, ldu, pg, ldg, R.cur_stream())
    torch.cuda.synchronize()
    Xc = U.compensate(np.concatenate([xu[bt["cand2req"]], xg], 1), n_u, P)
    ref_g = U.layer_norm(U.mixup(Xc, n_u), gam, bet, 1e-5)[:, n_u:]
    Xr = np.concatenate([xu, np.zeros((B_r, n_g, D))], 1)
    ref_u = U.layer_norm(U.mixup(Xr, n_u), gam, bet, 1e-5)[:, :n_u]
    t = tol(dtype)
    if n_g:
        assert rel_err(to_np(pg[:, :n_g * D]), ref_g.reshape(B_c, -1)) <= t
        assert torch.isnan(pg[:, n_g * D:]).all()
    if n_u:
        assert rel_err(to_np(pu[:, :n_u * D]), ref_u.reshape(B_r, -1)) <= t
        assert torch.isnan(pu[:, n_u * D:]).all()


# ------------------------------------------------------------------ whole layer stack

FWD_CASES = [  # config, dtype, mode, shuffled, padded leading dimension
    ("tiny", "bf16", 0, False, 0),
    ("tiny", "f32", 0, False, 0),
    ("small", "bf16", 0, False, 0),
    ("small", "bf16", 1, False, 0),
    ("small", "f32", 0, True, 0),
    ("small", "f32", 1, False, 0),
    ("small", "bf16", 0, True, 16),
]


@pytest.mark.parametrize("name,dtype,mode,shuffled,pad", FWD_CASES)
def test_forward_matches_oracle(name, dtype, mode, shuffled, pad):
    inp = S.make_ugsep_inputs(S.ugsep_config(name, dtype), seed=300 + len(name))
    if shuffled:
        inp = S.shuffle_ugsep_candidates(inp, seed=3)
    y_u, y_g = run_forward(inp, dtype, mode, pad)
    ref = U.ugsep_forward(inp)
    t = tol(dtype)
    assert rel_err(y_g, ref["y_g"]) <= t
    if mode == 0:
        assert rel_err(y_u, ref["y_u"]) <= t


def test_shared_and_dense_modes_agree_and_shuffle_permutes():
    inp = S.make_ugsep_inputs(S.ugsep_config("small", "bf16"), seed=17)
    _, g_shared = run_forward(inp, "bf16", 0)
    _, g_dense = run_forward(inp, "bf16", 1)
    assert rel_err(g_dense, g_shared) <= 1e-2  # both sides agree with the oracle to 2e-2; here to each other
    sh = S.shuffle_ugsep_candidates(inp, seed=9)
    u1, g1 = run_forward(inp, "bf16", 0)
    u2, g2 = run_forward(sh, "bf16", 0)
    np.testing.assert_array_equal(g2, g1[sh["perm"]])  # same launch shapes: same bits
    np.testing.assert_array_equal(u2, u1)


def test_forward_edge_cases():
    base = S.ugsep_config("tiny", "bf16")
    # no candidates at all: only the U side runs
    inp = S.make_ugsep_inputs(base, seed=4, counts=[0, 0, 0])
    y_u, y_g = run_forward(inp, "bf16")
    assert y_g.shape[0] == 0
    assert rel_err(y_u, U.ugsep_forward(inp)["y_u"]) <= tol("bf16")
    # no U tokens (nothing shared), and no G tokens (nothing per candidate)
    for n_u, n_g in ((0, 4), (4, 0)):
        cfg = S.UgsepConfig("edge", 3, ("uniform", 0, 30), n_u, n_g, 32, 48, 2, n_u > 0 and n_g > 0, "bf16")
        inp = S.make_ugsep_inputs(cfg, seed=5 + n_u)
        y_u, y_g = run_forward(inp, "bf16")
        ref = U.ugsep_forward(inp)
        if n_g:
            assert rel_err(y_g, ref["y_g"]) <= tol("bf16")
        if n_u:
            assert rel_err(y_u, ref["y_u"]) <= tol("bf16")
    # one layer (outputs written straight from the first layer)
    cfg = S.UgsepConfig("one", 4, ("uniform", 1, 50), 2, 6, 64, 32, 1, True, "f32")
    inp = S.make_ugsep_inputs(cfg, seed=8)
    y_u, y_g = run_forward(inp, "f32")
    ref = U.ugsep_forward(inp)
    assert rel_err(y_g, ref["y_g"]) <= tol("f32") and rel_err(y_u, ref["y_u"]) <= tol("f32")


def test_out_of_range_request_gives_nan_rows():
    inp = S.make_ugsep_inputs(S.ugsep_config("tiny", "f32"), seed=12)
    inp = dict(inp)
    c2r = inp["cand2req"].copy()
    bad = len(c2r) // 2
    c2r[bad] = inp["x_u"].shape[0]  # one past the last request
    inp["cand2req"], inp["offsets"] = c2r, None
    y_u, y_g = run_forward(inp, "f32")
    assert np.isnan(y_g[bad]).all()
    ok = np.arange(len(c2r)) != bad
    ref = U.ugsep_forward(inp, candidates=np.nonzero(ok)[0])
    assert rel_err(y_g[ok], ref["y_g"]) <= tol("f32")


def test_full_size_workload_sampled():
    """The benchmarked workload (8 U + 8 G tokens, width 1280, FFN 2560, 2
    layers, 32 requests with 64..512 candidates) on sampled rows."""
    cfg = S.ugsep_config("tokenmixer")
    inp = S.make_ugsep_inputs(cfg)
    y_u, y_g = run_forward(inp, "bf16", 0)
    assert np.isfinite(y_g).all() and np.isfinite(y_u).all()
    B_c = len(inp["cand2req"])
    rng = np.random.default_rng(1)
    cand = np.unique(np.concatenate([[0, B_c - 1], rng.integers(0, B_c, 22)]))
    req = np.array([0, 7, 31])
    ref = U.ugsep_forward(inp, candidates=cand, requests=req)
    assert rel_err(y_g[cand], ref["y_g"]) <= tol("bf16")
    assert rel_err(y_u[req], ref["y_u"]) <= tol("bf16")


def test_full_size_dense_comparator_sampled():
    """The dense comparator (U tokens copied to every candidate) at the
    benchmarked size, on sampled candidates: it computes the same layer."""
    inp = S.make_ugsep_inputs(S.ugsep_config("tokenmixer"))
    _, y_g = run_forward(inp, "bf16", 1)
    assert np.isfinite(y_g).all()
    B_c = len(inp["cand2req"])
    cand = np.unique(np.concatenate([[0, B_c - 1], np.random.default_rng(2).integers(0, B_c, 14)]))
    ref = U.ugsep_forward(inp, candidates=cand, requests=[])
    assert rel_err(y_g[cand], ref["y_g"]) <= tol("bf16")


# ------------------------------------------------------------------ U side on 8-bit weights

W8_CASES = [  # requests (activation rows of the U side's GEMMs), shuffled candidates
    (5, False),   # up to 16 rows: 16 output channels per workgroup
    (24, True),   # 17..32 rows: one 32-row tile
    (40, False),  # 33..64 rows: two tiles, ragged
    (64, False),  # the largest request count the mode takes
]


@pytest.mark.parametrize("B,shuffled", W8_CASES)
def test_w8a16_u_side_matches_oracle_on_dequantized_weights(B, shuffled):
    """ROCS_UGSEP_SHARED_W8A16 against the oracle TokenMixer whose U tokens'
    FFN weights are the dequantized codes (G outputs read U tokens through
    the Mixup, so both sides are checked)."""
    cfg = S.UgsepConfig("w8", B, ("uniform", 0, 6), 2, 2, 256, 384, 2, True, "bf16")
    inp = S.make_ugsep_inputs(cfg, seed=400 + B)
    if shuffled:
        inp = S.shuffle_ugsep_candidates(inp, seed=5)
    quant = S.make_ugsep_w8a16(inp, seed=410 + B)
    R = _R()
    y_u, y_g = run_forward(inp, "bf16", R.ROCS_UGSEP_SHARED_W8A16, quant=quant)
    ref = U.ugsep_forward(dict(inp, layers=U.with_u_w8a16(inp["layers"], quant, inp["n_u"])))
    assert rel_err(y_u, ref["y_u"]) <= tol("bf16")
    assert rel_err(y_g, ref["y_g"]) <= tol("bf16")
    # the 8-bit weights are the ones used: the bf16 U weights give other outputs
    plain = U.ugsep_forward(inp, requests=[0], candidates=[])
    assert rel_err(y_u[:1], plain["y_u"]) > 10 * tol("bf16")


def test_w8a16_u_side_full_size_sampled():
    """The benchmarked TokenMixer (8 U + 8 G tokens, width 1280, FFN 2560,
    2 layers, 32 requests) with the U side on 8-bit weights, sampled rows."""
    inp = S.make_ugsep_inputs(S.ugsep_config("tokenmixer"))
    quant = S.make_ugsep_w8a16(inp)
    y_u, y_g = run_forward(inp, "bf16", _R().ROCS_UGSEP_SHARED_W8A16, quant=quant)
    assert np.isfinite(y_g).all() and np.isfinite(y_u).all()
    B_c = len(inp["cand2req"])
    cand = np.unique(np.concatenate([[0, B_c - 1], np.random.default_rng(3).integers(0, B_c, 10)]))
    req = np.array([0, 13, 31])
    ref = U.ugsep_forward(dict(inp, layers=U.with_u_w8a16(inp["layers"], quant, inp["n_u"])), candidates=cand,
                          requests=req)
    assert rel_err(y_g[cand], ref["y_g"]) <= tol("bf16")
    assert rel_err(y_u[req], ref["y_u"]) <= tol("bf16")
