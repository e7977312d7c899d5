"""rocs_dca_cross_attn_noalloc (no workspace, static scratch) against
rocs_dca_cross_attn (caller workspace) through the C ABI: two calls in a row
on one GPU, the second with a smaller batch, both in random candidate order
(the plan's per-request counts live in the shared static array and must be
cleared by each call).  Each result is also checked against the oracle's
attention."""

import numpy as np
import pytest

import rocs_synth as S
from gpu_util import TOL_BF16, dev, rand, rel_err, to_np
from oracle import ops

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _case(counts, L, H, seed):
    from request_candidate_sharing_amd import rocs as R

    rng = np.random.default_rng(seed)
    d = H * 64
    bt = S.make_batch(counts)
    B, Bc = len(counts), int(sum(counts))
    q_r, q_c = rand(rng, (B, d), True), rand(rng, (Bc, d), True)
    kv = rand(rng, (B * L, 4 * d), True)  # [K_R | V_R | K_C | V_C] per event
    perm = np.random.default_rng(seed + 1).permutation(Bc)
    m = bt["cand2req"]
    kvt = dev(kv, torch.bfloat16)
    qr_t, qc_t = dev(q_r, torch.bfloat16), dev(q_c[perm], torch.bfloat16)
    c2r = torch.as_tensor(m[perm].astype(np.int32), device="cuda")
    batch = R.batch(B, Bc, None, c2r)
    outs = []
    for noalloc in (False, True):
        ar = torch.full((B, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        ac = torch.full((max(Bc, 1), d), float("nan"), dtype=torch.bfloat16, device="cuda")
        args = (batch, R.ROCS_BF16, H, 64, L, qr_t, d, qc_t, d, kvt, kvt[:, d:], kvt[:, 2 * d:], kvt[:, 3 * d:], 4 * d,
                0.0, ar, d, ac, d)
        if noalloc:
            print(f"no-alloc call: counts={counts} L={L} H={H}", flush=True)
            R.rocs_dca_cross_attn_noalloc(*args, R.cur_stream())
        else:
            wsb = R.rocs_dca_cross_attn_workspace_size(B, Bc, H, L)
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            R.rocs_dca_cross_attn(*args, ws, wsb, R.cur_stream())
        torch.cuda.synchronize()
        outs.append((to_np(ar), to_np(ac[:Bc])))
    K = kv.reshape(B, L, 4 * d)
    ref_r = ops.attention(q_r[:, None, :], K[:, :, :d], K[:, :, d:2 * d], H)[:, 0]
    ref_c = ops.attention(q_c[perm][:, None, :], K[m[perm]][:, :, 2 * d:3 * d], K[m[perm]][:, :, 3 * d:], H)[:, 0]
    return outs, ref_r, ref_c


def test_noalloc_cross_attention_matches_workspace_entry_point_twice():
    for counts, L, H, seed in (([300, 5, 129, 0, 64, 211], 200, 2, 3), ([3, 40], 64, 1, 4)):
        outs, ref_r, ref_c = _case(counts, L, H, seed)
        (wr, wc), (nr, nc) = outs
        print(f"bitwise equal to the workspace entry point: {np.array_equal(nr, wr) and np.array_equal(nc, wc)}")
        assert np.all(np.isfinite(nr)) and np.all(np.isfinite(nc))
        assert rel_err(nr, wr) <= TOL_BF16 and rel_err(nc, wc) <= TOL_BF16
        assert rel_err(nc, ref_c) <= TOL_BF16 and rel_err(nr, ref_r) <= TOL_BF16
