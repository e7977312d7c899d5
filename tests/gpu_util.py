"""Helpers shared by the GPU parity tests (no method arithmetic here)."""

import numpy as np

import rocs_synth as S

TOL_F32 = 1e-5  # max|gpu - oracle| / max|oracle|, fp32 path
TOL_BF16 = 2e-2  # same metric, bf16 storage with fp32 accumulation


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    scale = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (scale if scale > 0 else 1.0)


def tol(dtype: str) -> float:
    return TOL_F32 if dtype == "f32" else TOL_BF16


def dev(a, dtype, device="cuda"):
    import torch

    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.float32), device=device).to(dtype).contiguous()


def to_np(t):
    return t.float().cpu().numpy()


def ragged(counts, rng=None):
    return S.make_batch(counts)


def rand(rng, shape, bf16, scale=1.0):
    a = (rng.standard_normal(shape) * scale).astype(np.float32)
    return S.round_bf16(a) if bf16 else a
