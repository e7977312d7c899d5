"""Pins of the W8A16 oracle (CPU only).  Citation: "Compute Only Once:
UG-Separation for Efficient Large Recommendation Models" (xllm-io review),
§3 stage 4 and the W8A16 configuration table."""

import numpy as np
import pytest

from oracle import w8a16 as W


def test_every_code_matches_torch_float8_e4m3fn():
    torch = pytest.importorskip("torch")
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = W.decode_e4m3(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))  # -0 for 0x80


def test_hand_values_from_the_format():
    v = W.decode_e4m3([0x00, 0x01, 0x07, 0x08, 0x38, 0x39, 0x40, 0x7E, 0xB8, 0xFE])
    np.testing.assert_array_equal(v, [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.125, 2.0, 448.0, -1.0, -448.0])
    assert np.isnan(W.decode_e4m3([0x7F, 0xFF])).all()


def test_linear_matches_scalar_loops():
    rng = np.random.default_rng(3)
    M, N, K = 3, 5, 7
    x = rng.standard_normal((M, K))
    codes = rng.integers(0, 0x7F, (N, K)) | (rng.integers(0, 2, (N, K)) << 7)
    scale = rng.uniform(0.5, 2.0, N)
    b = rng.standard_normal(N)
    got = W.w8a16_linear(x, codes, scale, b, act=1)
    vals = W.decode_e4m3(codes)
    for m in range(M):
        for n in range(N):
            s = sum(float(x[m, k]) * float(scale[n]) * float(vals[n, k]) for k in range(K)) + float(b[n])
            assert abs(got[m, n] - max(s, 0.0)) <= 1e-12 * (1 + abs(s))
