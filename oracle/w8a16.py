"""Oracle for the W8A16 linear layer (8-bit float weights, 16-bit activations).

TEST INFRASTRUCTURE ONLY (same rule as the rest of this package).

Citation: [U] "Compute Only Once: UG-Separation for Efficient Large
Recommendation Models" (xllm-io review), §3 framework tree (stage 4: 8-bit
FP8 weights, BF16 activations) and §6 W8A16 configuration table.  The page
names the formats only.  Readings:

W1  FP8 is the E4M3 encoding with no infinities (sign bit, 4 exponent bits
    with bias 7, 3 mantissa bits; exponent field 0 is subnormal, value
    m * 2^-9; the all-ones code S.1111.111 is NaN; the largest finite
    magnitude is 448).
W2  One fp32 scale per output channel: W[n, k] = scale[n] * fp8(code[n, k]).
W3  y = act(x W^T + b): bias in the activation dtype, ReLU or none.

Pins (tests/test_oracle_w8a16.py): every one of the 256 codes against
torch's float8_e4m3fn decode (a library route), hand values from the
format's definition, and the linear layer against a pure-Python loop.
"""

from __future__ import annotations

import numpy as np

F64 = np.float64


def decode_e4m3(codes) -> np.ndarray:
    """Values of E4M3 codes (W1), float64."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(F64)
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(F64) - 7.0)
    sub = sign * m * 2.0 ** -9
    v = np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def dequantize(codes, scale) -> np.ndarray:
    """W[n, k] = scale[n] * fp8(code[n, k]) (W2)."""
    return decode_e4m3(codes) * np.asarray(scale, dtype=F64)[:, None]


def w8a16_linear(x, codes, scale, bias=None, act: int = 0) -> np.ndarray:
    """y = act(x W^T + b) with the dequantized weight (W3)."""
    y = np.asarray(x, dtype=F64) @ dequantize(codes, scale).T
    if bias is not None:
        y = y + np.asarray(bias, dtype=F64)
    return np.maximum(y, 0.0) if act == 1 else y
