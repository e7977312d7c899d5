"""Seeded synthetic inputs for the ROCS shared-forward stack.

This module is the only code shared by the CPU oracle (``oracle/``) and the
HIP path (``request_candidate_sharing_amd``).  It draws random numbers and
lays out the ragged request/candidate batch; it contains none of the method's
arithmetic (no linear maps, norms, interactions or attention).

Workload shapes follow the five stack configurations of the ROCS problem
statement (liuzhao09.github.io ROCS review, section 2 "method" for the
operators; the workload sizes themselves are the benchmark's own).  Every
reading of an unstated detail about the inputs (variance notation, fan-in,
count distributions) is applied here once and documented with the
configuration.  How the layers compose (which encoder depth feeds which
interaction layer, for instance) is not decided here: the oracle and the
stack descriptor each implement that reading on their own.

Conventions
-----------
* N(0, v): the second parameter is a variance, so N(0, 1/fan_in) draws with
  standard deviation fan_in**-0.5.
* fan_in of a GLM linear layer is the full dense input width d_in_r + d_in_c.
* A dense GLM weight is drawn as one ``[d_out_r + d_out_c, d_in_r + d_in_c]``
  matrix.  Its request-output x candidate-input block is drawn like the rest
  and left in place: zeroing it is the operator's job (the mask), not the
  generator's.
* bf16 workloads round every drawn array once, fp32 -> bf16 with
  round-to-nearest-even, and return float32 arrays holding bf16 values.
* Draw order: counts -> x_r -> x_c -> sequence -> weights in layer order.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Any, Dict, Optional

import numpy as np

__all__ = [
    "StackConfig",
    "config",
    "small_config",
    "rrr_config",
    "make_inputs",
    "make_batch",
    "shuffle_candidates",
    "round_bf16",
    "glm_weight",
    "CONFIG_NAMES",
    "UgsepConfig",
    "ugsep_config",
    "make_ugsep_inputs",
    "shuffle_ugsep_candidates",
    "UGSEP_NAMES",
]

CONFIG_NAMES = {
    1: "tiny GLM check (fp32)",
    2: "GLM MLP stack (bf16)",
    3: "DCA sequence block (bf16)",
    4: "Wukong-style ROCSified interaction layer (bf16)",
    5: "ranking-scale full stack (bf16)",
}


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bf16.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return u.view(np.float32).reshape(a.shape)


@dataclasses.dataclass(frozen=True)
class StackConfig:
    """Shape description of one workload.

    kind is one of ``glm_tiny`` (config 1), ``glm_mlp`` (config 2),
    ``dca`` (configs 3 and 5) and ``wukong`` (config 4).
    """

    key: int
    kind: str
    dtype: str  # "f32" or "bf16"
    B: int
    counts: tuple  # ("uniform", lo, hi) | ("fixed", n) | ("lognormal", median, sigma, lo, hi)
    d_r: int = 0
    d_c: int = 0
    hidden: int = 0  # hidden width of the GLM MLPs (candidate group; request group too unless hidden_r)
    hidden_r: int = 0  # request-group hidden width when it differs (request-side scaling r)
    n_blocks: int = 0  # glm_mlp: residual MLP blocks
    # DCA
    L: int = 0
    d_seq: int = 0
    n_heads: int = 0
    head_dim: int = 64
    ffn: int = 0
    n_enc: int = 0
    n_int: int = 0
    qgen_lcb: bool = False  # config 3: an LCB (GLM linear + ReLU) in front of the query MLP
    head: bool = True
    # Wukong-style tokens
    n_tok_r: int = 0
    n_tok_c: int = 0
    tok_dim: int = 0
    tok_out: int = 0  # tokens per group after the token-axis LCB
    x_var: float = 1.0
    eps: float = 1e-5

    def name(self) -> str:
        return CONFIG_NAMES.get(self.key, self.kind)

    @property
    def hid_r(self) -> int:
        """Request-group hidden width of the GLM MLP blocks."""
        return self.hidden_r or self.hidden

    def with_(self, **kw) -> "StackConfig":
        return dataclasses.replace(self, **kw)

    def to_dict(self) -> Dict[str, Any]:
        return dataclasses.asdict(self)


def config(k: int) -> StackConfig:
    """The five benchmark workloads at full size."""
    if k == 1:
        return StackConfig(key=1, kind="glm_tiny", dtype="f32", B=4, counts=("uniform", 1, 16),
                           d_r=32, d_c=32, hidden=32, head=False)
    if k == 2:
        return StackConfig(key=2, kind="glm_mlp", dtype="bf16", B=256, counts=("uniform", 64, 512),
                           d_r=512, d_c=512, hidden=1024, n_blocks=3, head=True)
    if k == 3:
        return StackConfig(key=3, kind="dca", dtype="bf16", B=64, counts=("fixed", 500),
                           d_r=256, d_c=256, hidden=1024, L=256, d_seq=256, n_heads=4, head_dim=64,
                           ffn=1024, n_enc=2, n_int=1, qgen_lcb=True, head=False)
    if k == 4:
        return StackConfig(key=4, kind="wukong", dtype="bf16", B=128,
                           counts=("lognormal", 200.0, 0.5, 16, 1024),
                           n_tok_r=32, n_tok_c=16, tok_dim=128, tok_out=64, hidden=1024,
                           x_var=0.1, head=True)
    if k == 5:
        return StackConfig(key=5, kind="dca", dtype="bf16", B=32,
                           counts=("lognormal", 1000.0, math.log(1.3), 700, 1300),
                           d_r=512, d_c=512, hidden=2048, L=1024, d_seq=512, n_heads=8, head_dim=64,
                           ffn=2048, n_enc=2, n_int=4, qgen_lcb=False, head=True)
    raise ValueError(f"no configuration {k}")


def rrr_config(r: int, n: Optional[int] = None) -> StackConfig:
    """The GLM MLP stack with the request-side path r times as wide.

    Request-oriented resource reallocation (ROCS review, section 2.3) scales
    the request-side width of every module by r: d_R = r * 512 and the
    request-group hidden width r * 1024, the candidate side unchanged.
    ``n`` fixes the candidates per request (otherwise U{64..512}).
    """
    c = config(2)
    counts = ("fixed", n) if n is not None else c.counts
    return c.with_(d_r=r * c.d_r, hidden_r=r * c.hidden, counts=counts)


def small_config(k: int) -> StackConfig:
    """Reduced variants of each workload for CPU-oracle parity at every tile path.

    Same composition and dtype as the full configuration, sizes cut so the
    float64 oracle finishes in about a second while the GPU kernels still
    see several tiles per dimension and ragged tails.
    """
    c = config(k)
    if k == 1:
        return c
    if k == 2:
        return c.with_(B=12, counts=("uniform", 0, 150), d_r=136, d_c=128, hidden=320, n_blocks=2)
    if k == 3:
        return c.with_(B=5, counts=("uniform", 0, 140), d_r=128, d_c=64, hidden=256, L=200, d_seq=128,
                       n_heads=2, ffn=512, n_enc=2, n_int=1)
    if k == 4:
        return c.with_(B=6, counts=("uniform", 0, 90), n_tok_r=8, n_tok_c=4, tok_dim=64, tok_out=16,
                       hidden=256)
    if k == 5:
        return c.with_(B=4, counts=("uniform", 1, 120), d_r=128, d_c=64, hidden=256, L=136, d_seq=128,
                       n_heads=2, ffn=256, n_enc=2, n_int=3)
    raise ValueError(k)


def _draw_counts(rng: np.random.Generator, cfg: StackConfig) -> np.ndarray:
    spec = cfg.counts
    if spec[0] == "uniform":
        return rng.integers(spec[1], spec[2] + 1, cfg.B).astype(np.int64)
    if spec[0] == "fixed":
        return np.full(cfg.B, int(spec[1]), dtype=np.int64)
    if spec[0] == "lognormal":
        median, sigma, lo, hi = spec[1:]
        z = rng.standard_normal(cfg.B)
        return np.clip(np.rint(median * np.exp(sigma * z)), lo, hi).astype(np.int64)
    raise ValueError(spec)


def make_batch(counts) -> Dict[str, np.ndarray]:
    """Ragged batch descriptor from per-request candidate counts.

    Candidates are stored contiguously per request: request b owns rows
    offsets[b] .. offsets[b+1]-1 and cand2req maps each row to its request.
    """
    counts = np.asarray(counts, dtype=np.int64)
    offsets = np.zeros(len(counts) + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    cand2req = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    return {"counts": counts, "offsets": offsets, "cand2req": cand2req}


def _normal(rng, shape, var, bf16):
    a = (rng.standard_normal(shape, dtype=np.float32) * np.float32(math.sqrt(var))).astype(np.float32)
    return round_bf16(a) if bf16 else a


def glm_weight(rng, d_in_r, d_in_c, d_out_r, d_out_c, bf16, fan_in=None):
    """Dense [d_out_r + d_out_c, d_in_r + d_in_c] weight drawn from N(0, 1/fan_in)."""
    fan_in = fan_in if fan_in is not None else (d_in_r + d_in_c)
    return _normal(rng, (d_out_r + d_out_c, d_in_r + d_in_c), 1.0 / fan_in, bf16)


def make_inputs(cfg: StackConfig, seed: Optional[int] = None, counts=None) -> Dict[str, Any]:
    """Draw one batch and one set of weights for ``cfg``.

    seed defaults to 100 + cfg.key.  ``counts`` overrides the drawn
    per-request candidate counts (the draw still happens so that the rest of
    the stream is unchanged).
    """
    seed = 100 + cfg.key if seed is None else seed
    rng = np.random.default_rng(seed)
    bf16 = cfg.dtype == "bf16"
    drawn = _draw_counts(rng, cfg)
    if counts is not None:
        drawn = np.asarray(counts, dtype=np.int64)
        assert len(drawn) == cfg.B
    out: Dict[str, Any] = {"cfg": cfg, "seed": seed}
    out.update(make_batch(drawn))
    Bc = int(drawn.sum())
    w: Dict[str, np.ndarray] = {}
    out["w"] = w

    if cfg.kind in ("glm_tiny", "glm_mlp", "dca"):
        out["x_r"] = _normal(rng, (cfg.B, cfg.d_r), cfg.x_var, bf16)
        out["x_c"] = _normal(rng, (Bc, cfg.d_c), cfg.x_var, bf16)
    elif cfg.kind == "wukong":
        out["x_r"] = _normal(rng, (cfg.B, cfg.n_tok_r, cfg.tok_dim), cfg.x_var, bf16)
        out["x_c"] = _normal(rng, (Bc, cfg.n_tok_c, cfg.tok_dim), cfg.x_var, bf16)
    if cfg.kind == "dca":
        out["seq"] = _normal(rng, (cfg.B, cfg.L, cfg.d_seq), 1.0, bf16)

    zeros = lambda n: np.zeros(n, dtype=np.float32)

    if cfg.kind == "glm_tiny":
        w["lin.W"] = glm_weight(rng, cfg.d_r, cfg.d_c, cfg.hidden, cfg.hidden, bf16)
        w["lin.b"] = zeros(2 * cfg.hidden)
    elif cfg.kind == "glm_mlp":
        for k in range(cfg.n_blocks):
            w[f"blk{k}.up.W"] = glm_weight(rng, cfg.d_r, cfg.d_c, cfg.hid_r, cfg.hidden, bf16)
            w[f"blk{k}.up.b"] = zeros(cfg.hid_r + cfg.hidden)
            w[f"blk{k}.down.W"] = glm_weight(rng, cfg.hid_r, cfg.hidden, cfg.d_r, cfg.d_c, bf16)
            w[f"blk{k}.down.b"] = zeros(cfg.d_r + cfg.d_c)
        w["head.W"] = glm_weight(rng, cfg.d_r, cfg.d_c, 0, 1, bf16)
        w["head.b"] = zeros(1)
    elif cfg.kind == "dca":
        d, f = cfg.d_seq, cfg.ffn
        for k in range(cfg.n_enc):
            w[f"enc{k}.w_qkv"] = _normal(rng, (3 * d, d), 1.0 / d, bf16)
            w[f"enc{k}.b_qkv"] = zeros(3 * d)
            w[f"enc{k}.w_o"] = _normal(rng, (d, d), 1.0 / d, bf16)
            w[f"enc{k}.b_o"] = zeros(d)
            w[f"enc{k}.w_1"] = _normal(rng, (f, d), 1.0 / d, bf16)
            w[f"enc{k}.b_1"] = zeros(f)
            w[f"enc{k}.w_2"] = _normal(rng, (d, f), 1.0 / f, bf16)
            w[f"enc{k}.b_2"] = zeros(d)
        din_r, din_c = cfg.d_r, cfg.d_c
        for i in range(cfg.n_int):
            for nm in ("wk_r", "wv_r", "wk_c", "wv_c"):
                w[f"kv{i}.{nm}"] = _normal(rng, (d, d), 1.0 / d, bf16)
            if cfg.qgen_lcb:
                w[f"int{i}.lcb.W"] = glm_weight(rng, din_r, din_c, din_r, din_c, bf16)
                w[f"int{i}.lcb.b"] = zeros(din_r + din_c)
            w[f"int{i}.mlp1.W"] = glm_weight(rng, din_r, din_c, cfg.hidden, cfg.hidden, bf16)
            w[f"int{i}.mlp1.b"] = zeros(2 * cfg.hidden)
            w[f"int{i}.mlp2.W"] = glm_weight(rng, cfg.hidden, cfg.hidden, d, d, bf16)
            w[f"int{i}.mlp2.b"] = zeros(2 * d)
            din_r, din_c = 2 * d, 2 * d  # next layer reads [G || A]
        if cfg.head:
            w["head.W"] = glm_weight(rng, din_r, din_c, 0, 1, bf16)
            w["head.b"] = zeros(1)
    elif cfg.kind == "wukong":
        nr, nc, D, T, H = cfg.n_tok_r, cfg.n_tok_c, cfg.tok_dim, cfg.tok_out, cfg.hidden
        w["tok.W"] = glm_weight(rng, nr, nc, T, T, bf16)
        u_r = nr * nr + T * D
        u_c = nc * (nr + nc) + T * D
        w["mlp1.W"] = glm_weight(rng, u_r, u_c, H, H, bf16)
        w["mlp1.b"] = zeros(2 * H)
        w["mlp2.W"] = glm_weight(rng, H, H, H, H, bf16)
        w["mlp2.b"] = zeros(2 * H)
        w["head.W"] = glm_weight(rng, H, H, 0, 1, bf16)
        w["head.b"] = zeros(1)
    else:
        raise ValueError(cfg.kind)
    return out


def shuffle_candidates(inputs: Dict[str, Any], seed: int = 7) -> Dict[str, Any]:
    """Same batch with candidate rows in a random global order.

    Returns a shallow copy whose candidate arrays and cand2req are permuted
    and whose offsets are None (candidates no longer contiguous per
    request); ``perm`` maps new row j to old row perm[j].
    """
    rng = np.random.default_rng(seed)
    Bc = len(inputs["cand2req"])
    perm = rng.permutation(Bc)
    out = dict(inputs)
    out["perm"] = perm
    out["cand2req"] = np.ascontiguousarray(inputs["cand2req"][perm])
    out["x_c"] = np.ascontiguousarray(inputs["x_c"][perm])
    out["offsets"] = None
    return out


# ---------------------------------------------------------------------------
# UG-Separation TokenMixer workload ("Compute Only Once: UG-Separation for
# Efficient Large Recommendation Models", xllm-io review).  The token count
# and widths follow the layer shapes of that page's W8A16 latency table
# (16 or 8 tokens, width 1280, FFN width 2560 or 640) at its preferred
# U:G = 1:1 split; the page gives no candidate counts, so the requests and
# their candidate counts are the GLM MLP stack's (uniform in 64..512).

UGSEP_NAMES = {
    "tiny": "UG-Sep TokenMixer, 2 U + 2 G tokens, width 32 (parity)",
    "small": "UG-Sep TokenMixer, 3 U + 5 G tokens, width 64 (parity)",
    "tokenmixer": "UG-Sep TokenMixer, 8 U + 8 G tokens, width 1280, FFN 2560, 2 layers (bf16)",
}


@dataclasses.dataclass(frozen=True)
class UgsepConfig:
    name: str
    B: int
    counts: tuple
    n_u: int
    n_g: int
    dim: int
    hidden: int
    n_layers: int
    comp: bool
    dtype: str  # "f32" | "bf16"
    eps: float = 1e-5

    @property
    def bf16(self) -> bool:
        return self.dtype == "bf16"


def ugsep_config(name: str, dtype: Optional[str] = None) -> UgsepConfig:
    base = {
        "tiny": UgsepConfig("tiny", 4, ("uniform", 0, 9), 2, 2, 32, 48, 2, True, "bf16"),
        "small": UgsepConfig("small", 5, ("uniform", 0, 40), 3, 5, 64, 96, 2, True, "bf16"),
        "tokenmixer": UgsepConfig("tokenmixer", 32, ("uniform", 64, 512), 8, 8, 1280, 2560, 2, True, "bf16"),
    }[name]
    return dataclasses.replace(base, dtype=dtype) if dtype else base


def make_ugsep_inputs(cfg: UgsepConfig, seed: int = 211, counts=None) -> Dict[str, Any]:
    """One batch and one set of layer weights for ``cfg``.

    Token features ~ N(0, 1); per-token FFN weights ~ N(0, 1/fan_in) with
    biases ~ N(0, 0.01); LayerNorm gammas ~ 1 + N(0, 0.01), betas ~ N(0,
    0.01); compensation weights ~ N(0, 1/n_u) (or None).  Draw order: counts
    -> x_u -> x_g -> layers in order (comp, ln1, w1, b1, w2, b2, ln2).
    """
    rng = np.random.default_rng(seed)
    if counts is None:
        spec = cfg.counts
        if spec[0] == "uniform":
            counts = rng.integers(spec[1], spec[2] + 1, cfg.B).astype(np.int64)
        else:
            counts = np.full(cfg.B, int(spec[1]), dtype=np.int64)
    out: Dict[str, Any] = dict(make_batch(counts))
    T, D, H = cfg.n_u + cfg.n_g, cfg.dim, cfg.hidden
    Bc = int(out["offsets"][-1])
    bf = cfg.bf16
    out.update(cfg=cfg, n_u=cfg.n_u, n_g=cfg.n_g, dim=D, hidden=H, eps=cfg.eps)
    out["x_u"] = _normal(rng, (cfg.B, cfg.n_u, D), 1.0, bf)
    out["x_g"] = _normal(rng, (Bc, cfg.n_g, D), 1.0, bf)
    layers = []
    for _ in range(cfg.n_layers):
        p: Dict[str, Any] = {}
        p["comp"] = _normal(rng, (cfg.n_g, cfg.n_u), 1.0 / max(cfg.n_u, 1), False) if cfg.comp and cfg.n_u > 0 else None
        g1 = _normal(rng, (D,), 0.01, False) + 1.0
        p["ln1_g"] = round_bf16(g1) if bf else g1
        p["ln1_b"] = _normal(rng, (D,), 0.01, bf)
        p["w1"] = _normal(rng, (T, H, D), 1.0 / D, bf)
        p["b1"] = _normal(rng, (T, H), 0.01, bf)
        p["w2"] = _normal(rng, (T, D, H), 1.0 / H, bf)
        p["b2"] = _normal(rng, (T, D), 0.01, bf)
        g2 = _normal(rng, (D,), 0.01, False) + 1.0
        p["ln2_g"] = round_bf16(g2) if bf else g2
        p["ln2_b"] = _normal(rng, (D,), 0.01, bf)
        layers.append(p)
    out["layers"] = layers
    return out


def make_ugsep_w8a16(inputs: Dict[str, Any], seed: int = 223) -> list:
    """8-bit weights of the U tokens' FFNs for the UG-Sep W8A16 mode, one
    dict per layer: w1_q [n_u, hidden, dim] and w2_q [n_u, dim, hidden] codes
    drawn uniformly from the finite E4M3 codes (every byte except 0x7F and
    0xFF), and per-output-channel scales w1_scale [n_u, hidden], w2_scale
    [n_u, dim] ~ U(0.5, 1.5) / (100 sqrt(fan_in)) (the finite codes' values
    have an RMS of about 100, so the weights have about the bf16 weights'
    spread).  Draw order: layers in order (w1_q, w1_scale, w2_q, w2_scale)."""
    rng = np.random.default_rng(seed)
    n_u, D, H = int(inputs["n_u"]), int(inputs["dim"]), int(inputs["hidden"])

    def codes(shape):
        c = rng.integers(0, 254, shape).astype(np.uint8)
        return np.where(c >= 0x7F, c + 1, c).astype(np.uint8)  # skip 0x7F; 0xFF is never drawn

    out = []
    for _ in inputs["layers"]:
        q: Dict[str, Any] = {}
        q["w1_q"] = codes((n_u, H, D))
        q["w1_scale"] = (rng.uniform(0.5, 1.5, (n_u, H)) / (100.0 * math.sqrt(D))).astype(np.float32)
        q["w2_q"] = codes((n_u, D, H))
        q["w2_scale"] = (rng.uniform(0.5, 1.5, (n_u, D)) / (100.0 * math.sqrt(H))).astype(np.float32)
        out.append(q)
    return out


def shuffle_ugsep_candidates(inputs: Dict[str, Any], seed: int = 7) -> Dict[str, Any]:
    """Same UG-Sep batch with candidate rows in a random global order (offsets None)."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(len(inputs["cand2req"]))
    out = dict(inputs)
    out["perm"] = perm
    out["cand2req"] = np.ascontiguousarray(inputs["cand2req"][perm])
    out["x_g"] = np.ascontiguousarray(inputs["x_g"][perm])
    out["offsets"] = None
    return out


# ---------------------------------------------------------------------------
# W8A16 linear layer (8-bit float weights, bf16 activations; "Compute Only
# Once: UG-Separation ...", W8A16 configuration).  The page's latency table
# lists layer shapes (batch 1; 16 or 8 tokens; width 1280; 2560 or 640
# outputs).

W8A16_SHAPES = [(16, 1280, 2560), (16, 1280, 640), (8, 1280, 2560), (8, 1280, 640)]  # (M tokens, K, N)


def make_w8a16_inputs(M: int, K: int, N: int, seed: int = 5, bias: bool = True) -> Dict[str, Any]:
    """x ~ N(0, 1) (bf16 values); weight codes drawn uniformly from the
    finite 8-bit E4M3 codes (every byte except the two NaN codes 0x7F and
    0xFF); per-output-channel scales ~ U(0.5, 1.5) / (16 sqrt(K)); bias ~
    N(0, 0.01) (bf16 values).  Draw order: x, codes, scales, bias."""
    rng = np.random.default_rng(seed)
    x = round_bf16(rng.standard_normal((M, K)).astype(np.float32))
    codes = rng.integers(0, 254, (N, K)).astype(np.uint8)
    codes = np.where(codes >= 0x7F, codes + 1, codes).astype(np.uint8)  # skip 0x7F; 0xFF is never drawn
    scale = (rng.uniform(0.5, 1.5, N) / (16.0 * math.sqrt(K))).astype(np.float32)
    b = round_bf16((rng.standard_normal(N) * 0.1).astype(np.float32)) if bias else None
    return {"x": x, "codes": codes, "scale": scale, "bias": b}
