"""Stack descriptors for the five ROCS workloads, built on device memory.

Marshalling only: dense GLM weights are split into the three blocks the
kernels read (W_RR, W_CR, W_CC; the request-output x candidate-input block
W_RC is structurally zero under the mask of the ROCS review's §2.1 and is
never handed to the library), tensors are moved to the GPU, and a
``rocs_stack_desc`` describing the layer sequence is filled in.  All
computation runs in librocs.

Compositions (the pages fix the operators; these stacks are the workloads):
  glm_tiny  LINEAR (64->64), NORM (layer, ReLU after)
  glm_mlp   per block: LINEAR up (ReLU) -> LINEAR down (+ residual x) ->
            NORM (rms), then HEAD
  dca       per interaction layer: [LINEAR lcb (ReLU)] -> LINEAR mlp1 (ReLU)
            -> LINEAR mlp2 = G into columns [0, d) -> XATTN into columns
            [d, 2d) of the same slot; optional HEAD
  wukong    FM and TOKEN_LCB writing adjacent columns of u -> LINEAR (ReLU)
            -> NORM (layer) -> LINEAR (ReLU, + residual) -> NORM -> HEAD
"""

from __future__ import annotations

import ctypes
from typing import Any, Dict, List, Optional

import numpy as np

from . import rocs as R


def _torch():
    import torch

    return torch


def encoder_depths(n_enc: int, n_int: int) -> list:
    """Encoder output index (1..n_enc) read by each interaction layer's K/V.

    Depth i of n_int pairs with encoder output ceil(i * n_enc / n_int) (the
    ROCS review, section 2.2, pairs depth i with the i-th encoder output;
    with fewer encoder layers the depths are spread evenly).
    """
    return [((i + 1) * n_enc + n_int - 1) // n_int for i in range(n_int)]


class DeviceStack:
    """One workload's inputs, weights, descriptor and outputs on a GPU."""

    def __init__(self, inputs: Dict[str, Any], device="cuda", mode: int = R.ROCS_EXEC_SHARED, fusion: bool = False):
        self.flags = R.ROCS_STACK_FUSE_MLP if fusion else 0
        torch = _torch()
        self.torch = torch
        self.inputs = inputs
        cfg = inputs["cfg"]
        self.cfg = cfg
        self.device = torch.device(device)
        self.mode = mode
        self.tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
        self.rdt = R.ROCS_F32 if cfg.dtype == "f32" else R.ROCS_BF16
        self._keep: List[Any] = []
        self.B_r = cfg.B
        self.B_c = int(len(inputs["cand2req"]))
        dev = self.device
        self.cand2req = torch.as_tensor(np.asarray(inputs["cand2req"], dtype=np.int32), device=dev)
        self.offsets = None
        if inputs.get("offsets") is not None:
            self.offsets = torch.as_tensor(np.asarray(inputs["offsets"], dtype=np.int32), device=dev)
        self.batch = R.batch(self.B_r, self.B_c, self.offsets, self.cand2req)

        xr = np.asarray(inputs["x_r"], dtype=np.float32)
        xc = np.asarray(inputs["x_c"], dtype=np.float32)
        self.x_r = self.t(xr.reshape(self.B_r, -1))
        self.x_c = self.t(xc.reshape(self.B_c, -1)) if self.B_c > 0 else self.t(np.zeros((1, xr[0].size), np.float32))
        self.seq = self.t(inputs["seq"].reshape(self.B_r * cfg.L, cfg.d_seq)) if cfg.kind == "dca" else None

        self.slots: List[tuple] = []
        self.layers: List[R.rocs_layer] = []
        self.dca = None
        getattr(self, "_build_" + cfg.kind)()
        self._finish()

    # ------------------------------------------------------------ helpers
    def t(self, a, dtype=None) -> Any:
        torch = self.torch
        x = torch.as_tensor(np.ascontiguousarray(a), device=self.device).to(dtype or self.tdt).contiguous()
        self._keep.append(x)
        return x

    def glm_blocks(self, W, b, d_in_r, d_out_r):
        W = np.asarray(W, dtype=np.float32)
        w_rr = self.t(W[:d_out_r, :d_in_r]) if d_out_r > 0 else None
        w_cr = self.t(W[d_out_r:, :d_in_r])
        w_cc = self.t(W[d_out_r:, d_in_r:])
        b_r = b_c = None
        if b is not None:
            b = np.asarray(b, dtype=np.float32)
            b_r = self.t(b[:d_out_r]) if d_out_r > 0 else None
            b_c = self.t(b[d_out_r:])
        return w_rr, w_cr, w_cc, b_r, b_c

    def slot(self, wr, wc) -> int:
        self.slots.append((int(wr), int(wc)))
        return len(self.slots) - 1

    def layer(self, **kw) -> R.rocs_layer:
        L = R.rocs_layer()
        L.res = -1
        for k, v in kw.items():
            if k in ("w_rr", "w_cr", "w_cc", "b_r", "b_c", "gamma_r", "beta_r", "gamma_c", "beta_c"):
                v = R.ptr(v)
            setattr(L, k, v)
        self.layers.append(L)
        return L

    def linear(self, src, dst, W, b, d_in, d_out, act=R.ROCS_ACT_NONE, res=-1, src_col=(0, 0), dst_col=(0, 0),
               res_col=(0, 0)):
        w_rr, w_cr, w_cc, b_r, b_c = self.glm_blocks(W, b, d_in[0], d_out[0])
        self.layer(kind=R.ROCS_OP_LINEAR, src=src, src_col_r=src_col[0], src_col_c=src_col[1], dst=dst,
                   dst_col_r=dst_col[0], dst_col_c=dst_col[1], res=res, res_col_r=res_col[0], res_col_c=res_col[1],
                   d_in_r=d_in[0], d_in_c=d_in[1], d_out_r=d_out[0], d_out_c=d_out[1], act=act, w_rr=w_rr, w_cr=w_cr,
                   w_cc=w_cc, b_r=b_r, b_c=b_c)

    def norm(self, src, dst, widths, kind, act=R.ROCS_ACT_NONE, res=-1):
        self.layer(kind=R.ROCS_OP_NORM, src=src, dst=dst, res=res, d_in_r=widths[0], d_in_c=widths[1], act=act,
                   norm=kind, eps=float(self.cfg.eps))

    def head(self, src, d_in):
        W = np.asarray(self.inputs["w"]["head.W"], dtype=np.float32)
        b = np.asarray(self.inputs["w"]["head.b"], dtype=np.float32)
        self.layer(kind=R.ROCS_OP_HEAD, src=src, d_in_r=d_in[0], d_in_c=d_in[1], d_out_c=1,
                   w_cr=self.t(W[0, :d_in[0]]), w_cc=self.t(W[0, d_in[0]:]), b_c=self.t(b))

    # ------------------------------------------------------------ workloads
    def _build_glm_tiny(self):
        c, w = self.cfg, self.inputs["w"]
        s0 = self.slot(c.d_r, c.d_c)
        s1 = self.slot(c.hidden, c.hidden)
        s2 = self.slot(c.hidden, c.hidden)
        self.linear(s0, s2, w["lin.W"], w["lin.b"], (c.d_r, c.d_c), (c.hidden, c.hidden))
        self.norm(s2, s1, (c.hidden, c.hidden), R.ROCS_NORM_LAYER, act=R.ROCS_ACT_RELU)
        self.has_head = False

    def _build_glm_mlp(self):
        c, w = self.cfg, self.inputs["w"]
        d, H = (c.d_r, c.d_c), (c.hidden_r or c.hidden, c.hidden)
        s0 = self.slot(*d)
        s1 = self.slot(*d)
        sh = self.slot(*H)
        st = self.slot(*d)
        cur = s0
        for k in range(c.n_blocks):
            self.linear(cur, sh, w[f"blk{k}.up.W"], w[f"blk{k}.up.b"], d, H, act=R.ROCS_ACT_RELU)
            self.linear(sh, st, w[f"blk{k}.down.W"], w[f"blk{k}.down.b"], H, d, res=cur)
            self.norm(st, s1, d, R.ROCS_NORM_RMS)
            cur = s1
        self.head(s1, d)
        self.has_head = True

    def _build_dca(self):
        c, w = self.cfg, self.inputs["w"]
        dq, H = c.d_seq, c.hidden
        s0 = self.slot(c.d_r, c.d_c)
        s1 = self.slot(2 * dq, 2 * dq)
        s_lcb = self.slot(c.d_r, c.d_c) if c.qgen_lcb else None
        s_h = self.slot(H, H)
        s_y = [self.slot(2 * dq, 2 * dq), self.slot(2 * dq, 2 * dq)]
        src, din = s0, (c.d_r, c.d_c)
        for i in range(c.n_int):
            out = s1 if i == c.n_int - 1 else s_y[i % 2]
            if c.qgen_lcb:
                self.linear(src, s_lcb, w[f"int{i}.lcb.W"], w[f"int{i}.lcb.b"], din, din, act=R.ROCS_ACT_RELU)
                src = s_lcb
            self.linear(src, s_h, w[f"int{i}.mlp1.W"], w[f"int{i}.mlp1.b"], din, (H, H), act=R.ROCS_ACT_RELU)
            self.linear(s_h, out, w[f"int{i}.mlp2.W"], w[f"int{i}.mlp2.b"], (H, H), (dq, dq))
            self.layer(kind=R.ROCS_OP_XATTN, src=out, dst=out, dst_col_r=dq, dst_col_c=dq, depth=i)
            src, din = out, (2 * dq, 2 * dq)
        self.has_head = bool(c.head)
        if c.head:
            self.head(s1, din)
        # request-only encoder and per-depth K/V weights
        enc = (R.rocs_enc_layer * max(1, c.n_enc))()
        for k in range(c.n_enc):
            e = enc[k]
            for nm in ("w_qkv", "b_qkv", "w_o", "b_o", "w_1", "b_1", "w_2", "b_2"):
                setattr(e, nm, R.ptr(self.t(w[f"enc{k}.{nm}"])))
        kvw = (R.rocs_kv_w * c.n_int)()
        for i in range(c.n_int):
            for nm in ("wk_r", "wv_r", "wk_c", "wv_c"):
                setattr(kvw[i], nm, R.ptr(self.t(w[f"kv{i}.{nm}"])))
        src_arr = (ctypes.c_int32 * c.n_int)(*encoder_depths(c.n_enc, c.n_int))
        self._dca_arrays = (enc, kvw, src_arr)
        self.dca = R.rocs_dca_desc(c.L, dq, c.n_heads, c.ffn, c.n_enc, enc, c.n_int, src_arr, kvw)

    def _build_wukong(self):
        c, w = self.cfg, self.inputs["w"]
        nr, nc, D, T, H = c.n_tok_r, c.n_tok_c, c.tok_dim, c.tok_out, c.hidden
        fr, fc = nr * nr, nc * (nr + nc)
        ur, uc = fr + T * D, fc + T * D
        s0 = self.slot(nr * D, nc * D)
        s1 = self.slot(H, H)
        su = self.slot(ur, uc)
        s3 = self.slot(H, H)
        self.layer(kind=R.ROCS_OP_FM, src=s0, dst=su, n_r=nr, n_c=nc, dim=D)
        Wt = np.asarray(w["tok.W"], dtype=np.float32)
        self.layer(kind=R.ROCS_OP_TOKEN_LCB, src=s0, dst=su, dst_col_r=fr, dst_col_c=fc, n_r=nr, n_c=nc, dim=D,
                   d_out_r=T, d_out_c=T, w_rr=self.t(Wt[:T, :nr]), w_cr=self.t(Wt[T:, :nr]), w_cc=self.t(Wt[T:, nr:]))
        self.linear(su, s3, w["mlp1.W"], w["mlp1.b"], (ur, uc), (H, H), act=R.ROCS_ACT_RELU)
        self.norm(s3, s3, (H, H), R.ROCS_NORM_LAYER)
        self.linear(s3, s1, w["mlp2.W"], w["mlp2.b"], (H, H), (H, H), act=R.ROCS_ACT_RELU, res=s3)
        self.norm(s1, s1, (H, H), R.ROCS_NORM_LAYER)
        self.head(s1, (H, H))
        self.has_head = True

    # ------------------------------------------------------------ descriptor / run
    def _finish(self):
        torch = self.torch
        n = len(self.slots)
        self._slot_arr = (R.rocs_slot * n)(*[R.rocs_slot(a, b) for a, b in self.slots])
        self._layer_arr = (R.rocs_layer * len(self.layers))(*self.layers)
        self.desc = R.rocs_stack_desc(self.rdt, self.mode, n, self._slot_arr, len(self.layers), self._layer_arr,
                                      ctypes.pointer(self.dca) if self.dca is not None else None, self.flags)
        wr1, wc1 = self.slots[1]
        self.y_r = torch.empty((self.B_r, wr1), dtype=self.tdt, device=self.device)
        self.y_c = torch.empty((max(self.B_c, 1), wc1), dtype=self.tdt, device=self.device)
        self.logits = torch.empty((max(self.B_c, 1),), dtype=torch.float32, device=self.device)
        self.io = R.rocs_stack_io(R.ptr(self.x_r), self.x_r.shape[1], R.ptr(self.x_c), self.x_c.shape[1],
                                  R.ptr(self.y_r), wr1, R.ptr(self.y_c), wc1, R.ptr(self.seq), R.ptr(self.logits))
        self.ws_bytes = R.rocs_stack_workspace_size(self.desc, self.B_r, self.B_c)
        if self.ws_bytes == 0:
            raise R.RocsError(R.ROCS_ERR_INVALID_ARG, R.last_error())
        self.ws = torch.empty((self.ws_bytes,), dtype=torch.uint8, device=self.device)

    def run(self, stream: Optional[int] = None):
        s = R.cur_stream() if stream is None else stream
        R.rocs_stack_forward(self.desc, self.batch, self.io, self.ws, self.ws_bytes, s)

    def outputs(self) -> Dict[str, np.ndarray]:
        torch = self.torch
        torch.cuda.synchronize()
        out = {"y_r": self.y_r.float().cpu().numpy(), "y_c": self.y_c[: self.B_c].float().cpu().numpy()}
        out["logits"] = self.logits[: self.B_c].cpu().numpy() if self.has_head else None
        return out


class DeviceUgsep:
    """The UG-Separation TokenMixer workload ("Compute Only Once:
    UG-Separation for Efficient Large Recommendation Models", xllm-io review,
    §3) on a GPU: token rows, per-layer weights, descriptor, workspace and
    outputs.  Marshalling only; rocs_ugsep_forward does the work."""

    def __init__(self, inputs: Dict[str, Any], device="cuda", mode: int = R.ROCS_UGSEP_SHARED, quant=None):
        """``quant``: per-layer dicts of the U tokens' 8-bit weights (w1_q,
        w1_scale, w2_q, w2_scale) for ROCS_UGSEP_SHARED_W8A16."""
        torch = _torch()
        self.inputs, self.mode = inputs, mode
        cfg = inputs["cfg"]
        self.dtype = R.ROCS_BF16 if cfg.dtype == "bf16" else R.ROCS_F32
        tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        n_u, n_g, D, H = inputs["n_u"], inputs["n_g"], inputs["dim"], inputs["hidden"]
        self.B_r, self.B_c = inputs["x_u"].shape[0], inputs["x_g"].shape[0]

        def t(a, dt=tdt):
            return torch.as_tensor(np.ascontiguousarray(a, dtype=np.float32), device=device).to(dt).contiguous()

        self.x_u = t(np.asarray(inputs["x_u"]).reshape(self.B_r, n_u * D))
        self.x_g = t(np.asarray(inputs["x_g"]).reshape(self.B_c, n_g * D))
        self.y_u = torch.empty(max(self.B_r, 1), max(n_u * D, 8), dtype=tdt, device=device)
        self.y_g = torch.empty(max(self.B_c, 1), max(n_g * D, 8), dtype=tdt, device=device)
        self.c2r = torch.as_tensor(inputs["cand2req"], dtype=torch.int32, device=device)
        offs = inputs.get("offsets")
        self.offs = None if offs is None else torch.as_tensor(offs, dtype=torch.int32, device=device)
        layers = []
        for p in inputs["layers"]:
            d = {k: t(p[k]) for k in ("ln1_g", "ln1_b", "w1", "b1", "w2", "b2", "ln2_g", "ln2_b")}
            d["comp"] = None if p["comp"] is None else t(p["comp"], torch.float32)
            layers.append(d)
        for d, q in zip(layers, quant or ()):
            for k in ("w1_q", "w2_q"):
                d[k] = torch.as_tensor(np.ascontiguousarray(q[k], dtype=np.uint8), device=device)
            for k in ("w1_scale", "w2_scale"):
                d[k] = t(q[k], torch.float32)
        self.desc = R.ugsep_desc(n_u, n_g, D, H, inputs["eps"], layers)
        self.batch = R.batch(self.B_r, self.B_c, self.offs, self.c2r)
        self.ws_bytes = R.rocs_ugsep_workspace_size(self.desc, self.dtype, self.B_r, self.B_c, mode)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=device)
        self.ld_u, self.ld_g = max(n_u * D, 8), max(n_g * D, 8)

    def run(self, stream: Optional[int] = None):
        R.rocs_ugsep_forward(self.desc, self.batch, self.dtype, self.mode, self.x_u, self.ld_u, self.x_g, self.ld_g,
                             self.y_u, self.ld_u, self.y_g, self.ld_g, self.ws, self.ws_bytes,
                             R.cur_stream() if stream is None else stream)
