"""ctypes binding of librocs: the C-ABI entry points under the same names.

Argument marshalling only: tensors become device pointers, enums become
ints, the current torch stream becomes the hipStream_t.  Every computation
happens in librocs's HIP kernels.  If the built library is missing this
module raises on first use: there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Any, Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librocs.so")

ROCS_OK = 0
ROCS_ERR_INVALID_ARG = -1
ROCS_ERR_SHAPE = -2
ROCS_ERR_DTYPE = -3
ROCS_ERR_ALIGN = -4
ROCS_ERR_WORKSPACE = -5
ROCS_ERR_BATCH = -6
ROCS_ERR_HIP = -7
ROCS_ERR_UNSUPPORTED = -8

ROCS_F32, ROCS_BF16 = 0, 1
ROCS_ACT_NONE, ROCS_ACT_RELU = 0, 1
ROCS_NORM_LAYER, ROCS_NORM_RMS = 0, 1
ROCS_EXEC_SHARED, ROCS_EXEC_DENSE_BROADCAST, ROCS_EXEC_SHARED_SERIAL, ROCS_EXEC_SHARED_FUSED = 0, 1, 2, 3
ROCS_OP_LINEAR, ROCS_OP_NORM, ROCS_OP_FM, ROCS_OP_TOKEN_LCB, ROCS_OP_XATTN, ROCS_OP_HEAD = 1, 2, 3, 4, 5, 6

c_int32, c_int64, c_size_t, c_float, c_void_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p


class rocs_batch(ctypes.Structure):
    _fields_ = [("num_requests", c_int32), ("num_candidates", c_int32), ("offsets", c_void_p), ("cand2req", c_void_p)]


class rocs_enc_layer(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("w_qkv", "b_qkv", "w_o", "b_o", "ln1_g", "ln1_b", "w_1", "b_1", "w_2", "b_2",
                                        "ln2_g", "ln2_b")]


class rocs_kv_w(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("wk_r", "wv_r", "wk_c", "wv_c")]


class rocs_layer(ctypes.Structure):
    _fields_ = [
        ("kind", c_int32),
        ("src", c_int32), ("src_col_r", c_int32), ("src_col_c", c_int32),
        ("dst", c_int32), ("dst_col_r", c_int32), ("dst_col_c", c_int32),
        ("res", c_int32), ("res_col_r", c_int32), ("res_col_c", c_int32),
        ("d_in_r", c_int32), ("d_in_c", c_int32), ("d_out_r", c_int32), ("d_out_c", c_int32),
        ("act", c_int32), ("norm", c_int32), ("eps", c_float), ("depth", c_int32),
        ("n_r", c_int32), ("n_c", c_int32), ("dim", c_int32),
        ("w_rr", c_void_p), ("w_cr", c_void_p), ("w_cc", c_void_p),
        ("b_r", c_void_p), ("b_c", c_void_p),
        ("gamma_r", c_void_p), ("beta_r", c_void_p), ("gamma_c", c_void_p), ("beta_c", c_void_p),
    ]


class rocs_slot(ctypes.Structure):
    _fields_ = [("width_r", c_int32), ("width_c", c_int32)]


class rocs_dca_desc(ctypes.Structure):
    _fields_ = [
        ("L", c_int32), ("d", c_int32), ("n_heads", c_int32), ("ffn", c_int32),
        ("n_enc", c_int32), ("enc", ctypes.POINTER(rocs_enc_layer)),
        ("n_depths", c_int32), ("depth_src", ctypes.POINTER(c_int32)),
        ("kvw", ctypes.POINTER(rocs_kv_w)),
    ]


class rocs_stack_desc(ctypes.Structure):
    _fields_ = [
        ("dtype", c_int32), ("mode", c_int32),
        ("n_slots", c_int32), ("slots", ctypes.POINTER(rocs_slot)),
        ("n_layers", c_int32), ("layers", ctypes.POINTER(rocs_layer)),
        ("dca", ctypes.POINTER(rocs_dca_desc)),
        ("flags", ctypes.c_uint32),
    ]


ROCS_STACK_FUSE_MLP = 1


class rocs_stack_io(ctypes.Structure):
    _fields_ = [
        ("x_r", c_void_p), ("ld_xr", c_int64), ("x_c", c_void_p), ("ld_xc", c_int64),
        ("y_r", c_void_p), ("ld_yr", c_int64), ("y_c", c_void_p), ("ld_yc", c_int64),
        ("seq", c_void_p), ("logits", c_void_p),
    ]


class rocs_ugsep_layer(ctypes.Structure):
    _fields_ = [
        ("comp", c_void_p), ("ln1_gamma", c_void_p), ("ln1_beta", c_void_p), ("w1", c_void_p), ("b1", c_void_p),
        ("w2", c_void_p), ("b2", c_void_p), ("ln2_gamma", c_void_p), ("ln2_beta", c_void_p),
        ("w1_q", c_void_p), ("w1_scale", c_void_p), ("w2_q", c_void_p), ("w2_scale", c_void_p),
    ]


class rocs_ugsep_desc(ctypes.Structure):
    _fields_ = [
        ("n_u", c_int32), ("n_g", c_int32), ("dim", c_int32), ("hidden", c_int32), ("n_layers", c_int32),
        ("eps", c_float), ("layers", ctypes.POINTER(rocs_ugsep_layer)),
    ]


ROCS_UGSEP_SHARED = 0
ROCS_UGSEP_DENSE = 1
ROCS_UGSEP_SHARED_W8A16 = 2


class RocsError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_name(status)} ({status}): {msg}")
        self.status = status


_lib: Optional[ctypes.CDLL] = None

P = c_void_p
_SIGS = {
    "rocs_lcb_request": [c_int32, c_int32, P, c_int64, c_int32, P, P, P, c_int32, c_int32, c_int32, P, c_int64, P,
                         c_int64, P, c_int64, P],
    "rocs_lcb_candidate": [P, c_int32, P, c_int64, c_int32, P, P, c_int32, c_int32, P, c_int64, P, c_int64, P,
                           c_int64, P],
    "rocs_lcb_forward": [P, c_int32, P, c_int64, c_int32, P, c_int64, c_int32, P, P, P, P, P, c_int32, c_int32,
                         c_int32, P, c_int64, P, c_int64, P, c_int64, P, c_int64, P, c_int64, P],
    "rocs_lcb_fused_workspace_size": [c_int32],
    "rocs_lcb_forward_fused": [P, c_int32, P, c_int64, c_int32, P, c_int64, c_int32, P, P, P, P, P, c_int32, c_int32,
                               c_int32, P, c_int64, P, c_int64, P, c_int64, P, c_int64, P, c_int64, P, c_size_t, P],
    "rocs_head_forward": [P, c_int32, P, c_int64, c_int32, P, c_int64, c_int32, P, P, c_float, P, P, P],
    "rocs_group_norm": [c_int32, c_int32, c_float, c_int32, c_int32, c_int32, c_int32, P, c_int64, P, c_int64, P, P,
                        P, P, P, P, c_int32, P, c_int64, P, c_int64, P],
    "rocs_fm_masked": [P, c_int32, c_int32, c_int32, c_int32, P, c_int64, P, c_int64, P, c_int64, P, c_int64, P],
    "rocs_token_lcb": [P, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, P, c_int64, P, c_int64, P, P, P, P,
                       c_int64, P, c_int64, P, P],
    "rocs_dca_encode_kv_workspace_size": [c_int32, c_int32, c_int32, c_int32, c_int32],
    "rocs_dca_encode_kv": [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, P, c_int32, P, c_int32, P, P, P, P,
                           c_size_t, P],
    "rocs_dca_cross_attn_workspace_size": [c_int32, c_int32, c_int32, c_int32],
    "rocs_dca_request_attn_workspace_size": [c_int32, c_int32, c_int32],
    "rocs_dca_request_attn": [c_int32, c_int32, c_int32, c_int32, P, c_int64, P, c_int64, P, P, c_float, P, c_int64, P,
                              c_size_t, P],
    "rocs_dca_cross_attn": [P, c_int32, c_int32, c_int32, c_int32, P, c_int64, P, c_int64, P, P, P, P, c_int64,
                            c_float, P, c_int64, P, c_int64, P, c_size_t, P],
    "rocs_dca_cross_attn_noalloc": [P, c_int32, c_int32, c_int32, c_int32, P, c_int64, P, c_int64, P, P, P, P, c_int64,
                            c_float, P, c_int64, P, c_int64, P],
    "rocs_broadcast_rows": [P, c_int64, P, c_int64, P, c_int64, P],
    "rocs_stack_workspace_size": [P, c_int32, c_int32],
    "rocs_stack_forward": [P, P, P, P, c_size_t, P],
    "rocs_ugsep_compensation": [c_int32, c_int32, c_int32, c_int32, c_int32, P, c_int64, P, P, c_int64, P],
    "rocs_ugsep_mixup_norm": [P, c_int32, c_int32, c_int32, c_int32, c_float, P, c_int64, P, c_int64, P, c_int64, P,
                              P, P, c_int64, P, c_int64, P],
    "rocs_ugsep_workspace_size": [P, c_int32, c_int32, c_int32, c_int32],
    "rocs_ugsep_forward": [P, P, c_int32, c_int32, P, c_int64, P, c_int64, P, c_int64, P, c_int64, P, c_size_t, P],
    "rocs_w8a16_linear": [c_int32, c_int32, c_int32, P, c_int64, P, c_int64, P, P, c_int32, P, c_int64, P],
    "rocs_validate_batch": [P, P],
    "rocs_status_str": [ctypes.c_int],
    "rocs_last_error": [],
    "rocs_version": [],
}
_RES = {
    "rocs_lcb_fused_workspace_size": c_size_t,
    "rocs_dca_encode_kv_workspace_size": c_size_t,
    "rocs_dca_cross_attn_workspace_size": c_size_t,
    "rocs_dca_request_attn_workspace_size": c_size_t,
    "rocs_stack_workspace_size": c_size_t,
    "rocs_ugsep_workspace_size": c_size_t,
    "rocs_status_str": ctypes.c_char_p,
    "rocs_last_error": ctypes.c_char_p,
}
EXPORTED = tuple(_SIGS)


def lib() -> ctypes.CDLL:
    """Loads librocs.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"librocs is not built ({LIB_PATH} missing); run `python -m request_candidate_sharing_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = _RES.get(name, ctypes.c_int)
        _lib = L
    return _lib


def status_name(status: int) -> str:
    return lib().rocs_status_str(int(status)).decode()


def last_error() -> str:
    return lib().rocs_last_error().decode()


def _check(status: int) -> int:
    if status != ROCS_OK:
        raise RocsError(status, last_error())
    return status


def ptr(t: Any) -> Optional[int]:
    """Device/host address of a tensor (None stays NULL, ints pass through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def cur_stream() -> Optional[int]:
    import torch

    return torch.cuda.current_stream().cuda_stream


def batch(num_requests: int, num_candidates: int, offsets=None, cand2req=None) -> rocs_batch:
    """rocs_batch for device tensors; the struct keeps the tensors alive with it."""
    b = rocs_batch(int(num_requests), int(num_candidates), ptr(offsets), ptr(cand2req))
    b._keep = (offsets, cand2req)
    return b


def _b(b: rocs_batch):
    return ctypes.byref(b)


# ---------------------------------------------------------------- entry points (same names as the C ABI)


def rocs_lcb_request(dtype, B_r, x_r, ld_xr, d_in_r, w_rr, w_cr, b_r, d_out_r, d_out_c, act, res_r, ld_resr, y_r,
                     ld_yr, z, ld_z, stream=None, check=True):
    st = lib().rocs_lcb_request(dtype, B_r, ptr(x_r), ld_xr, d_in_r, ptr(w_rr), ptr(w_cr), ptr(b_r), d_out_r, d_out_c,
                                act, ptr(res_r), ld_resr, ptr(y_r), ld_yr, ptr(z), ld_z, stream)
    return _check(st) if check else st


def rocs_lcb_candidate(batch_, dtype, x_c, ld_xc, d_in_c, w_cc, b_c, d_out_c, act, z, ld_z, res_c, ld_resc, y_c,
                       ld_yc, stream=None, check=True):
    st = lib().rocs_lcb_candidate(_b(batch_), dtype, ptr(x_c), ld_xc, d_in_c, ptr(w_cc), ptr(b_c), d_out_c, act,
                                  ptr(z), ld_z, ptr(res_c), ld_resc, ptr(y_c), ld_yc, stream)
    return _check(st) if check else st


def rocs_lcb_forward(batch_, dtype, x_r, ld_xr, d_in_r, x_c, ld_xc, d_in_c, w_rr, w_cr, w_cc, b_r, b_c, d_out_r,
                     d_out_c, act, res_r, ld_resr, res_c, ld_resc, y_r, ld_yr, y_c, ld_yc, z, ld_z, stream=None,
                     check=True):
    st = lib().rocs_lcb_forward(_b(batch_), dtype, ptr(x_r), ld_xr, d_in_r, ptr(x_c), ld_xc, d_in_c, ptr(w_rr),
                                ptr(w_cr), ptr(w_cc), ptr(b_r), ptr(b_c), d_out_r, d_out_c, act, ptr(res_r), ld_resr,
                                ptr(res_c), ld_resc, ptr(y_r), ld_yr, ptr(y_c), ld_yc, ptr(z), ld_z, stream)
    return _check(st) if check else st


def rocs_lcb_fused_workspace_size(B_r) -> int:
    return int(lib().rocs_lcb_fused_workspace_size(B_r))


def rocs_lcb_forward_fused(batch_, dtype, x_r, ld_xr, d_in_r, x_c, ld_xc, d_in_c, w_rr, w_cr, w_cc, b_r, b_c,
                           d_out_r, d_out_c, act, res_r, ld_resr, res_c, ld_resc, y_r, ld_yr, y_c, ld_yc, z, ld_z,
                           workspace, ws_bytes, stream=None, check=True):
    st = lib().rocs_lcb_forward_fused(_b(batch_), dtype, ptr(x_r), ld_xr, d_in_r, ptr(x_c), ld_xc, d_in_c,
                                      ptr(w_rr), ptr(w_cr), ptr(w_cc), ptr(b_r), ptr(b_c), d_out_r, d_out_c, act,
                                      ptr(res_r), ld_resr, ptr(res_c), ld_resc, ptr(y_r), ld_yr, ptr(y_c), ld_yc,
                                      ptr(z), ld_z, ptr(workspace), ws_bytes, stream)
    return _check(st) if check else st


def rocs_head_forward(batch_, dtype, x_r, ld_xr, d_r, x_c, ld_xc, d_c, w_cr, w_cc, bias, z, logits, stream=None,
                      check=True):
    st = lib().rocs_head_forward(_b(batch_), dtype, ptr(x_r), ld_xr, d_r, ptr(x_c), ld_xc, d_c, ptr(w_cr), ptr(w_cc),
                                 float(bias), ptr(z), ptr(logits), stream)
    return _check(st) if check else st


def rocs_group_norm(dtype, kind, eps, rows_r, width_r, rows_c, width_c, x_r, ld_xr, x_c, ld_xc, res_r, res_c,
                    gamma_r, beta_r, gamma_c, beta_c, act_after, y_r, ld_yr, y_c, ld_yc, stream=None, check=True):
    st = lib().rocs_group_norm(dtype, kind, float(eps), rows_r, width_r, rows_c, width_c, ptr(x_r), ld_xr, ptr(x_c),
                               ld_xc, ptr(res_r), ptr(res_c), ptr(gamma_r), ptr(beta_r), ptr(gamma_c), ptr(beta_c),
                               act_after, ptr(y_r), ld_yr, ptr(y_c), ld_yc, stream)
    return _check(st) if check else st


def rocs_fm_masked(batch_, dtype, n_r, n_c, dim, x_r, ld_xr, x_c, ld_xc, f_r, ld_fr, f_c, ld_fc, stream=None,
                   check=True):
    st = lib().rocs_fm_masked(_b(batch_), dtype, n_r, n_c, dim, ptr(x_r), ld_xr, ptr(x_c), ld_xc, ptr(f_r), ld_fr,
                              ptr(f_c), ld_fc, stream)
    return _check(st) if check else st


def rocs_token_lcb(batch_, dtype, n_r, n_c, dim, t_r, t_c, x_r, ld_xr, x_c, ld_xc, w_rr, w_cr, w_cc, y_r, ld_yr, y_c,
                   ld_yc, z, stream=None, check=True):
    st = lib().rocs_token_lcb(_b(batch_), dtype, n_r, n_c, dim, t_r, t_c, ptr(x_r), ld_xr, ptr(x_c), ld_xc,
                              ptr(w_rr), ptr(w_cr), ptr(w_cc), ptr(y_r), ld_yr, ptr(y_c), ld_yc, ptr(z), stream)
    return _check(st) if check else st


def rocs_dca_encode_kv_workspace_size(B_r, L, d, ffn, n_enc) -> int:
    return int(lib().rocs_dca_encode_kv_workspace_size(B_r, L, d, ffn, n_enc))


def rocs_dca_encode_kv(dtype, B_r, L, d, n_heads, ffn, seq, n_enc, enc, n_depths, depth_src, kvw, kv, workspace,
                       ws_bytes, stream=None, check=True):
    st = lib().rocs_dca_encode_kv(dtype, B_r, L, d, n_heads, ffn, ptr(seq), n_enc, enc, n_depths, depth_src, kvw,
                                  ptr(kv), ptr(workspace), ws_bytes, stream)
    return _check(st) if check else st


def rocs_dca_cross_attn_workspace_size(B_r, B_c, n_heads, L) -> int:
    return int(lib().rocs_dca_cross_attn_workspace_size(B_r, B_c, n_heads, L))


def rocs_dca_cross_attn(batch_, dtype, n_heads, head_dim, L, q_r, ld_qr, q_c, ld_qc, k_r, v_r, k_c, v_c, ld_kv, scale,
                        a_r, ld_ar, a_c, ld_ac, workspace, ws_bytes, stream=None, check=True):
    st = lib().rocs_dca_cross_attn(_b(batch_), dtype, n_heads, head_dim, L, ptr(q_r), ld_qr, ptr(q_c), ld_qc,
                                   ptr(k_r), ptr(v_r), ptr(k_c), ptr(v_c), ld_kv, float(scale), ptr(a_r), ld_ar,
                                   ptr(a_c), ld_ac, ptr(workspace), ws_bytes, stream)
    return _check(st) if check else st


def rocs_dca_request_attn_workspace_size(B_r, n_heads, L) -> int:
    return int(lib().rocs_dca_request_attn_workspace_size(B_r, n_heads, L))


def rocs_dca_request_attn(dtype, B_r, n_heads, L, q_r, ld_qr, seq, ld_s, wk_r, wv_r, scale, a_r, ld_ar, workspace,
                          ws_bytes, stream=None, check=True):
    st = lib().rocs_dca_request_attn(dtype, B_r, n_heads, L, ptr(q_r), ld_qr, ptr(seq), ld_s, ptr(wk_r), ptr(wv_r),
                                     float(scale), ptr(a_r), ld_ar, ptr(workspace), ws_bytes, stream)
    return _check(st) if check else st


def rocs_dca_cross_attn_noalloc(batch_, dtype, n_heads, head_dim, L, q_r, ld_qr, q_c, ld_qc, k_r, v_r, k_c, v_c,
                                ld_kv, scale, a_r, ld_ar, a_c, ld_ac, stream=None, check=True):
    st = lib().rocs_dca_cross_attn_noalloc(_b(batch_), dtype, n_heads, head_dim, L, ptr(q_r), ld_qr, ptr(q_c), ld_qc,
                                           ptr(k_r), ptr(v_r), ptr(k_c), ptr(v_c), ld_kv, float(scale), ptr(a_r),
                                           ld_ar, ptr(a_c), ld_ac, stream)
    return _check(st) if check else st


ROCS_XATTN_NOALLOC_SCRATCH_BYTES = 4 << 20


def rocs_broadcast_rows(batch_, row_bytes, src, src_stride, dst, dst_stride, stream=None, check=True):
    st = lib().rocs_broadcast_rows(_b(batch_), row_bytes, ptr(src), src_stride, ptr(dst), dst_stride, stream)
    return _check(st) if check else st


def rocs_stack_workspace_size(desc: rocs_stack_desc, B_r, B_c) -> int:
    return int(lib().rocs_stack_workspace_size(ctypes.byref(desc), B_r, B_c))


def rocs_stack_forward(desc: rocs_stack_desc, batch_, io: rocs_stack_io, workspace, ws_bytes, stream=None,
                       check=True):
    st = lib().rocs_stack_forward(ctypes.byref(desc), _b(batch_), ctypes.byref(io), ptr(workspace), ws_bytes, stream)
    return _check(st) if check else st


def rocs_ugsep_compensation(dtype, B_r, n_u, n_g, dim, x_u, ld_xu, comp, u_comp, ld_uc, stream=None, check=True):
    st = lib().rocs_ugsep_compensation(dtype, B_r, n_u, n_g, dim, ptr(x_u), ld_xu, ptr(comp), ptr(u_comp), ld_uc,
                                       stream)
    return _check(st) if check else st


def rocs_ugsep_mixup_norm(batch_, dtype, n_u, n_g, dim, eps, x_u, ld_xu, x_g, ld_xg, u_comp, ld_uc, gamma, beta, p_u,
                          ld_pu, p_g, ld_pg, stream=None, check=True):
    st = lib().rocs_ugsep_mixup_norm(_b(batch_), dtype, n_u, n_g, dim, float(eps), ptr(x_u), ld_xu, ptr(x_g), ld_xg,
                                     ptr(u_comp), ld_uc, ptr(gamma), ptr(beta), ptr(p_u), ld_pu, ptr(p_g), ld_pg,
                                     stream)
    return _check(st) if check else st


def ugsep_desc(n_u, n_g, dim, hidden, eps, layers) -> rocs_ugsep_desc:
    """rocs_ugsep_desc over a list of per-layer dicts of device tensors (kept alive by the struct)."""
    arr = (rocs_ugsep_layer * len(layers))()
    for i, L in enumerate(layers):
        arr[i] = rocs_ugsep_layer(*(ptr(L.get(k)) for k in ("comp", "ln1_g", "ln1_b", "w1", "b1", "w2", "b2",
                                                            "ln2_g", "ln2_b", "w1_q", "w1_scale", "w2_q",
                                                            "w2_scale")))
    d = rocs_ugsep_desc(n_u, n_g, dim, hidden, len(layers), float(eps), arr)
    d._keep = (arr, layers)
    return d


def rocs_ugsep_workspace_size(desc: rocs_ugsep_desc, dtype, B_r, B_c, mode) -> int:
    return int(lib().rocs_ugsep_workspace_size(ctypes.byref(desc), dtype, B_r, B_c, mode))


def rocs_ugsep_forward(desc: rocs_ugsep_desc, batch_, dtype, mode, x_u, ld_xu, x_g, ld_xg, y_u, ld_yu, y_g, ld_yg,
                       workspace, ws_bytes, stream=None, check=True):
    st = lib().rocs_ugsep_forward(ctypes.byref(desc), _b(batch_), dtype, mode, ptr(x_u), ld_xu, ptr(x_g), ld_xg,
                                  ptr(y_u), ld_yu, ptr(y_g), ld_yg, ptr(workspace), ws_bytes, stream)
    return _check(st) if check else st


def rocs_w8a16_linear(M, N, K, x, ld_x, w_q, ld_w, w_scale, bias, act, y, ld_y, stream=None, check=True):
    st = lib().rocs_w8a16_linear(M, N, K, ptr(x), ld_x, ptr(w_q), ld_w, ptr(w_scale), ptr(bias), act, ptr(y), ld_y,
                                 stream)
    return _check(st) if check else st


def rocs_validate_batch(batch_, stream=None, check=True):
    st = lib().rocs_validate_batch(_b(batch_), stream)
    return _check(st) if check else st


def rocs_version() -> int:
    return int(lib().rocs_version())
