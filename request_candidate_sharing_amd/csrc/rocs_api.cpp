// librocs host side: argument validation, kernel dispatch, stack executor.
//
// Every entry point validates all host-visible arguments before its first HIP
// call, so invalid arguments return an error code without touching a device.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/rocs.h"
#include "rocs_internal.h"

using namespace rocs;

// Static device scratch of rocs_dca_cross_attn_noalloc (see noalloc_scratch).
static __device__ __align__(256) unsigned char scratch[ROCS_XATTN_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return ROCS_OK;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(ROCS_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

#define ROCS_TRY(expr)                \
  do {                                \
    const int _st = (expr);           \
    if (_st != ROCS_OK) return _st;   \
  } while (0)

#define ROCS_HIP(expr, where)                        \
  do {                                               \
    const hipError_t _e = (expr);                    \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int esize(rocs_dtype dt) { return dt == ROCS_F32 ? 4 : 2; }

int check_dtype(rocs_dtype dt, bool bf16_only, const char* fn) {
  if (dt != ROCS_F32 && dt != ROCS_BF16) return fail(ROCS_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, int(dt));
  if (bf16_only && dt != ROCS_BF16) return fail(ROCS_ERR_DTYPE, "%s: only ROCS_BF16 is supported", fn);
  return ROCS_OK;
}

int check_act(int act, const char* fn) {
  if (act != ROCS_ACT_NONE && act != ROCS_ACT_RELU) return fail(ROCS_ERR_INVALID_ARG, "%s: unknown act %d", fn, act);
  return ROCS_OK;
}

int check_nonneg(int64_t v, const char* fn, const char* name) {
  if (v < 0) return fail(ROCS_ERR_INVALID_ARG, "%s: %s = %lld is negative", fn, name, (long long)v);
  return ROCS_OK;
}

int check_ptr(const void* p, const char* fn, const char* name) {
  if (!p) return fail(ROCS_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return fail(ROCS_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, name);
  return ROCS_OK;
}

int check_opt_ptr(const void* p, const char* fn, const char* name) {
  if (p && reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(ROCS_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, name);
  return ROCS_OK;
}

// A [rows, width] matrix with leading dimension ld (elements of size es).
int check_mat(const void* p, int64_t ld, int64_t width, int es, bool required, const char* fn, const char* name) {
  if (!p) {
    if (required) return fail(ROCS_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);
    return ROCS_OK;
  }
  ROCS_TRY(check_opt_ptr(p, fn, name));
  if (ld < width) return fail(ROCS_ERR_SHAPE, "%s: ld of %s (%lld) < width %lld", fn, name, (long long)ld, (long long)width);
  if ((ld * es) % 16 != 0)
    return fail(ROCS_ERR_ALIGN, "%s: ld of %s (%lld elements) is not a multiple of 16 bytes", fn, name, (long long)ld);
  return ROCS_OK;
}

// Dense weight [rows, in]: rows must start 16-byte aligned.
int check_weight(const void* p, int64_t in, int es, const char* fn, const char* name) {
  ROCS_TRY(check_ptr(p, fn, name));
  if ((in * es) % 16 != 0)
    return fail(ROCS_ERR_ALIGN, "%s: input width %lld of %s is not a multiple of 16 bytes", fn, (long long)in, name);
  return ROCS_OK;
}

int check_batch(const rocs_batch* b, const char* fn) {
  if (!b) return fail(ROCS_ERR_INVALID_ARG, "%s: batch is NULL", fn);
  ROCS_TRY(check_nonneg(b->num_requests, fn, "batch.num_requests"));
  ROCS_TRY(check_nonneg(b->num_candidates, fn, "batch.num_candidates"));
  if (b->num_candidates > 0 && !b->cand2req) return fail(ROCS_ERR_INVALID_ARG, "%s: batch.cand2req is NULL", fn);
  if (b->num_candidates > 0 && b->num_requests == 0)
    return fail(ROCS_ERR_BATCH, "%s: candidates without requests", fn);
  return ROCS_OK;
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ------------------------------------------------------------------ GLM linear

int lcb_request_check(rocs_dtype dt, int32_t B_r, const void* x_r, int64_t ld_xr, int32_t d_in_r, const void* w_rr,
                      const void* w_cr, const void* b_r, int32_t d_out_r, int32_t d_out_c, int act, const void* res_r,
                      int64_t ld_resr, const void* y_r, int64_t ld_yr, const float* z, int64_t ld_z, const char* fn) {
  ROCS_TRY(check_dtype(dt, false, fn));
  ROCS_TRY(check_act(act, fn));
  ROCS_TRY(check_nonneg(B_r, fn, "B_r"));
  ROCS_TRY(check_nonneg(d_in_r, fn, "d_in_r"));
  ROCS_TRY(check_nonneg(d_out_r, fn, "d_out_r"));
  ROCS_TRY(check_nonneg(d_out_c, fn, "d_out_c"));
  if (B_r == 0 || d_out_r + d_out_c == 0) return ROCS_OK;
  const int es = esize(dt);
  ROCS_TRY(check_mat(x_r, ld_xr, d_in_r, es, d_in_r > 0, fn, "x_r"));
  if (d_out_r > 0) {
    ROCS_TRY(check_weight(w_rr, d_in_r, es, fn, "w_rr"));
    ROCS_TRY(check_opt_ptr(b_r, fn, "b_r"));
    ROCS_TRY(check_mat(res_r, ld_resr, d_out_r, es, false, fn, "res_r"));
    ROCS_TRY(check_mat(y_r, ld_yr, d_out_r, es, true, fn, "y_r"));
  }
  if (d_out_c > 0) {
    ROCS_TRY(check_weight(w_cr, d_in_r, es, fn, "w_cr"));
    ROCS_TRY(check_mat(z, ld_z, d_out_c, 4, true, fn, "z"));
  }
  return ROCS_OK;
}

GemmArgs lcb_request_args(int32_t B_r, const void* x_r, int64_t ld_xr, int32_t d_in_r, const void* w_rr,
                          const void* w_cr, const void* b_r, int32_t d_out_r, int32_t d_out_c, int act,
                          const void* res_r, int64_t ld_resr, void* y_r, int64_t ld_yr, float* z, int64_t ld_z,
                          int64_t ldw = 0) {
  GemmArgs g{};
  g.M = B_r;
  g.N = d_out_r + d_out_c;
  g.K = d_in_r;
  g.A = x_r;
  g.lda = ld_xr;
  if (d_out_r > 0 && d_out_c > 0) {
    g.nseg = 2;
    g.W[0] = w_rr;
    g.W[1] = w_cr;
    g.seg_end[0] = d_out_r;
    g.seg_end[1] = g.N;
  } else {
    g.nseg = 1;
    g.W[0] = d_out_r > 0 ? w_rr : w_cr;
    g.seg_end[0] = g.N;
  }
  g.ldw = ldw > 0 ? ldw : d_in_r;  // padded weight rows (stack executor) or contiguous ones
  g.n_split = d_out_r;
  g.out0 = y_r;
  g.ld0 = ld_yr;
  g.out1 = z;
  g.ld1 = ld_z;
  g.bias = b_r;
  g.act = act;
  g.res = res_r;
  g.ldres = ld_resr;
  return g;
}

int lcb_request_launch(rocs_dtype dt, int32_t B_r, const void* x_r, int64_t ld_xr, int32_t d_in_r, const void* w_rr,
                       const void* w_cr, const void* b_r, int32_t d_out_r, int32_t d_out_c, int act,
                       const void* res_r, int64_t ld_resr, void* y_r, int64_t ld_yr, float* z, int64_t ld_z,
                       hipStream_t s, int64_t ldw = 0) {
  if (B_r == 0 || d_out_r + d_out_c == 0) return ROCS_OK;
  const GemmArgs g = lcb_request_args(B_r, x_r, ld_xr, d_in_r, w_rr, w_cr, b_r, d_out_r, d_out_c, act, res_r, ld_resr,
                                      y_r, ld_yr, z, ld_z, ldw);
  ROCS_HIP(launch_gemm(DType(dt), g, s), "rocs_lcb_request");
  return ROCS_OK;
}

int lcb_candidate_check(const rocs_batch* batch, rocs_dtype dt, const void* x_c, int64_t ld_xc, int32_t d_in_c,
                        const void* w_cc, const void* b_c, int32_t d_out_c, int act, const float* z, int64_t ld_z,
                        const void* res_c, int64_t ld_resc, const void* y_c, int64_t ld_yc, const char* fn,
                        bool z_rows_are_candidates = false) {
  ROCS_TRY(check_batch(batch, fn));
  ROCS_TRY(check_dtype(dt, false, fn));
  ROCS_TRY(check_act(act, fn));
  ROCS_TRY(check_nonneg(d_in_c, fn, "d_in_c"));
  ROCS_TRY(check_nonneg(d_out_c, fn, "d_out_c"));
  (void)z_rows_are_candidates;
  if (batch->num_candidates == 0 || d_out_c == 0) return ROCS_OK;
  const int es = esize(dt);
  ROCS_TRY(check_mat(x_c, ld_xc, d_in_c, es, d_in_c > 0, fn, "x_c"));
  if (d_in_c > 0) ROCS_TRY(check_weight(w_cc, d_in_c, es, fn, "w_cc"));
  ROCS_TRY(check_opt_ptr(b_c, fn, "b_c"));
  ROCS_TRY(check_mat(z, ld_z, d_out_c, 4, true, fn, "z"));
  ROCS_TRY(check_mat(res_c, ld_resc, d_out_c, es, false, fn, "res_c"));
  ROCS_TRY(check_mat(y_c, ld_yc, d_out_c, es, true, fn, "y_c"));
  return ROCS_OK;
}

// zmap == nullptr: z holds one row per candidate (dense-broadcast comparator).
GemmArgs lcb_candidate_args(int B_c, int B_r, const int32_t* zmap, const void* x_c, int64_t ld_xc, int32_t d_in_c,
                            const void* w_cc, const void* b_c, int32_t d_out_c, int act, const float* z, int64_t ld_z,
                            const void* res_c, int64_t ld_resc, void* y_c, int64_t ld_yc) {
  GemmArgs g{};
  g.M = B_c;
  g.N = d_out_c;
  g.K = d_in_c;
  g.A = x_c;
  g.lda = ld_xc;
  g.nseg = 1;
  g.W[0] = w_cc;
  g.seg_end[0] = d_out_c;
  g.ldw = d_in_c;
  g.n_split = d_out_c;
  g.out0 = y_c;
  g.ld0 = ld_yc;
  g.z = z;
  g.ldz = ld_z;
  g.zmap = zmap;
  g.zrows = zmap ? B_r : B_c;
  g.bias = b_c;
  g.act = act;
  g.res = res_c;
  g.ldres = ld_resc;
  return g;
}

int lcb_candidate_launch(int B_c, int B_r, const int32_t* zmap, rocs_dtype dt, const void* x_c, int64_t ld_xc,
                         int32_t d_in_c, const void* w_cc, const void* b_c, int32_t d_out_c, int act, const float* z,
                         int64_t ld_z, const void* res_c, int64_t ld_resc, void* y_c, int64_t ld_yc, hipStream_t s,
                         int64_t ldw = 0) {
  if (B_c == 0 || d_out_c == 0) return ROCS_OK;
  GemmArgs g = lcb_candidate_args(B_c, B_r, zmap, x_c, ld_xc, d_in_c, w_cc, b_c, d_out_c, act, z, ld_z, res_c,
                                  ld_resc, y_c, ld_yc);
  if (ldw > 0) g.ldw = ldw;
  ROCS_HIP(launch_gemm(DType(dt), g, s), "rocs_lcb_candidate");
  return ROCS_OK;
}

// ------------------------------------------------------------------ DCA helpers

size_t enc_ws_bytes(int B_r, int L, int d, int ffn, int n_enc) {
  const size_t rows = size_t(B_r) * L;
  size_t b = 0;
  b += align_up(rows * d * 2, 256) * size_t(n_enc);  // S_1..S_n
  b += align_up(rows * 3 * d * 2, 256);              // qkv
  b += align_up(rows * d * 2, 256) * 2;              // attention output, residual sum
  b += align_up(rows * size_t(ffn) * 2, 256);        // FFN hidden
  return b;
}

int encode_kv_check(rocs_dtype dt, int32_t B_r, int32_t L, int32_t d, int32_t n_heads, int32_t ffn, const void* seq,
                    int32_t n_enc, const rocs_enc_layer* enc, int32_t n_depths, const int32_t* depth_src,
                    const rocs_kv_w* kvw, const void* kv, const char* fn) {
  ROCS_TRY(check_dtype(dt, true, fn));
  ROCS_TRY(check_nonneg(B_r, fn, "B_r"));
  ROCS_TRY(check_nonneg(n_enc, fn, "n_enc"));
  ROCS_TRY(check_nonneg(n_depths, fn, "n_depths"));
  if (L <= 0 || d <= 0 || n_heads <= 0 || ffn <= 0) return fail(ROCS_ERR_INVALID_ARG, "%s: L, d, n_heads, ffn must be > 0", fn);
  if (d != n_heads * 64) return fail(ROCS_ERR_UNSUPPORTED, "%s: head_dim must be 64 (d = %d, n_heads = %d)", fn, d, n_heads);
  if (ffn % 8 != 0) return fail(ROCS_ERR_ALIGN, "%s: ffn %% 8 != 0", fn);
  if (B_r == 0) return ROCS_OK;
  ROCS_TRY(check_ptr(seq, fn, "seq"));
  if (n_enc > 0 && !enc) return fail(ROCS_ERR_INVALID_ARG, "%s: enc is NULL", fn);
  for (int k = 0; k < n_enc; ++k) {
    const rocs_enc_layer& e = enc[k];
    ROCS_TRY(check_weight(e.w_qkv, d, 2, fn, "enc.w_qkv"));
    ROCS_TRY(check_weight(e.w_o, d, 2, fn, "enc.w_o"));
    ROCS_TRY(check_weight(e.w_1, d, 2, fn, "enc.w_1"));
    ROCS_TRY(check_weight(e.w_2, ffn, 2, fn, "enc.w_2"));
    for (const void* p : {e.b_qkv, e.b_o, e.b_1, e.b_2, e.ln1_g, e.ln1_b, e.ln2_g, e.ln2_b})
      ROCS_TRY(check_opt_ptr(p, fn, "enc bias/affine"));
  }
  if (n_depths > 0) {
    if (!depth_src || !kvw) return fail(ROCS_ERR_INVALID_ARG, "%s: depth_src / kvw is NULL", fn);
    ROCS_TRY(check_ptr(kv, fn, "kv"));
    for (int j = 0; j < n_depths; ++j) {
      if (depth_src[j] < 0 || depth_src[j] > n_enc)
        return fail(ROCS_ERR_INVALID_ARG, "%s: depth_src[%d] = %d out of [0, %d]", fn, j, depth_src[j], n_enc);
      ROCS_TRY(check_weight(kvw[j].wk_r, d, 2, fn, "kvw.wk_r"));
      ROCS_TRY(check_weight(kvw[j].wv_r, d, 2, fn, "kvw.wv_r"));
      ROCS_TRY(check_weight(kvw[j].wk_c, d, 2, fn, "kvw.wk_c"));
      ROCS_TRY(check_weight(kvw[j].wv_c, d, 2, fn, "kvw.wv_c"));
    }
  }
  return ROCS_OK;
}

int gemm_plain(const void* A, int64_t lda, int M, int N, int K, const void* W, const void* bias, int act,
               const void* res, int64_t ldres, void* out, int64_t ldo, hipStream_t s, const char* where) {
  GemmArgs g{};
  g.M = M;
  g.N = N;
  g.K = K;
  g.A = A;
  g.lda = lda;
  g.nseg = 1;
  g.W[0] = W;
  g.seg_end[0] = N;
  g.ldw = K;
  g.n_split = N;
  g.out0 = out;
  g.ld0 = ldo;
  g.bias = bias;
  g.act = act;
  g.res = res;
  g.ldres = ldres;
  ROCS_HIP(launch_gemm(BF16, g, s), where);
  return ROCS_OK;
}

int layer_norm_rows(int rows, int width, void* x, int64_t ld, const void* g, const void* b, hipStream_t s) {
  NormArgs n{};
  n.rows = rows;
  n.width = width;
  n.x = x;
  n.ldx = ld;
  n.gamma = g;
  n.beta = b;
  n.y = x;
  n.ldy = ld;
  n.kind = 0;
  n.eps = 1e-5f;
  ROCS_HIP(launch_norm(BF16, n, s), "encoder layer norm");
  return ROCS_OK;
}

// Encoder output S_k (k = 0..n_enc) of encode_kv_launch: S_0 is the input
// sequence, S_1.. live at the start of the encoder workspace.
const void* encoder_output(const void* seq, void* workspace, int k, int rows, int d) {
  if (k == 0) return seq;
  return reinterpret_cast<char*>(workspace) + size_t(k - 1) * align_up(size_t(rows) * d * 2, 256);
}

// cand_only: project only the candidate keys and values, kv[j] = [K_C | V_C]
// ([rows, 2d] per depth) for callers that compute the request side from S
// itself (rocs_rqattn.hip); otherwise kv[j] = [K_R | V_R | K_C | V_C].
// Encoder layers [from, to) (to < 0: all), then the K/V projections of the
// depths whose source output S[depth_src] they complete: sources from + 1 ..
// to, and source 0 (the sequence itself) when from == 0.  Stages run in
// order on one stream; the default is the whole encoder.
int encode_kv_launch(int32_t B_r, int32_t L, int32_t d, int32_t n_heads, int32_t ffn, const void* seq, int32_t n_enc,
                     const rocs_enc_layer* enc, int32_t n_depths, const int32_t* depth_src, const rocs_kv_w* kvw,
                     void* kv, void* workspace, hipStream_t s, bool cand_only = false, int from = 0, int to = -1) {
  if (to < 0) to = n_enc;
  if (B_r == 0) return ROCS_OK;
  const int rows = B_r * L;
  char* w = reinterpret_cast<char*>(workspace);
  std::vector<void*> S(n_enc + 1);
  for (int k = 0; k <= n_enc; ++k) S[k] = const_cast<void*>(encoder_output(seq, workspace, k, rows, d));
  w += align_up(size_t(rows) * d * 2, 256) * size_t(n_enc);
  bf16* qkv = reinterpret_cast<bf16*>(w);
  w += align_up(size_t(rows) * 3 * d * 2, 256);
  bf16* att = reinterpret_cast<bf16*>(w);
  w += align_up(size_t(rows) * d * 2, 256);
  bf16* tmp = reinterpret_cast<bf16*>(w);
  w += align_up(size_t(rows) * d * 2, 256);
  bf16* hid = reinterpret_cast<bf16*>(w);

  for (int k = from; k < to; ++k) {
    const rocs_enc_layer& e = enc[k];
    const void* Sin = S[k];
    ROCS_TRY(gemm_plain(Sin, d, rows, 3 * d, d, e.w_qkv, e.b_qkv, 0, nullptr, 0, qkv, 3 * d, s, "encoder qkv"));
    AttnArgs at{};
    at.n_heads = n_heads;
    at.L = L;
    at.q = qkv;
    at.ldq = 3 * d;
    at.k = qkv + d;
    at.v = qkv + 2 * d;
    at.ldkv = 3 * d;
    at.kv_group_stride = int64_t(L) * 3 * d;
    at.o = att;
    at.ldo = d;
    at.scale_log2 = 1.4426950408889634f / 8.0f;  // 1/sqrt(64) * log2(e)
    at.n_groups = B_r;
    at.q_rows_per_group = L;
    ROCS_HIP(launch_attn(at, s), "encoder self-attention");
    ROCS_TRY(gemm_plain(att, d, rows, d, d, e.w_o, e.b_o, 0, Sin, d, tmp, d, s, "encoder out-proj"));
    ROCS_TRY(layer_norm_rows(rows, d, tmp, d, e.ln1_g, e.ln1_b, s));
    ROCS_TRY(gemm_plain(tmp, d, rows, ffn, d, e.w_1, e.b_1, 1, nullptr, 0, hid, ffn, s, "encoder ffn1"));
    ROCS_TRY(gemm_plain(hid, ffn, rows, d, ffn, e.w_2, e.b_2, 0, tmp, d, S[k + 1], d, s, "encoder ffn2"));
    ROCS_TRY(layer_norm_rows(rows, d, S[k + 1], d, e.ln2_g, e.ln2_b, s));
  }
  const int nseg = cand_only ? 2 : 4;
  for (int j = 0; j < n_depths; ++j) {
    if (depth_src[j] > to || (depth_src[j] <= from && !(from == 0 && depth_src[j] == 0))) continue;
    GemmArgs g{};
    g.M = rows;
    g.N = nseg * d;
    g.K = d;
    g.A = S[depth_src[j]];
    g.lda = d;
    g.nseg = nseg;
    const void* ws4[4] = {kvw[j].wk_r, kvw[j].wv_r, kvw[j].wk_c, kvw[j].wv_c};
    for (int q = 0; q < nseg; ++q) {
      g.W[q] = ws4[4 - nseg + q];
      g.seg_end[q] = (q + 1) * d;
    }
    g.ldw = d;
    g.n_split = nseg * d;
    g.out0 = reinterpret_cast<bf16*>(kv) + size_t(j) * rows * nseg * d;
    g.ld0 = nseg * d;
    ROCS_HIP(launch_gemm(BF16, g, s), "K/V projection");
  }
  return ROCS_OK;
}

// the attention plan (tiles per request)
size_t xattn_ws_bytes(int B_r, int B_c) { return align_up(attn_plan_ws_bytes(B_r, B_c), 256); }

struct XattnPlan {
  int32_t* tiles = nullptr;
  int32_t* n_tiles = nullptr;
  int32_t* perm = nullptr;
  int max_tiles = 0;
};

int xattn_check(const rocs_batch* batch, rocs_dtype dt, int32_t n_heads, int32_t head_dim, int32_t L,
                const void* q_r, int64_t ld_qr, const void* q_c, int64_t ld_qc, const void* k_r, const void* v_r,
                const void* k_c, const void* v_c, int64_t ld_kv, const void* a_r, int64_t ld_ar, const void* a_c,
                int64_t ld_ac, const char* fn) {
  ROCS_TRY(check_batch(batch, fn));
  ROCS_TRY(check_dtype(dt, true, fn));
  if (n_heads <= 0 || L <= 0) return fail(ROCS_ERR_INVALID_ARG, "%s: n_heads and L must be > 0", fn);
  if (head_dim != 64) return fail(ROCS_ERR_UNSUPPORTED, "%s: head_dim must be 64", fn);
  if (ld_kv >= kMaxAttnLdkv)
    return fail(ROCS_ERR_UNSUPPORTED, "%s: ld_kv %lld must be below 2^24 elements", fn, (long long)ld_kv);
  const int64_t d = int64_t(n_heads) * 64;
  if (q_r || a_r) {
    ROCS_TRY(check_mat(q_r, ld_qr, d, 2, true, fn, "q_r"));
    ROCS_TRY(check_mat(a_r, ld_ar, d, 2, true, fn, "a_r"));
    ROCS_TRY(check_mat(k_r, ld_kv, d, 2, true, fn, "k_r"));
    ROCS_TRY(check_mat(v_r, ld_kv, d, 2, true, fn, "v_r"));
  }
  if (batch->num_candidates > 0) {
    ROCS_TRY(check_mat(q_c, ld_qc, d, 2, true, fn, "q_c"));
    ROCS_TRY(check_mat(a_c, ld_ac, d, 2, true, fn, "a_c"));
    ROCS_TRY(check_mat(k_c, ld_kv, d, 2, true, fn, "k_c"));
    ROCS_TRY(check_mat(v_c, ld_kv, d, 2, true, fn, "v_c"));
  }
  return ROCS_OK;
}

int xattn_request_launch(int B_r, int H, int L, const void* q_r, int64_t ld_qr, const void* k_r, const void* v_r,
                         int64_t ld_kv, float scale_log2, void* a_r, int64_t ld_ar, hipStream_t s) {
  if (B_r == 0 || !q_r) return ROCS_OK;
  AttnArgs at{};
  at.n_heads = H;
  at.L = L;
  at.q = reinterpret_cast<const bf16*>(q_r);
  at.ldq = ld_qr;
  at.k = reinterpret_cast<const bf16*>(k_r);
  at.v = reinterpret_cast<const bf16*>(v_r);
  at.ldkv = ld_kv;
  at.kv_group_stride = int64_t(L) * ld_kv;
  at.o = reinterpret_cast<bf16*>(a_r);
  at.ldo = ld_ar;
  at.scale_log2 = scale_log2;
  at.n_groups = B_r;
  at.q_rows_per_group = 1;
  ROCS_HIP(launch_attn(at, s), "request cross-attention");
  return ROCS_OK;
}

// with a plan: per-request query tiles (shared execution); without: one group per candidate
int xattn_candidate_launch(int B_r, int B_c, const XattnPlan& plan, int H, int L, const void* q_c, int64_t ld_qc,
                           const void* k_c, const void* v_c, int64_t ld_kv, int64_t kv_group_stride, float scale_log2,
                           void* a_c, int64_t ld_ac, hipStream_t s, bool persistent = false) {
  if (B_c == 0) return ROCS_OK;
  AttnArgs at{};
  at.persistent = persistent ? 1 : 0;
  at.n_heads = H;
  at.L = L;
  at.q = reinterpret_cast<const bf16*>(q_c);
  at.ldq = ld_qc;
  at.k = reinterpret_cast<const bf16*>(k_c);
  at.v = reinterpret_cast<const bf16*>(v_c);
  at.ldkv = ld_kv;
  at.kv_group_stride = kv_group_stride;
  at.o = reinterpret_cast<bf16*>(a_c);
  at.ldo = ld_ac;
  at.scale_log2 = scale_log2;
  at.n_groups = B_r;
  if (plan.tiles) {
    at.q_rows_per_group = 0;
    at.tile_info = plan.tiles;
    at.n_tiles_dev = plan.n_tiles;
    at.perm = plan.perm;
    at.max_tiles = plan.max_tiles;
  } else {  // one group per candidate (dense-broadcast comparator)
    at.n_groups = B_c;
    at.q_rows_per_group = 1;
  }
  ROCS_HIP(launch_attn(at, s), "candidate cross-attention");
  return ROCS_OK;
}

// Scratch of rocs_dca_cross_attn_noalloc: a static device array (one copy per
// GPU, held until the process ends).  Host code never passes the array's
// name to a kernel (in host code that name is not a device address): each
// device's address comes from hipGetSymbolAddress, called once per device
// with that device current, and kernels receive that pointer.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int noalloc_scratch(void** out, const char* fn) {
  int dev = 0;
  ROCS_HIP(hipGetDevice(&dev), fn);
  if (dev < 0 || dev >= kMaxDevices) return fail(ROCS_ERR_UNSUPPORTED, "%s: device index %d", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    ROCS_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), fn);
    if (!p) return fail(ROCS_ERR_HIP, "%s: no device address for the static scratch", fn);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ROCS_OK;
}

float scale_log2_of(float scale) {
  const float sc = scale > 0.f ? scale : 0.125f;
  return sc * 1.4426950408889634f;
}

}  // namespace

// ====================================================================== C ABI

extern "C" {

int rocs_version(void) { return ROCS_VERSION; }

const char* rocs_status_str(int status) {
  switch (status) {
    case ROCS_OK: return "ROCS_OK";
    case ROCS_ERR_INVALID_ARG: return "ROCS_ERR_INVALID_ARG";
    case ROCS_ERR_SHAPE: return "ROCS_ERR_SHAPE";
    case ROCS_ERR_DTYPE: return "ROCS_ERR_DTYPE";
    case ROCS_ERR_ALIGN: return "ROCS_ERR_ALIGN";
    case ROCS_ERR_WORKSPACE: return "ROCS_ERR_WORKSPACE";
    case ROCS_ERR_BATCH: return "ROCS_ERR_BATCH";
    case ROCS_ERR_HIP: return "ROCS_ERR_HIP";
    case ROCS_ERR_UNSUPPORTED: return "ROCS_ERR_UNSUPPORTED";
    default: return "ROCS_ERR_UNKNOWN";
  }
}

const char* rocs_last_error(void) { return g_err.c_str(); }

int rocs_lcb_request(rocs_dtype dtype, int32_t B_r, const void* x_r, int64_t ld_xr, int32_t d_in_r, const void* w_rr,
                     const void* w_cr, const void* b_r, int32_t d_out_r, int32_t d_out_c, rocs_act act,
                     const void* res_r, int64_t ld_resr, void* y_r, int64_t ld_yr, float* z, int64_t ld_z,
                     void* stream) {
  const char* fn = "rocs_lcb_request";
  ROCS_TRY(lcb_request_check(dtype, B_r, x_r, ld_xr, d_in_r, w_rr, w_cr, b_r, d_out_r, d_out_c, act, res_r, ld_resr,
                             y_r, ld_yr, z, ld_z, fn));
  ROCS_TRY(lcb_request_launch(dtype, B_r, x_r, ld_xr, d_in_r, w_rr, w_cr, b_r, d_out_r, d_out_c, act, res_r, ld_resr,
                              y_r, ld_yr, z, ld_z, as_stream(stream)));
  return ok();
}

int rocs_lcb_candidate(const rocs_batch* batch, rocs_dtype dtype, const void* x_c, int64_t ld_xc, int32_t d_in_c,
                       const void* w_cc, const void* b_c, int32_t d_out_c, rocs_act act, const float* z, int64_t ld_z,
                       const void* res_c, int64_t ld_resc, void* y_c, int64_t ld_yc, void* stream) {
  const char* fn = "rocs_lcb_candidate";
  ROCS_TRY(lcb_candidate_check(batch, dtype, x_c, ld_xc, d_in_c, w_cc, b_c, d_out_c, act, z, ld_z, res_c, ld_resc,
                               y_c, ld_yc, fn));
  ROCS_TRY(lcb_candidate_launch(batch->num_candidates, batch->num_requests, batch->cand2req, dtype, x_c, ld_xc,
                                d_in_c, w_cc, b_c, d_out_c, act, z, ld_z, res_c, ld_resc, y_c, ld_yc,
                                as_stream(stream)));
  return ok();
}

int rocs_lcb_forward(const rocs_batch* batch, rocs_dtype dtype, const void* x_r, int64_t ld_xr, int32_t d_in_r,
                     const void* x_c, int64_t ld_xc, int32_t d_in_c, const void* w_rr, const void* w_cr,
                     const void* w_cc, const void* b_r, const void* b_c, int32_t d_out_r, int32_t d_out_c,
                     rocs_act act, const void* res_r, int64_t ld_resr, const void* res_c, int64_t ld_resc, void* y_r,
                     int64_t ld_yr, void* y_c, int64_t ld_yc, float* z, int64_t ld_z, void* stream) {
  const char* fn = "rocs_lcb_forward";
  ROCS_TRY(check_batch(batch, fn));
  ROCS_TRY(lcb_request_check(dtype, batch->num_requests, x_r, ld_xr, d_in_r, w_rr, w_cr, b_r, d_out_r, d_out_c, act,
                             res_r, ld_resr, y_r, ld_yr, z, ld_z, fn));
  ROCS_TRY(lcb_candidate_check(batch, dtype, x_c, ld_xc, d_in_c, w_cc, b_c, d_out_c, act, z, ld_z, res_c, ld_resc,
                               y_c, ld_yc, fn));
  hipStream_t s = as_stream(stream);
  ROCS_TRY(lcb_request_launch(dtype, batch->num_requests, x_r, ld_xr, d_in_r, w_rr, w_cr, b_r, d_out_r, d_out_c, act,
                              res_r, ld_resr, y_r, ld_yr, z, ld_z, s));
  ROCS_TRY(lcb_candidate_launch(batch->num_candidates, batch->num_requests, batch->cand2req, dtype, x_c, ld_xc,
                                d_in_c, w_cc, b_c, d_out_c, act, z, ld_z, res_c, ld_resc, y_c, ld_yc, s));
  return ok();
}

size_t rocs_lcb_fused_workspace_size(int32_t B_r) {
  return B_r > 0 ? align_up(size_t((B_r + 31) / 32 + 1) * 4, 256) : 256;
}

int rocs_lcb_forward_fused(const rocs_batch* batch, rocs_dtype dtype, const void* x_r, int64_t ld_xr,
                           int32_t d_in_r, const void* x_c, int64_t ld_xc, int32_t d_in_c, const void* w_rr,
                           const void* w_cr, const void* w_cc, const void* b_r, const void* b_c, int32_t d_out_r,
                           int32_t d_out_c, rocs_act act, const void* res_r, int64_t ld_resr, const void* res_c,
                           int64_t ld_resc, void* y_r, int64_t ld_yr, void* y_c, int64_t ld_yc, float* z,
                           int64_t ld_z, void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "rocs_lcb_forward_fused";
  ROCS_TRY(check_batch(batch, fn));
  ROCS_TRY(lcb_request_check(dtype, batch->num_requests, x_r, ld_xr, d_in_r, w_rr, w_cr, b_r, d_out_r, d_out_c, act,
                             res_r, ld_resr, y_r, ld_yr, z, ld_z, fn));
  ROCS_TRY(lcb_candidate_check(batch, dtype, x_c, ld_xc, d_in_c, w_cc, b_c, d_out_c, act, z, ld_z, res_c, ld_resc,
                               y_c, ld_yc, fn));
  const int B_r = batch->num_requests, B_c = batch->num_candidates;
  const GemmArgs rq = lcb_request_args(B_r, x_r, ld_xr, d_in_r, w_rr, w_cr, b_r, d_out_r, d_out_c, act, res_r,
                                       ld_resr, y_r, ld_yr, z, ld_z);
  const GemmArgs cq = lcb_candidate_args(B_c, B_r, batch->cand2req, x_c, ld_xc, d_in_c, w_cc, b_c, d_out_c, act, z,
                                         ld_z, res_c, ld_resc, y_c, ld_yc);
  if (!glm_fused_supported(DType(dtype), rq, cq))
    return fail(ROCS_ERR_UNSUPPORTED, "%s: this shape does not fit one launch (use rocs_lcb_forward)", fn);
  const size_t need = rocs_lcb_fused_workspace_size(B_r);
  if (!workspace || ws_bytes < need)
    return fail(ROCS_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu", fn, ws_bytes, need);
  ROCS_TRY(check_ptr(workspace, fn, "workspace"));
  hipStream_t s = as_stream(stream);
  const int n = glm_fused_flag_count(rq) + 1;
  int* fl = static_cast<int*>(workspace);
  ROCS_HIP(launch_pad_rows(1, 0, n, 4, nullptr, 0, fl, n, s), fn);
  ROCS_HIP(launch_glm_fused(DType(dtype), rq, cq, fl, fl + n - 1, s), fn);
  return ok();
}

int rocs_head_forward(const rocs_batch* batch, rocs_dtype dtype, const void* x_r, int64_t ld_xr, int32_t d_r,
                      const void* x_c, int64_t ld_xc, int32_t d_c, const void* w_cr, const void* w_cc, float bias,
                      float* z, float* logits, void* stream) {
  const char* fn = "rocs_head_forward";
  ROCS_TRY(check_batch(batch, fn));
  ROCS_TRY(check_dtype(dtype, false, fn));
  ROCS_TRY(check_nonneg(d_r, fn, "d_r"));
  ROCS_TRY(check_nonneg(d_c, fn, "d_c"));
  const int es = esize(dtype);
  const int B_r = batch->num_requests, B_c = batch->num_candidates;
  if (B_c == 0) return ok();
  if (d_r > 0) {
    ROCS_TRY(check_mat(x_r, ld_xr, d_r, es, true, fn, "x_r"));
    ROCS_TRY(check_weight(w_cr, d_r, es, fn, "w_cr"));
  }
  if (d_c > 0) {
    ROCS_TRY(check_mat(x_c, ld_xc, d_c, es, true, fn, "x_c"));
    ROCS_TRY(check_weight(w_cc, d_c, es, fn, "w_cc"));
  }
  ROCS_TRY(check_ptr(z, fn, "z"));
  ROCS_TRY(check_ptr(logits, fn, "logits"));
  hipStream_t s = as_stream(stream);
  DotArgs r{};
  r.rows = B_r;
  r.width = d_r;
  r.x = x_r;
  r.ldx = ld_xr;
  r.w = w_cr;
  r.out = z;
  ROCS_HIP(launch_rowdot(DType(dtype), r, s), fn);
  DotArgs c{};
  c.rows = B_c;
  c.width = d_c;
  c.x = x_c;
  c.ldx = ld_xc;
  c.w = w_cc;
  c.z = z;
  c.zmap = batch->cand2req;
  c.zrows = B_r;
  c.bias = bias;
  c.out = logits;
  ROCS_HIP(launch_rowdot(DType(dtype), c, s), fn);
  return ok();
}

int rocs_group_norm(rocs_dtype dtype, rocs_norm kind, float eps, int32_t rows_r, int32_t width_r, int32_t rows_c,
                    int32_t width_c, const void* x_r, int64_t ld_xr, const void* x_c, int64_t ld_xc,
                    const void* res_r, const void* res_c, const void* gamma_r, const void* beta_r,
                    const void* gamma_c, const void* beta_c, rocs_act act_after, void* y_r, int64_t ld_yr, void* y_c,
                    int64_t ld_yc, void* stream) {
  const char* fn = "rocs_group_norm";
  ROCS_TRY(check_dtype(dtype, false, fn));
  ROCS_TRY(check_act(act_after, fn));
  if (kind != ROCS_NORM_LAYER && kind != ROCS_NORM_RMS) return fail(ROCS_ERR_INVALID_ARG, "%s: unknown norm kind", fn);
  if (!(eps >= 0.f)) return fail(ROCS_ERR_INVALID_ARG, "%s: eps must be >= 0", fn);
  ROCS_TRY(check_nonneg(rows_r, fn, "rows_r"));
  ROCS_TRY(check_nonneg(rows_c, fn, "rows_c"));
  ROCS_TRY(check_nonneg(width_r, fn, "width_r"));
  ROCS_TRY(check_nonneg(width_c, fn, "width_c"));
  const int es = esize(dtype);
  const int64_t maxw = dtype == ROCS_F32 ? 16 * 64 * 4 : 16 * 64 * 8;
  if (width_r > maxw || width_c > maxw) return fail(ROCS_ERR_UNSUPPORTED, "%s: width above %lld", fn, (long long)maxw);
  const bool do_r = rows_r > 0 && width_r > 0, do_c = rows_c > 0 && width_c > 0;
  if (do_r) {
    ROCS_TRY(check_mat(x_r, ld_xr, width_r, es, true, fn, "x_r"));
    ROCS_TRY(check_mat(res_r, ld_xr, width_r, es, false, fn, "res_r"));
    ROCS_TRY(check_mat(y_r, ld_yr, width_r, es, true, fn, "y_r"));
    ROCS_TRY(check_opt_ptr(gamma_r, fn, "gamma_r"));
    ROCS_TRY(check_opt_ptr(beta_r, fn, "beta_r"));
  }
  if (do_c) {
    ROCS_TRY(check_mat(x_c, ld_xc, width_c, es, true, fn, "x_c"));
    ROCS_TRY(check_mat(res_c, ld_xc, width_c, es, false, fn, "res_c"));
    ROCS_TRY(check_mat(y_c, ld_yc, width_c, es, true, fn, "y_c"));
    ROCS_TRY(check_opt_ptr(gamma_c, fn, "gamma_c"));
    ROCS_TRY(check_opt_ptr(beta_c, fn, "beta_c"));
  }
  hipStream_t s = as_stream(stream);
  if (do_r) {
    NormArgs n{rows_r, width_r, x_r, ld_xr, res_r, gamma_r, beta_r, y_r, ld_yr, int(kind), eps, int(act_after), 0};
    ROCS_HIP(launch_norm(DType(dtype), n, s), fn);
  }
  if (do_c) {
    NormArgs n{rows_c, width_c, x_c, ld_xc, res_c, gamma_c, beta_c, y_c, ld_yc, int(kind), eps, int(act_after), 0};
    ROCS_HIP(launch_norm(DType(dtype), n, s), fn);
  }
  return ok();
}

int rocs_fm_masked(const rocs_batch* batch, rocs_dtype dtype, int32_t n_r, int32_t n_c, int32_t dim, const void* x_r,
                   int64_t ld_xr, const void* x_c, int64_t ld_xc, void* f_r, int64_t ld_fr, void* f_c, int64_t ld_fc,
                   void* stream) {
  const char* fn = "rocs_fm_masked";
  ROCS_TRY(check_batch(batch, fn));
  ROCS_TRY(check_dtype(dtype, true, fn));
  if (n_r <= 0 || n_c < 0 || dim <= 0) return fail(ROCS_ERR_INVALID_ARG, "%s: need n_r > 0, n_c >= 0, dim > 0", fn);
  if (dim % 32 != 0) return fail(ROCS_ERR_UNSUPPORTED, "%s: dim %% 32 != 0", fn);
  if (n_r > 64 || n_c > 64) return fail(ROCS_ERR_UNSUPPORTED, "%s: n_r, n_c <= 64", fn);
  const int B_r = batch->num_requests, B_c = batch->num_candidates;
  if (B_r > 0 || B_c > 0) {
    ROCS_TRY(check_mat(x_r, ld_xr, int64_t(n_r) * dim, 2, true, fn, "x_r"));
    ROCS_TRY(check_mat(f_r, ld_fr, int64_t(n_r) * n_r, 2, true, fn, "f_r"));
  }
  if (B_c > 0 && n_c > 0) {
    ROCS_TRY(check_mat(x_c, ld_xc, int64_t(n_c) * dim, 2, true, fn, "x_c"));
    ROCS_TRY(check_mat(f_c, ld_fc, int64_t(n_c) * (n_r + n_c), 2, true, fn, "f_c"));
  }
  FmArgs a{};
  a.B_r = B_r;
  a.B_c = n_c > 0 ? B_c : 0;
  a.n_r = n_r;
  a.n_c = n_c;
  a.dim = dim;
  a.x_r = reinterpret_cast<const bf16*>(x_r);
  a.ldxr = ld_xr;
  a.x_c = reinterpret_cast<const bf16*>(x_c);
  a.ldxc = ld_xc;
  a.map = batch->cand2req;
  a.map_rows = B_r;
  a.f_r = reinterpret_cast<bf16*>(f_r);
  a.ldfr = ld_fr;
  a.f_c = reinterpret_cast<bf16*>(f_c);
  a.ldfc = ld_fc;
  ROCS_HIP(launch_fm(a, as_stream(stream)), fn);
  return ok();
}

int rocs_token_lcb(const rocs_batch* batch, rocs_dtype dtype, int32_t n_r, int32_t n_c, int32_t dim, int32_t t_r,
                   int32_t t_c, const void* x_r, int64_t ld_xr, const void* x_c, int64_t ld_xc, const void* w_rr,
                   const void* w_cr, const void* w_cc, void* y_r, int64_t ld_yr, void* y_c, int64_t ld_yc, float* z,
                   void* stream) {
  const char* fn = "rocs_token_lcb";
  ROCS_TRY(check_batch(batch, fn));
  ROCS_TRY(check_dtype(dtype, true, fn));
  if (n_r <= 0 || n_c <= 0 || dim <= 0 || t_r < 0 || t_c < 0)
    return fail(ROCS_ERR_INVALID_ARG, "%s: need n_r, n_c, dim > 0 and t_r, t_c >= 0", fn);
  if (dim % 8 != 0) return fail(ROCS_ERR_UNSUPPORTED, "%s: dim %% 8 != 0", fn);
  if (n_r > 64 || n_c > 64 || t_r > 256 || t_c > 256 || int64_t(t_c) * dim > 32768 || int64_t(n_r) * dim > 32768)
    return fail(ROCS_ERR_UNSUPPORTED, "%s: sizes outside n_r, n_c <= 64, t <= 256, t*dim, n_r*dim <= 32768", fn);
  const int B_r = batch->num_requests, B_c = batch->num_candidates;
  if (B_r > 0) {
    ROCS_TRY(check_mat(x_r, ld_xr, int64_t(n_r) * dim, 2, true, fn, "x_r"));
    if (t_r > 0) {
      ROCS_TRY(check_ptr(w_rr, fn, "w_rr"));
      ROCS_TRY(check_mat(y_r, ld_yr, int64_t(t_r) * dim, 2, true, fn, "y_r"));
    }
    if (t_c > 0) {
      ROCS_TRY(check_ptr(w_cr, fn, "w_cr"));
      ROCS_TRY(check_ptr(z, fn, "z"));
    }
  }
  if (B_c > 0 && t_c > 0) {
    ROCS_TRY(check_mat(x_c, ld_xc, int64_t(n_c) * dim, 2, true, fn, "x_c"));
    ROCS_TRY(check_ptr(w_cc, fn, "w_cc"));
    ROCS_TRY(check_mat(y_c, ld_yc, int64_t(t_c) * dim, 2, true, fn, "y_c"));
  }
  TokLcbArgs a{};
  a.B_r = B_r;
  a.B_c = t_c > 0 ? B_c : 0;
  a.n_r = n_r;
  a.n_c = n_c;
  a.dim = dim;
  a.t_r = t_r;
  a.t_c = t_c;
  a.x_r = reinterpret_cast<const bf16*>(x_r);
  a.ldxr = ld_xr;
  a.x_c = reinterpret_cast<const bf16*>(x_c);
  a.ldxc = ld_xc;
  a.w_rr = reinterpret_cast<const bf16*>(w_rr);
  a.w_cr = reinterpret_cast<const bf16*>(w_cr);
  a.w_cc = reinterpret_cast<const bf16*>(w_cc);
  a.y_r = reinterpret_cast<bf16*>(y_r);
  a.ldyr = ld_yr;
  a.y_c = reinterpret_cast<bf16*>(y_c);
  a.ldyc = ld_yc;
  a.z = z;
  a.map = batch->cand2req;
  a.map_rows = B_r;
  hipStream_t s = as_stream(stream);
  ROCS_HIP(launch_token_lcb_request(a, s), fn);
  ROCS_HIP(launch_token_lcb_candidate(a, s), fn);
  return ok();
}

size_t rocs_dca_encode_kv_workspace_size(int32_t B_r, int32_t L, int32_t d, int32_t ffn, int32_t n_enc) {
  if (B_r < 0 || L < 0 || d < 0 || ffn < 0 || n_enc < 0) return 0;
  return enc_ws_bytes(B_r, L, d, ffn, n_enc);
}

int rocs_dca_encode_kv(rocs_dtype dtype, int32_t B_r, int32_t L, int32_t d, int32_t n_heads, int32_t ffn,
                       const void* seq, int32_t n_enc, const rocs_enc_layer* enc, int32_t n_depths,
                       const int32_t* depth_src, const rocs_kv_w* kvw, void* kv, void* workspace, size_t ws_bytes,
                       void* stream) {
  const char* fn = "rocs_dca_encode_kv";
  ROCS_TRY(encode_kv_check(dtype, B_r, L, d, n_heads, ffn, seq, n_enc, enc, n_depths, depth_src, kvw, kv, fn));
  if (B_r == 0) return ok();
  const size_t need = enc_ws_bytes(B_r, L, d, ffn, n_enc);
  if (!workspace || ws_bytes < need)
    return fail(ROCS_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu", fn, ws_bytes, need);
  ROCS_TRY(check_ptr(workspace, fn, "workspace"));
  ROCS_TRY(encode_kv_launch(B_r, L, d, n_heads, ffn, seq, n_enc, enc, n_depths, depth_src, kvw, kv, workspace,
                            as_stream(stream)));
  return ok();
}

size_t rocs_dca_cross_attn_workspace_size(int32_t B_r, int32_t B_c, int32_t n_heads, int32_t L) {
  if (B_r < 0 || B_c < 0 || n_heads <= 0 || L <= 0) return 0;
  return xattn_ws_bytes(B_r, B_c);
}

int rocs_dca_cross_attn(const rocs_batch* batch, rocs_dtype dtype, int32_t n_heads, int32_t head_dim, int32_t L,
                        const void* q_r, int64_t ld_qr, const void* q_c, int64_t ld_qc, const void* k_r,
                        const void* v_r, const void* k_c, const void* v_c, int64_t ld_kv, float scale, void* a_r,
                        int64_t ld_ar, void* a_c, int64_t ld_ac, void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "rocs_dca_cross_attn";
  ROCS_TRY(xattn_check(batch, dtype, n_heads, head_dim, L, q_r, ld_qr, q_c, ld_qc, k_r, v_r, k_c, v_c, ld_kv, a_r,
                       ld_ar, a_c, ld_ac, fn));
  const int B_r = batch->num_requests, B_c = batch->num_candidates;
  const size_t need = xattn_ws_bytes(B_r, B_c);
  const bool work = B_c > 0;
  if (work && (!workspace || ws_bytes < need))
    return fail(ROCS_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu", fn, ws_bytes, need);
  if (work) ROCS_TRY(check_ptr(workspace, fn, "workspace"));
  hipStream_t s = as_stream(stream);
  const float sl2 = scale_log2_of(scale);
  ROCS_TRY(xattn_request_launch(B_r, n_heads, L, q_r, ld_qr, k_r, v_r, ld_kv, sl2, a_r, ld_ar, s));
  if (B_c > 0) {
    XattnPlan p;
    ROCS_HIP(launch_attn_plan(B_r, B_c, batch->offsets, batch->cand2req, workspace, &p.tiles, &p.n_tiles, &p.perm,
                              &p.max_tiles, s),
             fn);
    ROCS_TRY(xattn_candidate_launch(B_r, B_c, p, n_heads, L, q_c, ld_qc, k_c, v_c, ld_kv, int64_t(L) * ld_kv, sl2,
                                    a_c, ld_ac, s));
  }
  return ok();
}

int rocs_broadcast_rows(const rocs_batch* batch, int64_t row_bytes, const void* src, int64_t src_stride, void* dst,
                        int64_t dst_stride, void* stream) {
  const char* fn = "rocs_broadcast_rows";
  ROCS_TRY(check_batch(batch, fn));
  ROCS_TRY(check_nonneg(row_bytes, fn, "row_bytes"));
  if (row_bytes % 16 != 0 || src_stride % 16 != 0 || dst_stride % 16 != 0)
    return fail(ROCS_ERR_ALIGN, "%s: row_bytes and strides must be multiples of 16", fn);
  if (batch->num_candidates == 0 || row_bytes == 0) return ok();
  if (src_stride < row_bytes || dst_stride < row_bytes) return fail(ROCS_ERR_SHAPE, "%s: stride < row_bytes", fn);
  ROCS_TRY(check_ptr(src, fn, "src"));
  ROCS_TRY(check_ptr(dst, fn, "dst"));
  ROCS_HIP(launch_broadcast_rows(batch->num_candidates, batch->cand2req, batch->num_requests, row_bytes, src,
                                 src_stride, dst, dst_stride, as_stream(stream)),
           fn);
  return ok();
}

int rocs_dca_cross_attn_noalloc(const rocs_batch* batch, rocs_dtype dtype, int32_t n_heads, int32_t head_dim,
                                int32_t L, const void* q_r, int64_t ld_qr, const void* q_c, int64_t ld_qc,
                                const void* k_r, const void* v_r, const void* k_c, const void* v_c, int64_t ld_kv,
                                float scale, void* a_r, int64_t ld_ar, void* a_c, int64_t ld_ac, void* stream) {
  const char* fn = "rocs_dca_cross_attn_noalloc";
  ROCS_TRY(xattn_check(batch, dtype, n_heads, head_dim, L, q_r, ld_qr, q_c, ld_qc, k_r, v_r, k_c, v_c, ld_kv, a_r,
                       ld_ar, a_c, ld_ac, fn));
  const int B_r = batch->num_requests, B_c = batch->num_candidates;
  // the attention plan is the only scratch
  const size_t need = B_c > 0 ? xattn_ws_bytes(B_r, B_c) : 0;
  if (need > ROCS_XATTN_NOALLOC_SCRATCH_BYTES)
    return fail(ROCS_ERR_WORKSPACE, "%s: the attention plan of %d requests and %d candidates needs %zu bytes, more "
                "than the %d-byte static scratch", fn, B_r, B_c, need, int(ROCS_XATTN_NOALLOC_SCRATCH_BYTES));
  hipStream_t s = as_stream(stream);
  const float sl2 = scale_log2_of(scale);
  ROCS_TRY(xattn_request_launch(B_r, n_heads, L, q_r, ld_qr, k_r, v_r, ld_kv, sl2, a_r, ld_ar, s));
  if (B_c > 0) {
    void* scratch = nullptr;
    ROCS_TRY(noalloc_scratch(&scratch, fn));
    XattnPlan p;
    ROCS_HIP(launch_attn_plan(B_r, B_c, batch->offsets, batch->cand2req, scratch, &p.tiles, &p.n_tiles, &p.perm,
                              &p.max_tiles, s),
             fn);
    ROCS_TRY(xattn_candidate_launch(B_r, B_c, p, n_heads, L, q_c, ld_qc, k_c, v_c, ld_kv, int64_t(L) * ld_kv, sl2,
                                    a_c, ld_ac, s));
  }
  return ok();
}

size_t rocs_dca_request_attn_workspace_size(int32_t B_r, int32_t n_heads, int32_t L) {
  if (B_r < 0 || !rq_attn_supported(n_heads, L)) return 0;
  return rq_attn_ws_bytes(B_r, L, n_heads);
}

int rocs_dca_request_attn(rocs_dtype dtype, int32_t B_r, int32_t n_heads, int32_t L, const void* q_r, int64_t ld_qr,
                          const void* seq, int64_t ld_s, const void* wk_r, const void* wv_r, float scale, void* a_r,
                          int64_t ld_ar, void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "rocs_dca_request_attn";
  ROCS_TRY(check_dtype(dtype, true, fn));
  ROCS_TRY(check_nonneg(B_r, fn, "B_r"));
  if (L <= 0) return fail(ROCS_ERR_INVALID_ARG, "%s: L must be > 0", fn);
  if (!rq_attn_supported(n_heads, L))
    return fail(ROCS_ERR_UNSUPPORTED, "%s: n_heads must be 1, 2, 4 or 8 and L at most 65536", fn);
  if (B_r == 0) return ok();
  const int64_t d = int64_t(n_heads) * 64;
  ROCS_TRY(check_mat(q_r, ld_qr, d, 2, true, fn, "q_r"));
  ROCS_TRY(check_mat(seq, ld_s, d, 2, true, fn, "seq"));
  ROCS_TRY(check_mat(a_r, ld_ar, d, 2, true, fn, "a_r"));
  ROCS_TRY(check_weight(wk_r, d, 2, fn, "wk_r"));
  ROCS_TRY(check_weight(wv_r, d, 2, fn, "wv_r"));
  const size_t need = rq_attn_ws_bytes(B_r, L, n_heads);
  if (!workspace || ws_bytes < need) return fail(ROCS_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu", fn, ws_bytes, need);
  ROCS_TRY(check_ptr(workspace, fn, "workspace"));
  RqAttnArgs a{};
  a.B_r = B_r;
  a.H = n_heads;
  a.L = L;
  a.q = reinterpret_cast<const bf16*>(q_r);
  a.ldq = ld_qr;
  a.s = reinterpret_cast<const bf16*>(seq);
  a.lds = ld_s;
  a.wk = reinterpret_cast<const bf16*>(wk_r);
  a.wv = reinterpret_cast<const bf16*>(wv_r);
  a.ldw = d;
  a.scale_log2 = scale_log2_of(scale);
  a.o = reinterpret_cast<bf16*>(a_r);
  a.ldo = ld_ar;
  rq_attn_carve(a, workspace);
  ROCS_HIP(launch_rq_attn(a, as_stream(stream)), fn);
  return ok();
}

int rocs_validate_batch(const rocs_batch* batch, void* stream) {
  const char* fn = "rocs_validate_batch";
  ROCS_TRY(check_batch(batch, fn));
  if (batch->num_candidates == 0 && !batch->offsets) return ok();
  int32_t flag = 0;
  ROCS_HIP(launch_validate_batch(batch->num_requests, batch->num_candidates, batch->offsets, batch->cand2req, &flag,
                                 as_stream(stream)),
           fn);
  if (flag & 1) return fail(ROCS_ERR_BATCH, "%s: cand2req out of range or outside its request's offsets range", fn);
  if (flag & 2) return fail(ROCS_ERR_BATCH, "%s: offsets not a prefix sum of 0..B_c", fn);
  return ok();
}

}  // extern "C"

// ====================================================================== stack executor
#include "rocs_stack.inc"

// ====================================================================== UG-Separation TokenMixer
#include "rocs_ugsep.inc"

// ====================================================================== W8A16 linear
#include "rocs_w8a16.inc"
