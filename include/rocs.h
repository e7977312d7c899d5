/*
 * librocs -- C ABI of the ROCS (Request-Oriented Compute Sharing) shared
 * forward pass on AMD Instinct MI355X (gfx950).
 *
 * Citations name the web pages by title:
 *   [R] "ROCS：面向请求的大规模推荐计算共享" (liuzhao09.github.io review):
 *       §2.1 Generalized Layer Masking, §2.2 Deep Cross Attention,
 *       §2.4 In-Kernel Broadcast Optimization, §4 summary.
 *   [D] "Meta推出ROCS：推荐系统推理效率提升3倍，零质量损失" (longzhangge.com
 *       PaperDaily digest), section on kernel-level optimisation (IKBO).
 *
 * The ragged batch ([R] §1 and §2.4): B_r requests, B_c candidates, and a map
 * m (cand2req) with m[i] = the request of candidate i.  Request tensors stay
 * at request-batch size B_r and candidate tensors at candidate-batch size
 * B_c; every candidate-side kernel resolves m[i] itself, so no broadcast
 * tensor is ever materialized ([R] §2.4) -- except in the explicitly
 * requested dense-broadcast comparator mode of rocs_stack_forward.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument named as a tensor is DEVICE memory owned by the
 *    caller.  The library never allocates device memory, never frees a
 *    caller pointer and keeps no pointer after the call returns.  Scratch
 *    memory is caller-provided ("workspace") and sized by the matching
 *    *_workspace_size() call.  Host arrays are marked "host".
 *  - Matrices are row-major.  ld_* arguments are leading dimensions (row
 *    strides) in ELEMENTS of the tensor's dtype.  Weights are [out, in]
 *    (row = one output channel), so both GEMM operands are contiguous along
 *    the reduction axis.
 *  - Alignment (the padding rule of [R] §2.4 and [D]): every tensor base
 *    address must be 16-byte aligned and every ld must be a multiple of 16
 *    bytes (8 bf16 or 4 fp32 elements); otherwise ROCS_ERR_ALIGN.  Widths
 *    themselves may be any size; the stack executor pads its own buffers.
 *  - dtype selects the element type of activations, weights, biases and
 *    outputs: ROCS_F32, or ROCS_BF16 with fp32 accumulation.  Buffers named
 *    z, logits and scale/eps are always fp32.
 *  - All calls are asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL = the default stream) and return after enqueueing.  Host-side
 *    argument validation runs before any HIP call, so invalid arguments
 *    never touch the device.  A HIP launch error returns ROCS_ERR_HIP.
 *  - Status codes are below; rocs_last_error() returns a thread-local
 *    message for the last failing call.  No C++ exception crosses the ABI.
 *  - Empty batches: B_c = 0 is a successful no-op for candidate outputs; a
 *    request with zero candidates is legal.
 *  - cand2req values must lie in [0, B_r).  Kernels never read outside the
 *    request tensors: a candidate whose map entry is out of range gets NaN
 *    outputs.  rocs_validate_batch() checks a batch explicitly.
 *  - Results are deterministic: no atomics on any output path.  A launch's
 *    reduction order depends only on its own shape (rows, width, K), so a
 *    request's outputs are bit-identical whatever candidates accompany it,
 *    and a candidate's whatever order the candidates come in.
 */
#ifndef ROCS_H_
#define ROCS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ROCS_VERSION 10000 /* major*10000 + minor*100 + patch */

enum rocs_status {
  ROCS_OK = 0,
  ROCS_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad enum */
  ROCS_ERR_SHAPE = -2,       /* inconsistent dimensions (ld < width, ...) */
  ROCS_ERR_DTYPE = -3,       /* dtype not supported by this call */
  ROCS_ERR_ALIGN = -4,       /* base not 16-B aligned or ld*elem % 16 != 0 */
  ROCS_ERR_WORKSPACE = -5,   /* workspace missing or too small */
  ROCS_ERR_BATCH = -6,       /* offsets/cand2req inconsistent (rocs_validate_batch) */
  ROCS_ERR_HIP = -7,         /* HIP launch or runtime error */
  ROCS_ERR_UNSUPPORTED = -8  /* valid request outside the implemented envelope */
};

typedef enum rocs_dtype { ROCS_F32 = 0, ROCS_BF16 = 1 } rocs_dtype;
typedef enum rocs_act { ROCS_ACT_NONE = 0, ROCS_ACT_RELU = 1 } rocs_act;
typedef enum rocs_norm { ROCS_NORM_LAYER = 0, ROCS_NORM_RMS = 1 } rocs_norm;

/* Ragged request/candidate batch ([R] §2.4: the index map m).
 * cand2req (device, [num_candidates]) is authoritative.  offsets (device,
 * [num_requests+1] prefix sums) may be given when candidates are stored
 * contiguously per request (request b owns rows offsets[b]..offsets[b+1]-1);
 * it lets attention tile queries per request without a sort.  NULL means
 * arbitrary candidate order. */
typedef struct rocs_batch {
  int32_t num_requests;
  int32_t num_candidates;
  const int32_t* offsets;
  const int32_t* cand2req;
} rocs_batch;

/* ------------------------------------------------------------------ GLM linear (LCB)
 * [R] §2.1 masked-weight linear equation and two-group block matrix:
 *   [Y_R; Y_C] = [[W_RR, 0], [W_CR, W_CC]] [X_R; X_C] + b
 * executed in the decomposed form of [R] §2.4:
 *   request batch   y_r = act(x_r W_RR^T + b_r) + res_r,   z = x_r W_CR^T (fp32)
 *   candidate batch y_c[i] = act(x_c[i] W_CC^T + z[m_i] + b_c) + res_c[i]
 * The candidate GEMM adds z[m_i] in its epilogue (in registers; no
 * broadcast tensor, no intermediate written).  The request half is one GEMM
 * over the stacked weight [W_RR; W_CR].
 *
 * Shapes: x_r [B_r, d_in_r] (ld_xr), x_c [B_c, d_in_c] (ld_xc),
 * w_rr [d_out_r, d_in_r], w_cr [d_out_c, d_in_r], w_cc [d_out_c, d_in_c]
 * (dense, ld = in width), b_r [d_out_r], b_c [d_out_c] (nullable = 0),
 * res_r [B_r, d_out_r] (ld_resr, nullable), res_c [B_c, d_out_c] (ld_resc,
 * nullable), y_r [B_r, d_out_r] (ld_yr), y_c [B_c, d_out_c] (ld_yc),
 * z [B_r, d_out_c] fp32 (ld_z; caller scratch, overwritten).
 * d_out_r may be 0 (then w_rr, b_r, res_r, y_r are ignored).  Weight base
 * addresses must be 16-B aligned and in widths multiples of 16 bytes.
 * Outputs may not alias inputs. */
int rocs_lcb_request(rocs_dtype dtype, int32_t B_r, const void* x_r, int64_t ld_xr, int32_t d_in_r,
                     const void* w_rr, const void* w_cr, const void* b_r, int32_t d_out_r, int32_t d_out_c,
                     rocs_act act, const void* res_r, int64_t ld_resr, void* y_r, int64_t ld_yr, float* z,
                     int64_t ld_z, void* stream);

int rocs_lcb_candidate(const rocs_batch* batch, rocs_dtype dtype, const void* x_c, int64_t ld_xc,
                       int32_t d_in_c, const void* w_cc, const void* b_c, int32_t d_out_c, rocs_act act,
                       const float* z, int64_t ld_z, const void* res_c, int64_t ld_resc, void* y_c,
                       int64_t ld_yc, void* stream);

int rocs_lcb_forward(const rocs_batch* batch, rocs_dtype dtype, const void* x_r, int64_t ld_xr, int32_t d_in_r,
                     const void* x_c, int64_t ld_xc, int32_t d_in_c, const void* w_rr, const void* w_cr,
                     const void* w_cc, const void* b_r, const void* b_c, int32_t d_out_r, int32_t d_out_c,
                     rocs_act act, const void* res_r, int64_t ld_resr, const void* res_c, int64_t ld_resc,
                     void* y_r, int64_t ld_yr, void* y_c, int64_t ld_yc, float* z, int64_t ld_z, void* stream);

/* rocs_lcb_forward as one launch ([R] §2.4: the request and candidate tiles
 * of the LCB in one mega-kernel, the dependency on z a completion flag
 * instead of a kernel boundary; §3.5 Table 4, last step).  Same arguments and
 * outputs, bit-identical to rocs_lcb_forward, plus a workspace of at least
 * rocs_lcb_fused_workspace_size(B_r) bytes (caller-owned, 16-byte aligned,
 * contents arbitrary; the call zeroes the completion counters in it first,
 * one small launch, and the fused launch follows on the same stream; calls
 * that share a workspace must be ordered on one stream).  The request tiles
 * take the lowest workgroup ids; a candidate tile polls the counters of the
 * 32-row request blocks its map entries name before it reads z.  A poll
 * gives up after a bounded number of tries (it cannot be reached while
 * workgroups dispatch in id order); the tile's accumulators are then NaN
 * (NaN outputs, zeros after ReLU) and the int after the counters, at int
 * index (B_r + 31) / 32 of the workspace, is set to 1 (the call clears it).
 * Tests force that path from the host: with the environment variable
 * ROCS_TEST_FUSED_GIVE_UP=n (n > 0) the call waits for a count no request
 * tile reaches and gives up after n polls per candidate tile.
 * Returns ROCS_ERR_UNSUPPORTED, having enqueued nothing, unless dtype is
 * bf16, 0 < B_r < 2048, B_c >= 2048, d_out_c > 128 and a multiple of 256,
 * at most one of ReLU and res_c is used, and every row offset of y_c, res_c
 * and z fits in 31 bits; ROCS_ERR_WORKSPACE for a short or NULL workspace. */
/* Workspace bytes of rocs_lcb_forward_fused: (B_r + 31) / 32 completion
 * counters and the error word, as ints, rounded up to 256 bytes. */
size_t rocs_lcb_fused_workspace_size(int32_t B_r);
int rocs_lcb_forward_fused(const rocs_batch* batch, rocs_dtype dtype, const void* x_r, int64_t ld_xr,
                           int32_t d_in_r, const void* x_c, int64_t ld_xc, int32_t d_in_c, const void* w_rr,
                           const void* w_cr, const void* w_cc, const void* b_r, const void* b_c, int32_t d_out_r,
                           int32_t d_out_c, rocs_act act, const void* res_r, int64_t ld_resr, const void* res_c,
                           int64_t ld_resc, void* y_r, int64_t ld_yr, void* y_c, int64_t ld_yc, float* z,
                           int64_t ld_z, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ scalar head
 * The GLM linear of [R] §2.1 with d_out_r = 0 and d_out_c = 1 (a candidate
 * score): z[b] = w_cr . x_r[b];  logits[i] = w_cc . x_c[i] + z[m_i] + bias.
 * x_r [B_r, d_r] (ld_xr), x_c [B_c, d_c] (ld_xc), w_cr [d_r], w_cc [d_c],
 * z [B_r] fp32 scratch, logits [B_c] fp32. */
int rocs_head_forward(const rocs_batch* batch, rocs_dtype dtype, const void* x_r, int64_t ld_xr, int32_t d_r,
                      const void* x_c, int64_t ld_xc, int32_t d_c, const void* w_cr, const void* w_cc,
                      float bias, float* z, float* logits, void* stream);

/* ------------------------------------------------------------------ group-local norm
 * [R] §2.1, Figure 2(b): statistics per group, never across groups.
 *   y = act(norm(x + res) * gamma + beta)
 * LAYER: (v - mean) / sqrt(biased var + eps); RMS: v / sqrt(mean(v^2) + eps).
 * Statistics in fp32 over each row of one group's slice.  Request rows
 * x_r [rows_r, width_r], candidate rows x_c [rows_c, width_c]; res_* share
 * the ld of x_* and are nullable; gamma/beta [width] nullable (1 / 0).
 * In place (y == x) is allowed. */
int rocs_group_norm(rocs_dtype dtype, rocs_norm kind, float eps, int32_t rows_r, int32_t width_r, int32_t rows_c,
                    int32_t width_c, const void* x_r, int64_t ld_xr, const void* x_c, int64_t ld_xc,
                    const void* res_r, const void* res_c, const void* gamma_r, const void* beta_r,
                    const void* gamma_c, const void* beta_c, rocs_act act_after, void* y_r, int64_t ld_yr,
                    void* y_c, int64_t ld_yc, void* stream);

/* ------------------------------------------------------------------ masked FM
 * [R] §2.1 masked-FM equation, Figure 2(c): with request tokens
 * X_R[b] [n_r, dim] and candidate tokens X_C[i] [n_c, dim],
 *   f_r[b] = vec(X_R[b] X_R[b]^T)                   (n_r*n_r values)
 *   f_c[i] = vec(X_C[i] [X_R[m_i]; X_C[i]]^T)         (n_c*(n_r+n_c) values)
 * flattened token-major (row a, then columns; candidate columns list the
 * request tokens first).  The structurally zero request x candidate block
 * is not stored.  x_r [B_r, n_r*dim], x_c [B_c, n_c*dim] contiguous rows;
 * f_r (ld_fr), f_c (ld_fc).  bf16 only; dim % 32 == 0, n_r <= 64,
 * n_c <= 64. */
int rocs_fm_masked(const rocs_batch* batch, rocs_dtype dtype, int32_t n_r, int32_t n_c, int32_t dim,
                   const void* x_r, int64_t ld_xr, const void* x_c, int64_t ld_xc, void* f_r, int64_t ld_fr,
                   void* f_c, int64_t ld_fc, void* stream);

/* ------------------------------------------------------------------ token-axis LCB
 * The GLM linear of [R] §2.1 applied along the token axis (the LCB
 * compression of Figure 1(d)):  T_R[b] = W_RR X_R[b];
 * T_C[i] = W_CC X_C[i] + Z[m_i] with Z[b] = W_CR X_R[b] computed once per
 * request ([R] §2.4).  w_rr [t_r, n_r], w_cr [t_c, n_r], w_cc [t_c, n_c]
 * (dense, same dtype), x_* as in rocs_fm_masked, outputs flattened
 * token-major: y_r [B_r, t_r*dim] (ld_yr), y_c [B_c, t_c*dim] (ld_yc),
 * z [B_r, t_c*dim] fp32 scratch.  bf16 only; dim % 64 == 0, n_r, n_c <= 64,
 * t_r, t_c <= 256. */
int rocs_token_lcb(const rocs_batch* batch, rocs_dtype dtype, int32_t n_r, int32_t n_c, int32_t dim, int32_t t_r,
                   int32_t t_c, const void* x_r, int64_t ld_xr, const void* x_c, int64_t ld_xc, const void* w_rr,
                   const void* w_cr, const void* w_cc, void* y_r, int64_t ld_yr, void* y_c, int64_t ld_yc,
                   float* z, void* stream);

/* ------------------------------------------------------------------ DCA
 * [R] §2.2: a request-only sequence encoder S_k = Enc_k(S_{k-1}) and per
 * interaction depth the shared projections K = S W_K, V = S W_V for the
 * request and candidate query groups, computed once per request.
 * Encoder layer (post-LN, ReLU FFN, no mask):
 *   S' = LN(S + MHA(S)),  S'' = LN(S' + W_2 ReLU(W_1 S' + b_1) + b_2),
 * MHA with a fused in-projection [3d, d] (q, k, v row blocks) + bias and an
 * output projection [d, d] + bias; heads are contiguous head_dim slices. */
typedef struct rocs_enc_layer {
  const void* w_qkv; const void* b_qkv; /* [3d, d], [3d] (bias nullable) */
  const void* w_o;   const void* b_o;   /* [d, d],  [d] */
  const void* ln1_g; const void* ln1_b; /* [d] nullable (1 / 0) */
  const void* w_1;   const void* b_1;   /* [ffn, d], [ffn] */
  const void* w_2;   const void* b_2;   /* [d, ffn], [d] */
  const void* ln2_g; const void* ln2_b; /* [d] nullable */
} rocs_enc_layer;

typedef struct rocs_kv_w {
  const void* wk_r; const void* wv_r; const void* wk_c; const void* wv_c; /* each [d, d], no bias */
} rocs_kv_w;

/* Encodes the sequences and writes every depth's keys/values.
 * seq [B_r, L, d] contiguous.  kv (output) is [n_depths][B_r*L][4*d]: row
 * (b*L + l) of depth j holds [K_R | V_R | K_C | V_C] of token l of request b.
 * depth_src (host, [n_depths]) picks the encoder output each depth reads
 * (0 = raw sequence, k = after layer k).  enc (host, [n_enc]), kvw (host,
 * [n_depths]).  bf16 only; head_dim == 64; d = n_heads*64; ffn % 8 == 0.
 * workspace >= rocs_dca_encode_kv_workspace_size(B_r, L, d, ffn, n_enc). */
size_t rocs_dca_encode_kv_workspace_size(int32_t B_r, int32_t L, int32_t d, int32_t ffn, int32_t n_enc);
int rocs_dca_encode_kv(rocs_dtype dtype, int32_t B_r, int32_t L, int32_t d, int32_t n_heads, int32_t ffn,
                       const void* seq, int32_t n_enc, const rocs_enc_layer* enc, int32_t n_depths,
                       const int32_t* depth_src, const rocs_kv_w* kvw, void* kv, void* workspace, size_t ws_bytes,
                       void* stream);

/* Grouped cross-attention ([R] §2.2, IKBO-DCA of [R] §2.4): per head h,
 *   a_r[b]_h = softmax(q_r[b]_h K_R[b]_h^T * scale) V_R[b]_h
 *   a_c[i]_h = softmax(q_c[i]_h K_C[m_i]_h^T * scale) V_C[m_i]_h
 * with no mask.  Keys/values stay at request-batch size: k_* / v_* point at
 * [B_r][L] rows of row stride ld_kv elements (request b's token l is row
 * b*L + l); head h uses columns [h*64, h*64+64).  All queries of one
 * request share each staged key/value tile.  q_r [B_r, H*64] (ld_qr),
 * q_c [B_c, H*64] (ld_qc); outputs a_r (ld_ar), a_c (ld_ac).  q_r/a_r
 * nullable (skip the request group).  bf16 only, head_dim == 64,
 * ld_kv < 2^24 (ROCS_ERR_UNSUPPORTED otherwise), scale <= 0 selects
 * 1/sqrt(head_dim).  workspace >=
 * rocs_dca_cross_attn_workspace_size(B_r, B_c, n_heads, L): the per-request
 * query tiles and a device counting sort of cand2req when batch->offsets
 * is NULL (the size depends on B_r and B_c only; n_heads and L are
 * accepted for callers that size workspaces per layer).  Needed whenever
 * there are candidates. */
size_t rocs_dca_cross_attn_workspace_size(int32_t B_r, int32_t B_c, int32_t n_heads, int32_t L);
int rocs_dca_cross_attn(const rocs_batch* batch, rocs_dtype dtype, int32_t n_heads, int32_t head_dim, int32_t L,
                        const void* q_r, int64_t ld_qr, const void* q_c, int64_t ld_qc, const void* k_r,
                        const void* v_r, const void* k_c, const void* v_c, int64_t ld_kv, float scale, void* a_r,
                        int64_t ld_ar, void* a_c, int64_t ld_ac, void* workspace, size_t ws_bytes, void* stream);

/* Request-side cross-attention computed from the encoder output ([R] §2.2,
 * grouped cross-attention of the request query group, one query row per
 * request and head): a_r[b] = concat_h softmax(q_h K_h^T * scale) V_h with
 * K = S W_K^T and V = S W_V^T over request b's L events S[b*L .. b*L+L-1].
 * With a single query per request and head, the keys and values need not
 * be projected: the call re-associates the products, scores
 * (W_K,h^T q_h) . S_l and output W_V,h (sum_l p_h(l) S_l), exactly equal in
 * real arithmetic (fp32 accumulation, one bf16 rounding of the output).
 *   seq    [B_r * L, ld_s] bf16 (rows of request b at b*L)
 *   wk_r, wv_r  [d, d] bf16, [out, in] (row stride d), d = 64 * n_heads
 *   q_r    [B_r, ld_qr], a_r [B_r, ld_ar] bf16
 *   scale  score scale (0 selects 1/sqrt(64))
 * n_heads in {1, 2, 4, 8} and L <= 65536 (else ROCS_ERR_UNSUPPORTED); bf16 only.
 * Workspace: rocs_dca_request_attn_workspace_size (fp32 q' and per-chunk
 * partial sums).  The stack executor uses this path for the request query
 * group and projects only the candidates' keys and values. */
size_t rocs_dca_request_attn_workspace_size(int32_t B_r, int32_t n_heads, int32_t L);
int rocs_dca_request_attn(rocs_dtype dtype, int32_t B_r, int32_t n_heads, int32_t L, const void* q_r, int64_t ld_qr,
                          const void* seq, int64_t ld_s, const void* wk_r, const void* wv_r, float scale, void* a_r,
                          int64_t ld_ar, void* workspace, size_t ws_bytes, void* stream);

/* Variant of rocs_dca_cross_attn that allocates nothing and takes no
 * workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, results and errors as rocs_dca_cross_attn, except that
 * its only scratch, the attention plan (per-request counts and offsets,
 * the candidate permutation, the query tiles), lives in a static device
 * array of ROCS_XATTN_NOALLOC_SCRATCH_BYTES per GPU, held until the process
 * ends; a batch whose plan needs more (about 4 bytes per candidate plus 24
 * bytes per request) returns ROCS_ERR_WORKSPACE before anything is
 * enqueued.  Every call on one GPU shares that GPU's array, which keeps the last
 * call's contents (each call clears what must start at zero).  Calls that
 * overlap on one GPU (other streams, other host threads) race. */
#define ROCS_XATTN_NOALLOC_SCRATCH_BYTES (4 << 20)
int rocs_dca_cross_attn_noalloc(const rocs_batch* batch, rocs_dtype dtype, int32_t n_heads, int32_t head_dim,
                                int32_t L, const void* q_r, int64_t ld_qr, const void* q_c, int64_t ld_qc,
                                const void* k_r, const void* v_r, const void* k_c, const void* v_c, int64_t ld_kv,
                                float scale, void* a_r, int64_t ld_ar, void* a_c, int64_t ld_ac, void* stream);

/* ------------------------------------------------------------------ explicit broadcast (comparator)
 * dst row i = src row m_i, copied byte for byte (the materialized broadcast
 * of [R] §2.4, Figure 3(a); used only by the dense-broadcast comparator).
 * row_bytes % 16 == 0; strides in bytes, multiples of 16. */
int rocs_broadcast_rows(const rocs_batch* batch, int64_t row_bytes, const void* src, int64_t src_stride,
                        void* dst, int64_t dst_stride, void* stream);

/* ------------------------------------------------------------------ stack executor
 * Runs a ROCSified layer stack ([R] §2.1 composition closure) on one
 * stream.  Activations live in "slots": slot 0 is the caller's input
 * (io->x_r / io->x_c), slot 1 the caller's output (io->y_r / io->y_c), and
 * slots >= 2 are carved from the workspace with 16-byte-padded rows.  Each
 * slot has a request part [B_r, width_r] and a candidate part
 * [B_c, width_c].  Layers read and write column ranges of slots, so a
 * concatenation is two layers writing adjacent columns of one slot.
 * A layer's output view may not overlap the views it reads (tiles would
 * overwrite rows other tiles still read), with two element-wise
 * exceptions: a NORM may run in place (src view == dst view), and a
 * residual view may equal the output view.  Other overlaps are rejected
 * with ROCS_ERR_INVALID_ARG before anything is enqueued.
 * Widths whose rows are not whole 16-byte chunks (e.g. 37 bf16 elements)
 * are zero-padded in the workspace ([R] §2.4, the alignment fix of the
 * decomposed dimensions): caller slots of such widths are staged through
 * padded copies (any row stride >= width, element-aligned pointers), GLM
 * weight blocks with such input widths are copied into padded rows once per
 * call, and the columns after such an input view are zeroed, so every GEMM
 * reads whole 16-byte chunks.  Column offsets of views stay multiples of 16
 * bytes, and no view may cover the zero padding after a ragged GLM input
 * (ROCS_ERR_ALIGN).  The standalone rocs_lcb_* calls read caller rows in
 * 16-byte chunks and keep requiring them. */
typedef enum rocs_exec_mode {
  ROCS_EXEC_SHARED = 0,          /* request work at B_r size, map resolved in-kernel */
  ROCS_EXEC_DENSE_BROADCAST = 1, /* comparator: request contributions and K/V copied to B_c rows first */
  ROCS_EXEC_SHARED_SERIAL = 2,   /* as ROCS_EXEC_SHARED, every launch on the caller's stream */
  ROCS_EXEC_SHARED_FUSED = 3     /* as ROCS_EXEC_SHARED_SERIAL, each GLM linear's two halves in one launch */
} rocs_exec_mode;
/* ROCS_EXEC_SHARED_FUSED ([R] §2.4: request and candidate tiles in one
 * mega-kernel, the dependency on the request contribution a completion flag
 * instead of a kernel boundary; §3.5 Table 4, last step): every launch on the
 * caller's stream, and a GLM linear whose request and candidate GEMMs fit
 * one launch runs them as one grid.  Such a linear needs bf16, B_r < 2048,
 * B_c >= 2048, d_out_c > 128 and a multiple of 256, d_out_c + d_out_r split
 * as in rocs_lcb_forward, and at most one of ReLU and a residual (the
 * candidate epilogue with Z in the accumulators); other layers make the
 * launches of ROCS_EXEC_SHARED_SERIAL.  The request tiles take the lowest
 * workgroup ids (dispatched first, they wait for nothing); a candidate tile
 * polls one completion counter per 32 request rows it reads, in the
 * workspace, zeroed once at the start of the call.  A poll gives up after a
 * bounded number of tries; the tile's accumulators are then NaN.  The
 * candidate cross-attention (the persistent attention kernel of §2.4) runs
 * on one round of workgroups, three per compute unit, each walking the
 * (query tile, head) pairs of its XCD's range; test variable
 * ROCS_TEST_ATTN_ROUND=n sets that round to n workgroups (a multiple of 8).
 * Outputs are bit-identical to ROCS_EXEC_SHARED_SERIAL. */
/* Schedule of ROCS_EXEC_SHARED with both row groups present and a DCA
 * descriptor of more than one depth ([R] §2.4: the request and candidate
 * tiles share the GPU, the dependency on the request contribution is a
 * completion signal instead of a kernel boundary; other stacks, with no
 * request-only work to overlap across layers, run as
 * ROCS_EXEC_SHARED_SERIAL): the request rows' work runs on an internal
 * stream of the device (created once
 * per device at default priority, kept until the process ends) and the
 * candidate rows' work on the caller's stream.  A candidate launch that reads
 * a request result (Z, the request dots of the head, the keys and values of
 * the encoder) first waits for an event recorded after its producer; the
 * internal stream starts after an event recorded on the caller's stream at
 * the call, and the caller's stream waits for the internal one at the end, so
 * to the caller the call is ordered on its stream as one unit (also under
 * stream capture).  The encoder and the K/V projections are enqueued in
 * stages, each before the first cross-attention that needs its output.  Every launch is the one ROCS_EXEC_SHARED_SERIAL makes, so
 * the two modes give identical bits.  Calls that overlap on one device share
 * the internal stream (their request work runs in call order). */

typedef enum rocs_op_kind {
  ROCS_OP_LINEAR = 1,    /* rocs_lcb_forward                                      */
  ROCS_OP_NORM = 2,      /* rocs_group_norm                                        */
  ROCS_OP_FM = 3,        /* rocs_fm_masked, src holds tokens [n_r*dim | n_c*dim]   */
  ROCS_OP_TOKEN_LCB = 4, /* rocs_token_lcb (w_rr, w_cr, w_cc are the token maps)   */
  ROCS_OP_XATTN = 5,     /* rocs_dca_cross_attn at K/V depth `depth`; src = queries */
  ROCS_OP_HEAD = 6       /* rocs_head_forward into io->logits; b_c[0] = bias        */
} rocs_op_kind;

typedef struct rocs_layer {
  int32_t kind;                    /* rocs_op_kind */
  int32_t src, src_col_r, src_col_c; /* input slot and per-group column offsets */
  int32_t dst, dst_col_r, dst_col_c; /* output slot and per-group column offsets */
  int32_t res, res_col_r, res_col_c; /* residual slot (-1 = none) */
  int32_t d_in_r, d_in_c, d_out_r, d_out_c; /* per-group widths */
  int32_t act;                     /* rocs_act: LINEAR before the residual, NORM after */
  int32_t norm;                    /* rocs_norm (NORM) */
  float eps;                       /* NORM */
  int32_t depth;                   /* XATTN: K/V depth index */
  int32_t n_r, n_c, dim;           /* FM / TOKEN_LCB token counts and token dim */
  const void* w_rr; const void* w_cr; const void* w_cc;
  const void* b_r; const void* b_c;
  const void* gamma_r; const void* beta_r; const void* gamma_c; const void* beta_c;
} rocs_layer;

typedef struct rocs_slot { int32_t width_r, width_c; } rocs_slot;

typedef struct rocs_dca_desc {
  int32_t L, d, n_heads, ffn;
  int32_t n_enc; const rocs_enc_layer* enc;   /* host [n_enc] */
  int32_t n_depths; const int32_t* depth_src; /* host [n_depths] */
  const rocs_kv_w* kvw;                       /* host [n_depths] */
} rocs_dca_desc;

/* Executor fusion (opt-in).  With ROCS_STACK_FUSE_MLP set, a bf16 stack runs
 * the pattern
 *   LINEAR(src=x, dst=h) ; LINEAR(src=h, dst=t [, res=x]) [; NORM(src=t)]
 * as one fused candidate-side kernel when h (and t, if a NORM follows) is a
 * workspace slot that no later layer reads, the candidate widths satisfy
 * d_in % 128 == 0, hidden % 64 == 0, d_out % 32 == 0, d_out <= 512, and the
 * operands are 16-byte aligned: the hidden activation then never reaches
 * HBM.  Otherwise, and for request rows always, the layers run unfused.
 * Without a fused NORM the result is bit-identical to the unfused layers;
 * with one it differs by the rounding of the pre-norm sum (the unfused path
 * stores it in the stack dtype first). */
#define ROCS_STACK_FUSE_MLP 1u

typedef struct rocs_stack_desc {
  rocs_dtype dtype;
  rocs_exec_mode mode;
  int32_t n_slots; const rocs_slot* slots;   /* host [n_slots], n_slots >= 2 */
  int32_t n_layers; const rocs_layer* layers; /* host [n_layers] */
  const rocs_dca_desc* dca;                  /* NULL when no layer is XATTN */
  uint32_t flags;                            /* ROCS_STACK_* bits */
} rocs_stack_desc;

typedef struct rocs_stack_io {
  const void* x_r; int64_t ld_xr; const void* x_c; int64_t ld_xc; /* slot 0 */
  void* y_r; int64_t ld_yr; void* y_c; int64_t ld_yc;             /* slot 1 (nullable if unused) */
  const void* seq;                                                /* DCA sequences [B_r, L, d] */
  float* logits;                                                  /* HEAD output [B_c] */
} rocs_stack_io;

size_t rocs_stack_workspace_size(const rocs_stack_desc* desc, int32_t B_r, int32_t B_c);
int rocs_stack_forward(const rocs_stack_desc* desc, const rocs_batch* batch, const rocs_stack_io* io,
                       void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ UG-Separation TokenMixer
 * [U] "Compute Only Once: UG-Separation for Efficient Large Recommendation
 * Models" (xllm-io review), §3: the framework tree (U tokens, G tokens, the
 * mask that keeps G from affecting U, U side computed once), the core
 * formulas (TokenMixer layer P = LN(Mixup(X)), X' = LN(PFFN(P) + X), the
 * token concatenation, the separation mask, the compensation G + Proj(U)).
 *
 * A sample holds T = n_u + n_g tokens of width dim, stored side by side in
 * one row: U tokens x_u [B_r, n_u * dim] (one row per request), G tokens
 * x_g [B_c, n_g * dim] (one row per candidate); token t starts at column
 * t * dim.  Candidate i's sample is [U tokens of request m_i ; its G tokens].
 * A layer computes, per sample:
 *   G'  = G + P U            (P [n_g, n_u] fp32 token-axis map; optional)
 *   Pm  = LN1(Mixup_UG([U ; G']))
 *   out = LN2(PFFN(Pm) + [U ; G'])
 * Mixup_UG: each token is cut into T chunks of width c = dim / T; output
 * token h is the concatenation over input tokens t of chunk h of token t,
 * except that in U outputs (h < n_u) the chunks of G tokens are zero (G may
 * not affect U).  LN: LayerNorm over one token's dim features (biased
 * variance), gamma/beta shared by the tokens of a layer.  PFFN: per-token
 * weights, F_t = W2_t ReLU(W1_t Pm_t + b1_t) + b2_t.  The residual adds
 * token h to output token h, so the U side never reads a G token: U outputs
 * are computed once per request (B_r rows), G outputs once per candidate,
 * reading the request's U rows and P U through cand2req.
 *
 * Constraints: dim a multiple of T with the chunk c a multiple of 16 bytes
 * (8 bf16 / 4 fp32 elements), dim <= 2048 (bf16) / 1024 (fp32), hidden a
 * multiple of 16 bytes; otherwise ROCS_ERR_SHAPE / ROCS_ERR_UNSUPPORTED /
 * ROCS_ERR_ALIGN.  A candidate whose map entry is out of range gets NaN. */

typedef struct rocs_ugsep_layer {
  const float* comp;       /* [n_g, n_u] fp32 compensation map P; NULL = none */
  const void* ln1_gamma;   /* [dim] */
  const void* ln1_beta;    /* [dim] */
  const void* w1;          /* [T, hidden, dim]: token t's first FFN weight */
  const void* b1;          /* [T, hidden] (nullable = 0) */
  const void* w2;          /* [T, dim, hidden] */
  const void* b2;          /* [T, dim] (nullable = 0) */
  const void* ln2_gamma;   /* [dim] */
  const void* ln2_beta;    /* [dim] */
  /* ROCS_UGSEP_SHARED_W8A16 only (else ignored): the U tokens' FFN weights as
   * 8-bit E4M3 codes with one fp32 scale per output channel, in the encoding
   * rocs_w8a16_linear reads; w1 and w2 are then read for the G tokens only.
   * Token t < n_u computes with w1_scale[t, h] * e4m3(w1_q[t, h, :]) and
   * w2_scale[t, d] * e4m3(w2_q[t, d, :]). */
  const uint8_t* w1_q;     /* [n_u, hidden, dim] codes */
  const float* w1_scale;   /* [n_u, hidden] */
  const uint8_t* w2_q;     /* [n_u, dim, hidden] codes */
  const float* w2_scale;   /* [n_u, dim] */
} rocs_ugsep_layer;

typedef struct rocs_ugsep_desc {
  int32_t n_u, n_g, dim, hidden, n_layers;
  float eps;                       /* LayerNorm epsilon, inside the root */
  const rocs_ugsep_layer* layers;  /* host [n_layers] */
} rocs_ugsep_desc;

typedef enum rocs_ugsep_mode {
  ROCS_UGSEP_SHARED = 0, /* U side once per request */
  ROCS_UGSEP_DENSE = 1,  /* comparator: U tokens copied to every candidate and
                            recomputed per candidate; y_u is not written */
  ROCS_UGSEP_SHARED_W8A16 = 2 /* shared, with the U side's FFN on 8-bit weights
                            ([U] §3 stage 4 and the W8A16 configuration: the
                            per-request U side is a small-batch, weight-bound
                            layer).  bf16 only; needs the layers' w1_q/w2_q
                            codes and scales, num_requests <= 64, dim and hidden
                            multiples of 128; ROCS_ERR_UNSUPPORTED otherwise.  The G side is as
                            in ROCS_UGSEP_SHARED. */
} rocs_ugsep_mode;

/* u_comp [B_r, n_g * dim] fp32 (ld_uc) = P x_u along the token axis (the
 * compensation Proj(U), once per request).  No-op when B_r, n_u or n_g is 0. */
int rocs_ugsep_compensation(rocs_dtype dtype, int32_t B_r, int32_t n_u, int32_t n_g, int32_t dim, const void* x_u,
                            int64_t ld_xu, const float* comp, float* u_comp, int64_t ld_uc, void* stream);

/* One layer's LN1(Mixup_UG(.)): p_u [B_r, n_u * dim] (U outputs of each
 * request, ld_pu) and p_g [B_c, n_g * dim] (G outputs of each candidate,
 * ld_pg), reading G tokens as x_g + u_comp[m_i] when u_comp is non-NULL.
 * gamma, beta: [dim]. */
int rocs_ugsep_mixup_norm(const rocs_batch* batch, rocs_dtype dtype, int32_t n_u, int32_t n_g, int32_t dim, float eps,
                          const void* x_u, int64_t ld_xu, const void* x_g, int64_t ld_xg, const float* u_comp,
                          int64_t ld_uc, const void* gamma, const void* beta, void* p_u, int64_t ld_pu, void* p_g,
                          int64_t ld_pg, void* stream);

/* n_layers TokenMixer layers: y_u [B_r, n_u * dim] (ld_yu), y_g [B_c, n_g *
 * dim] (ld_yg).  Outputs may not alias inputs.  The workspace holds the
 * per-token FFN activations and the inter-layer tokens. */
size_t rocs_ugsep_workspace_size(const rocs_ugsep_desc* desc, rocs_dtype dtype, int32_t B_r, int32_t B_c,
                                 int32_t mode);
int rocs_ugsep_forward(const rocs_ugsep_desc* desc, const rocs_batch* batch, rocs_dtype dtype, int32_t mode,
                       const void* x_u, int64_t ld_xu, const void* x_g, int64_t ld_xg, void* y_u, int64_t ld_yu,
                       void* y_g, int64_t ld_yg, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ W8A16 linear
 * [U] "Compute Only Once: UG-Separation for Efficient Large Recommendation
 * Models" (xllm-io review), §3 framework tree stage 4 and the W8A16
 * configuration table: weights stored in 8 bits, activations in bf16, for
 * the memory-bound small-batch layers.
 *   y[m, n] = act( sum_k x[m, k] * w_scale[n] * e4m3(w_q[n, k]) + bias[n] )
 * w_q: [N, K] bytes (ld_w bytes per row), each the 8-bit E4M3 encoding with
 * no infinities (sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * exponent 0 is subnormal; S.1111.111 is NaN; largest magnitude 448).
 * w_scale: [N] fp32, one scale per output channel.  x: [M, K] bf16 (ld_x),
 * bias: [N] bf16 (nullable), y: [M, N] bf16 (ld_y).  Products accumulate in
 * fp32; the scale, bias and ReLU are applied once at the end.
 * Supported: 1 <= M <= 64, N a multiple of 16, K a positive multiple of 128
 * (ROCS_ERR_UNSUPPORTED otherwise); x, w_q, y 16-byte aligned with 16-byte
 * row strides (ROCS_ERR_ALIGN).  M == 0 or N == 0 is a no-op. */
int rocs_w8a16_linear(int32_t M, int32_t N, int32_t K, const void* x, int64_t ld_x, const uint8_t* w_q, int64_t ld_w,
                      const float* w_scale, const void* bias, rocs_act act, void* y, int64_t ld_y, void* stream);

/* ------------------------------------------------------------------ utilities */
/* Checks offsets/cand2req on the device (synchronizes `stream`): cand2req in
 * range, and when offsets is given, offsets[0] == 0, offsets[B_r] == B_c,
 * nondecreasing, and cand2req[i] == b for every i in request b's range.
 * Returns ROCS_OK or ROCS_ERR_BATCH. */
int rocs_validate_batch(const rocs_batch* batch, void* stream);
const char* rocs_status_str(int status);
const char* rocs_last_error(void);
int rocs_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ROCS_H_ */
