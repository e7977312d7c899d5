// Internal kernel interfaces of librocs (gfx950 only).  Host validation lives
// in rocs_api.cpp; everything here assumes arguments were already checked.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rocs {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum DType { F32 = 0, BF16 = 1 };

// C[M,N] = A[M,K] . W[N,K]^T followed by the GLM epilogue.
// Columns [0, n_split) go to out0 through the full epilogue
//   v = acc + z[zrow(m)][n] + bias[n];  v = act(v);  v += res[m][n]
// with zrow(m) = zmap ? zmap[m] : m (the in-kernel broadcast of the
// request contribution); columns [n_split, N) go raw to out1 (fp32).
// The weight operand may be split into up to four row segments (e.g. the
// stacked [W_RR; W_CR] of the request half, or [Wk_R; Wv_R; Wk_C; Wv_C]),
// segment s covering rows [seg_end[s-1], seg_end[s]).
struct GemmArgs {
  int M, N, K;
  const void* A;
  int64_t lda;
  int nseg;
  const void* W[4];
  int seg_end[4];
  int64_t ldw;
  int n_split;
  void* out0;
  int64_t ld0;
  int out0_f32;  // 1: out0 is fp32 even for bf16 compute
  float* out1;
  int64_t ld1;
  const float* z;
  int64_t ldz;
  const int32_t* zmap;
  int zrows;
  const void* bias;
  int act;
  const void* res;
  int64_t ldres;
  int epi;  // epilogue variant, set by launch_gemm (callers leave it 0)
  // Optional batch of `batch` independent GEMMs of this shape: GEMM i reads
  // A, W[*], bias, res and writes out0 at i times these byte strides, and
  // reads Z at i * sz floats (out1 and zmap are shared).  0 or 1 = one GEMM.
  int batch;
  int64_t sA, sW, s0, sbias, sres, sz;
};

// GEMM i of a batched launch (pointers advanced by i strides).
__host__ __device__ inline GemmArgs batch_slice(const GemmArgs& a, int i) {
  GemmArgs b = a;
  if (i > 0) {
    b.A = static_cast<const char*>(a.A) + i * a.sA;
    for (int k = 0; k < 4; ++k)
      if (a.W[k]) b.W[k] = static_cast<const char*>(a.W[k]) + i * a.sW;
    b.out0 = static_cast<char*>(a.out0) + i * a.s0;
    if (a.bias) b.bias = static_cast<const char*>(a.bias) + i * a.sbias;
    if (a.res) b.res = static_cast<const char*>(a.res) + i * a.sres;
    if (a.z) b.z = a.z + i * a.sz;
  }
  return b;
}

hipError_t launch_gemm(DType dt, const GemmArgs& a, hipStream_t s);
// Compute units of the current device (cached per device; 256 if unknown).
int device_cus();
// Launch choices of launch_gemm, by shape: the epilogue variant, whether a
// launch of fewer than 2,048 rows splits K, and the candidate tile plan.
int epilogue_variant(const GemmArgs& a);
bool uses_splitk(const GemmArgs& a);
struct CandPlan {
  int h;             // uniform tile height, or 0 for the mixed plan
  int M1, h2, grid;  // mixed plan: rows [0, M1) in 256-row tiles, then h2-row tiles
};
CandPlan cand_plan(int M, int ntn);
// One launch for both halves of a GLM linear: the request tiles ([Y_R | Z])
// and the candidate tiles, which wait for the request rows they read on
// completion counters instead of a kernel boundary.  `flags` holds
// glm_fused_flag_count(req) zeroed ints (left nonzero: zero them again
// before the next launch), `err` one int set to 1 if a wait gave up.  Returns
// hipErrorNotSupported, having launched nothing, when the pair does not fit
// (glm_fused_supported).
bool glm_fused_supported(DType dt, const GemmArgs& req, const GemmArgs& cand);
int glm_fused_flag_count(const GemmArgs& req);
hipError_t launch_glm_fused(DType dt, const GemmArgs& req, const GemmArgs& cand, int* flags, int* err,
                            hipStream_t s);
// Whether launch_gemm sums this launch as Z + products (accumulators started
// at the gathered Z rows) rather than products + Z.
bool gemm_z_in_accumulators(const GemmArgs& a);

// y = act(norm(x + res) * gamma + beta) on rows of width w (one launch per group).
struct NormArgs {
  int rows, width;
  const void* x;
  int64_t ldx;
  const void* res;
  const void* gamma;
  const void* beta;
  void* y;
  int64_t ldy;
  int kind;  // 0 layer, 1 rms
  float eps;
  int act;
  int64_t ldres;  // 0: same as ldx
  // Optional score head on the rounded output rows, with launch_rowdot's
  // arithmetic and order (same bits): head_out[i] = head_w . y[i]
  // (+ head_z[head_zmap[i]], NaN for a map entry out of range) + head_bias
  // (+ head_bias_dev[0]).  head_w null: no head.
  const void* head_w;
  const float* head_z;
  const int32_t* head_zmap;
  int head_zrows;
  float head_bias;
  const void* head_bias_dev;
  float* head_out;
};
hipError_t launch_norm(DType dt, const NormArgs& a, hipStream_t s);
// Two independent row groups in one launch (either may be empty).
hipError_t launch_norm2(DType dt, const NormArgs& a, const NormArgs& b, hipStream_t s);

// dot rows: out[i] = w . x[i] (+ z[zmap[i]]) (+ bias)
struct DotArgs {
  int rows, width;
  const void* x;
  int64_t ldx;
  const void* w;
  const float* z;
  const int32_t* zmap;
  int zrows;
  float bias;
  const void* bias_dev;  // optional device scalar (dtype of x), added after bias
  float* out;
};
hipError_t launch_rowdot(DType dt, const DotArgs& a, hipStream_t s);

// dst row r = src row (map[r / inner] * inner + r % inner), rows = map entries * inner.
hipError_t launch_broadcast_rows(int rows, const int32_t* map, int map_rows, int64_t row_bytes, const void* src,
                                 int64_t src_stride, void* dst, int64_t dst_stride, hipStream_t s, int inner = 1);

// Grouped attention, bf16, head_dim 64.  Query rows are grouped; group g
// attends keys/values rows [g*L, g*L + L) (row stride ldkv) of its K/V.
// Query tiles come from a tile table (see launch_attn_plan) or, for uniform
// groups (q_rows_per_group > 0), are implicit.
struct AttnArgs {
  int n_heads;
  int L;
  const bf16* q;
  int64_t ldq;
  const bf16* k;
  const bf16* v;
  int64_t ldkv;
  int64_t kv_group_stride;  // elements between groups (normally L*ldkv)
  bf16* o;
  int64_t ldo;
  float scale_log2;  // scale * log2(e), > 0 (the lazy softmax rescaling relies on it)
  // grouping
  int n_groups;
  int q_rows_per_group;      // > 0: uniform groups, row r belongs to group r / q_rows_per_group
  const int32_t* tile_info;  // per tile: group, row_begin, row_end (3 ints), from the plan
  const int32_t* n_tiles_dev;
  const int32_t* perm;  // optional row permutation: logical row r is physical row perm[r]
  int max_tiles;
  int persistent;  // 1: one round of workgroups walks the (tile, head) pairs (same bits)
};
// hipErrorInvalidValue when ldkv >= 2^24 (64 key rows are addressed by
// 32-bit byte offsets) or L <= 0
hipError_t launch_attn(const AttnArgs& a, hipStream_t s);
constexpr int64_t kMaxAttnLdkv = int64_t(1) << 24;
int attn_tile_rows();

// Builds per-request query tiles (and, without offsets, a counting sort of
// cand2req into a permutation).  ws layout is returned through the pointers.
// Request-side cross-attention from the encoder output (rocs_rqattn.hip):
// o[b, h*64 + e] = W_V,h (softmax_l(q'_h . S_l) S) with q'_h = W_K,h^T q_h,
// one query per request; d = 64 H, H in {1, 2, 4, 8}; S rows 16-byte aligned.
struct RqAttnArgs {
  int B_r, H, L;
  const bf16* q;
  int64_t ldq;
  const bf16* s;  // [B_r * L, lds], rows of request b at b*L
  int64_t lds;
  const bf16* wk;  // [d, d] ([out, in]), row stride ldw
  const bf16* wv;
  int64_t ldw;
  float scale_log2;  // score scale times log2(e)
  bf16* o;
  int64_t ldo;
  float* qf;       // workspace (rq_attn_carve)
  float* part_u;
  float* part_ml;
};
size_t rq_attn_ws_bytes(int B_r, int L, int H);
void rq_attn_carve(RqAttnArgs& a, void* ws);
bool rq_attn_supported(int H, int L);
hipError_t launch_rq_attn(const RqAttnArgs& a, hipStream_t s);

size_t attn_plan_ws_bytes(int B_r, int B_c);
hipError_t launch_attn_plan(int B_r, int B_c, const int32_t* offsets, const int32_t* cand2req, void* ws,
                            int32_t** tile_info, int32_t** n_tiles, int32_t** perm, int* max_tiles, hipStream_t s);

struct FmArgs {
  int B_r, B_c, n_r, n_c, dim;
  const bf16* x_r;
  int64_t ldxr;
  const bf16* x_c;
  int64_t ldxc;
  const int32_t* map;  // cand2req (NULL: candidate i reads request row i)
  int map_rows;
  bf16* f_r;
  int64_t ldfr;
  bf16* f_c;
  int64_t ldfc;
};
hipError_t launch_fm(const FmArgs& a, hipStream_t s);

struct TokLcbArgs {
  int B_r, B_c, n_r, n_c, dim, t_r, t_c;
  const bf16* x_r;
  int64_t ldxr;
  const bf16* x_c;
  int64_t ldxc;
  const bf16* w_rr;
  const bf16* w_cr;
  const bf16* w_cc;
  bf16* y_r;
  int64_t ldyr;
  bf16* y_c;
  int64_t ldyc;
  float* z;
  const int32_t* map;
  int map_rows;
};
hipError_t launch_token_lcb_request(const TokLcbArgs& a, hipStream_t s);
hipError_t launch_token_lcb_candidate(const TokLcbArgs& a, hipStream_t s);

// Fused candidate-side GLM MLP block (see rocs_mlp.hip):
//   y = norm(act2(act1(x W1^T + Z1[zrow] + b1) W2^T + Z2[zrow] + b2) + x?)
struct MlpArgs {
  int M, d_in, hidden, d_out;
  const bf16* x;
  int64_t ldx;
  const bf16* w1;  // [hidden, d_in]
  const bf16* b1;  // [hidden] or null
  const float* z1;
  int64_t ldz1;
  int act1;
  const bf16* w2;  // [d_out, hidden]
  const bf16* b2;  // [d_out] or null
  const float* z2;
  int64_t ldz2;
  int act2;
  const int32_t* zmap;  // null: Z rows are candidate rows
  int zrows;
  // 1: accumulate onto Z (Z + products), the order the unfused candidate GEMM
  // uses for the same layer (gemm_z_in_accumulators); 0: add Z at the end
  int z1_first, z2_first;
  int residual;  // add x (d_in == d_out)
  int norm;      // -1 none, 0 LayerNorm, 1 RMSNorm (statistics over d_out)
  float eps;
  const bf16* gamma;
  const bf16* beta;
  bf16* y;
  int64_t ldy;
};
bool mlp_block_supported(int d_in, int hidden, int d_out);
hipError_t launch_mlp_block(const MlpArgs& a, hipStream_t s);

// dst[r][c] = src[r][c] (c < w), 0 (w <= c < wpad); src NULL: zero [w, wpad) only
hipError_t launch_pad_rows(int64_t rows, int w, int wpad, int es, const void* src, int64_t lds, void* dst,
                           int64_t ldd, hipStream_t s);
hipError_t launch_validate_batch(int B_r, int B_c, const int32_t* offsets, const int32_t* cand2req, int32_t* flag,
                                 hipStream_t s);

// UG-Separation TokenMixer ([U] §3).  Sample rows hold their tokens side by
// side: x_u [rows_u, n_u * dim], x_g [rows_g, n_g * dim] (token t at column
// t * dim).  Compensation uc [rows_u, n_g * dim] fp32 = P x_u (token axis).
struct CompArgs {
  int rows, n_u, n_g, dim;
  const void* xu;
  int64_t ldxu;
  const float* P;  // [n_g, n_u] fp32
  float* uc;
  int64_t lduc;
};
hipError_t launch_ug_comp(DType dt, const CompArgs& a, hipStream_t s);

// LayerNorm(Mixup_UG(x)) for the U outputs of rows_u requests (pu) and the
// G outputs of rows_g candidates (pg, reading U of map[i] and G + uc[map[i]]).
// Needs dim % (n_u + n_g) == 0, the chunk dim / (n_u + n_g) a multiple of 16
// bytes, dim <= mixup_max_dim(dt), gamma and beta non-null.
struct MixupArgs {
  int rows_u, rows_g, n_u, n_g, dim;
  const void* xu;
  int64_t ldxu;
  const void* xg;
  int64_t ldxg;
  const float* uc;  // nullable
  int64_t lduc;
  const int32_t* map;
  const void* gamma;
  const void* beta;
  float eps;
  void* pu;
  int64_t ldpu;
  void* pg;
  int64_t ldpg;
};
int mixup_max_dim(DType dt);

// W8A16 linear: y = act(x (scale . fp8(wq))^T + bias); x [M, K] bf16 (ldx),
// wq [N, K] E4M3 codes (ldw bytes), scale [N] fp32, bias [N] bf16 or null,
// y [M, N] bf16 (ldy).  Needs 1 <= M <= 64, N % 32 == 0, K % 128 == 0.
struct W8Args {
  int M, N, K;
  const bf16* x;
  int64_t ldx;
  const uint8_t* wq;
  int64_t ldw;
  const float* scale;
  const bf16* bias;
  int act;
  bf16* y;
  int64_t ldy;
  const bf16* res;  // optional residual added after the activation (ld = ldres)
  int64_t ldres;
  // optional batch of `batch` GEMMs of this shape (grid.y): GEMM i reads x, wq,
  // scale, bias, res and writes y at i times these element strides
  int batch;
  int64_t sx, sw, sscale, sbias, sres, sy;
};
bool w8a16_supported(int M, int N, int K);
hipError_t launch_w8a16(const W8Args& a, hipStream_t s);
hipError_t launch_mixup_norm(DType dt, const MixupArgs& a, hipStream_t s);

}  // namespace rocs
