// Masked FM interaction and token-axis LCB ([R] §2.1 masked-FM equation,
// Figure 2(c); masked-weight linear along the token axis, Figure 2(a)).
#include "rocs_device.h"

namespace rocs {

namespace {

// ----------------------------------------------------------------- masked FM
// One wave per output item.  Candidate item i: rows a of X_C[i] (n_c) against
// rows b of [X_R[m_i]; X_C[i]] (n_r + n_c); request item b: rows of X_R[b]
// against themselves.  MFMA 16x16x32 with the "b" rows as the A operand so a
// lane holds 4 consecutive output columns of one output row.  The request x
// candidate block is never computed (it is structurally zero and not
// stored).  Request tokens are read from the request tensor through m_i
// (no broadcast copy).
__device__ __forceinline__ uint4 frag(const bf16* rowp, bool ok, int k) {
  return ok ? *reinterpret_cast<const uint4*>(rowp + k) : make_uint4(0, 0, 0, 0);
}

__global__ __launch_bounds__(256) void fm_kernel(FmArgs a, int request_mode) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n_items = request_mode ? a.B_r : a.B_c;
  if (item >= n_items) return;
  const int D = a.dim;
  const bf16 *P, *Q1, *Q2;
  int nP, nQ1, nQ2;
  bf16* out;
  int ncols;
  bool bad = false;
  if (request_mode) {
    P = a.x_r + int64_t(item) * a.ldxr;
    nP = a.n_r;
    Q1 = P;
    nQ1 = a.n_r;
    Q2 = nullptr;
    nQ2 = 0;
    out = a.f_r + int64_t(item) * a.ldfr;
    ncols = a.n_r;
  } else {
    int m = a.map ? a.map[item] : item;
    if ((unsigned)m >= (unsigned)a.map_rows) {
      bad = true;
      m = 0;
    }
    P = a.x_c + int64_t(item) * a.ldxc;
    nP = a.n_c;
    Q1 = a.x_r + int64_t(m) * a.ldxr;
    nQ1 = a.n_r;
    Q2 = P;
    nQ2 = a.n_c;
    out = a.f_c + int64_t(item) * a.ldfc;
    ncols = a.n_r + a.n_c;
  }
  const int nQ = nQ1 + nQ2;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  for (int pa = 0; pa < nP; pa += 16) {
    const int arow = pa + r16;
    const bool aok = arow < nP;
    const bf16* ap = P + int64_t(aok ? arow : 0) * D;
    for (int qb = 0; qb < nQ; qb += 16) {
      const int brow = qb + r16;
      const bool bok = brow < nQ;
      const bf16* bp = (brow < nQ1) ? Q1 + int64_t(brow) * D : Q2 + int64_t(bok ? brow - nQ1 : 0) * D;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int k = 0; k < D; k += 32) {
        const uint4 ua = frag(ap, aok, k + kq);
        const uint4 ub = frag(bp, bok, k + kq);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ub), __builtin_bit_cast(bf16x8, ua),
                                                      acc, 0, 0, 0);
      }
      const int orow = pa + r16;
      const int ocol = qb + 4 * (lane >> 4);
      if (orow < nP) {
        bf16* o = out + int64_t(orow) * ncols + ocol;
        const float nanv = nan_f();
        if (ocol + 4 <= nQ && (ncols & 3) == 0) {
          bf16x4 pk = {to_bf(bad ? nanv : acc[0]), to_bf(bad ? nanv : acc[1]), to_bf(bad ? nanv : acc[2]),
                       to_bf(bad ? nanv : acc[3])};
          *reinterpret_cast<bf16x4*>(o) = pk;
        } else {
          for (int j = 0; j < 4; ++j)
            if (ocol + j < nQ) o[j] = to_bf(bad ? nanv : acc[j]);
        }
      }
    }
  }
}

// Same products with the shape fixed at compile time: NPB x NQB output
// blocks of 16 x 16, KD k-steps of 32 (D = 32 KD).  Every fragment of the
// item is requested before the first MFMA, so one memory latency covers the
// item instead of one per k-step.
template <int NPB, int NQB, int KD>
__global__ __launch_bounds__(256) void fm_fast_kernel(FmArgs a, int request_mode) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n_items = request_mode ? a.B_r : a.B_c;
  if (item >= n_items) return;
  constexpr int D = 32 * KD;
  const bf16 *P, *Q1, *Q2;
  int nP, nQ1, nQ2;
  bf16* out;
  int ncols;
  bool bad = false;
  if (request_mode) {
    P = a.x_r + int64_t(item) * a.ldxr;
    nP = a.n_r;
    Q1 = P;
    nQ1 = a.n_r;
    Q2 = P;
    nQ2 = 0;
    out = a.f_r + int64_t(item) * a.ldfr;
    ncols = a.n_r;
  } else {
    int m = a.map ? a.map[item] : item;
    if ((unsigned)m >= (unsigned)a.map_rows) {
      bad = true;
      m = 0;
    }
    P = a.x_c + int64_t(item) * a.ldxc;
    nP = a.n_c;
    Q1 = a.x_r + int64_t(m) * a.ldxr;
    nQ1 = a.n_r;
    Q2 = P;
    nQ2 = a.n_c;
    out = a.f_c + int64_t(item) * a.ldfc;
    ncols = a.n_r + a.n_c;
  }
  const int nQ = nQ1 + nQ2;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  bf16x8 pf[NPB][KD], qf[NQB][KD];
#pragma unroll
  for (int pb = 0; pb < NPB; ++pb) {
    const int row = pb * 16 + r16;
    const bool ok = row < nP;
    const bf16* rp = P + int64_t(ok ? row : 0) * D + kq;
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) pf[pb][kd] = __builtin_bit_cast(bf16x8, frag(rp, ok, kd * 32));
  }
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int row = qb * 16 + r16;
    const bool ok = row < nQ;
    const bf16* rp = (row < nQ1 ? Q1 + int64_t(row) * D : Q2 + int64_t(ok ? row - nQ1 : 0) * D) + kq;
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) qf[qb][kd] = __builtin_bit_cast(bf16x8, frag(rp, ok, kd * 32));
  }
  const float nanv = nan_f();
#pragma unroll
  for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kd = 0; kd < KD; ++kd) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[qb][kd], pf[pb][kd], acc, 0, 0, 0);
      const int orow = pb * 16 + r16;
      const int ocol = qb * 16 + 4 * (lane >> 4);
      if (orow < nP) {
        bf16* o = out + int64_t(orow) * ncols + ocol;
        if (ocol + 4 <= nQ && (ncols & 3) == 0) {
          bf16x4 pk = {to_bf(bad ? nanv : acc[0]), to_bf(bad ? nanv : acc[1]), to_bf(bad ? nanv : acc[2]),
                       to_bf(bad ? nanv : acc[3])};
          *reinterpret_cast<bf16x4*>(o) = pk;
        } else {
          for (int j = 0; j < 4; ++j)
            if (ocol + j < nQ) o[j] = to_bf(bad ? nanv : acc[j]);
        }
      }
    }
}

// Candidate items with n_C <= 16 and n_R a multiple of 16 (NQR blocks of
// request rows), D = 32 KD.  A wave walks IPW consecutive candidates and
// keeps the fragments of its request's tokens X_R[m] in registers while m
// is unchanged; the candidate's own fragments serve both as the row
// operand and as the last column block (the candidate x candidate part),
// and the next candidate's are requested before the current one's MFMAs.
// The MFMA sequence of every output block is fm_fast_kernel's, so the
// results are bit-identical to it.
template <int NQR, int KD>
__global__ __launch_bounds__(256) void fm_cand_kernel(FmArgs a, int ipw) {
  constexpr int D = 32 * KD;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i0 = (blockIdx.x * 4 + wave) * ipw;
  const int i1 = min(i0 + ipw, a.B_c);
  if (i0 >= i1) return;
  const int nc = a.n_c, nr = a.n_r, ncols = nr + nc;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const bool prow = r16 < nc;
  auto load_p = [&](int i, bf16x8 (&pf)[KD]) {
    const bf16* rp = a.x_c + int64_t(i) * a.ldxc + int64_t(prow ? r16 : 0) * D + kq;
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) pf[kd] = __builtin_bit_cast(bf16x8, frag(rp, prow, kd * 32));
  };
  bf16x8 rq[NQR][KD];
  bf16x8 pf[KD], pn[KD];
  int mc = -1;
  load_p(i0, pf);
  const float nanv = nan_f();
  for (int i = i0; i < i1; ++i) {
    if (i + 1 < i1) load_p(i + 1, pn);
    int m = a.map ? a.map[i] : i;
    const bool bad = (unsigned)m >= (unsigned)a.map_rows;
    if (bad) m = 0;
    if (m != mc) {
#pragma unroll
      for (int qb = 0; qb < NQR; ++qb) {
        const bf16* rp = a.x_r + int64_t(m) * a.ldxr + int64_t(qb * 16 + r16) * D + kq;
#pragma unroll
        for (int kd = 0; kd < KD; ++kd) rq[qb][kd] = __builtin_bit_cast(bf16x8, frag(rp, true, kd * 32));
      }
      mc = m;
    }
    bf16* out = a.f_c + int64_t(i) * a.ldfc;
    const int orow = r16;
#pragma unroll
    for (int qb = 0; qb <= NQR; ++qb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kd = 0; kd < KD; ++kd)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb < NQR ? rq[qb][kd] : pf[kd], pf[kd], acc, 0, 0, 0);
      const int ocol = qb * 16 + 4 * (lane >> 4);
      if (orow < nc) {
        bf16* o = out + int64_t(orow) * ncols + ocol;
        if (ocol + 4 <= ncols && (ncols & 3) == 0) {
          bf16x4 pk = {to_bf(bad ? nanv : acc[0]), to_bf(bad ? nanv : acc[1]), to_bf(bad ? nanv : acc[2]),
                       to_bf(bad ? nanv : acc[3])};
          *reinterpret_cast<bf16x4*>(o) = pk;
        } else {
          for (int j = 0; j < 4; ++j)
            if (ocol + j < ncols) o[j] = to_bf(bad ? nanv : acc[j]);
        }
      }
    }
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) pf[kd] = pn[kd];
  }
}

// ----------------------------------------------------------------- token-axis LCB
// Request half: T_R[b] = W_RR X_R[b] (bf16) and Z[b] = W_CR X_R[b] (fp32), once
// per request.  One workgroup per request; thread item = (output token t, 8
// consecutive dims); the contraction over input tokens runs in ascending order.
__global__ __launch_bounds__(256) void tok_request_kernel(TokLcbArgs a) {
  extern __shared__ uint4 smem_raw[];
  bf16* xs = reinterpret_cast<bf16*>(smem_raw);  // [n_r][dim]
  const int b = blockIdx.x;
  const int D = a.dim, nr = a.n_r;
  const bf16* x = a.x_r + int64_t(b) * a.ldxr;
  for (int e = threadIdx.x; e < nr * D / 8; e += 256)
    reinterpret_cast<uint4*>(xs)[e] = reinterpret_cast<const uint4*>(x)[e];
  __syncthreads();
  const int dv = D / 8;
  const int items = (a.t_r + a.t_c) * dv;
  for (int it = threadIdx.x; it < items; it += 256) {
    const int t = it / dv, d0 = (it - t * dv) * 8;
    const bool is_r = t < a.t_r;
    const bf16* w = is_r ? a.w_rr + int64_t(t) * nr : a.w_cr + int64_t(t - a.t_r) * nr;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < nr; ++k) {
      const float wk = to_f(w[k]);
      const uint4 u = *reinterpret_cast<const uint4*>(xs + k * D + d0);
      const bf16* xv = reinterpret_cast<const bf16*>(&u);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(wk, to_f(xv[j]), acc[j]);
    }
    if (is_r) {
      bf16x8 pk;
#pragma unroll
      for (int j = 0; j < 8; ++j) pk[j] = to_bf(acc[j]);
      *reinterpret_cast<bf16x8*>(a.y_r + int64_t(b) * a.ldyr + int64_t(t) * D + d0) = pk;
    } else {
      float* z = a.z + int64_t(b) * (int64_t(a.t_c) * D) + int64_t(t - a.t_r) * D + d0;
      *reinterpret_cast<float4*>(z) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *reinterpret_cast<float4*>(z + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

// Candidate half: T_C[i] = W_CC X_C[i] + Z[m_i].  A workgroup walks CPW
// consecutive candidates; each thread owns IT fixed (token, 8-dim) items and
// keeps the fp32 request contribution Z[m] in registers while consecutive
// candidates share m, so Z is read once per (workgroup, request) instead of
// once per candidate.  The candidate tokens are staged in LDS.
template <int IT>
__global__ __launch_bounds__(256) void tok_candidate_kernel(TokLcbArgs a, int cpw) {
  extern __shared__ uint4 smem_raw[];
  const int D = a.dim, nc = a.n_c, tc = a.t_c;
  bf16* ws = reinterpret_cast<bf16*>(smem_raw);      // [t_c][n_c]
  bf16* xs = ws + ((tc * nc + 7) / 8) * 8;            // [n_c][D]
  for (int e = threadIdx.x; e < tc * nc; e += 256) ws[e] = a.w_cc[e];
  const int dv = D / 8;
  const int items = tc * dv;
  float zc[IT][8];
  int zm = -2;
  const int i0 = blockIdx.x * cpw;
  const int i1 = min(i0 + cpw, a.B_c);
  for (int i = i0; i < i1; ++i) {
    __syncthreads();
    const bf16* x = a.x_c + int64_t(i) * a.ldxc;
    for (int e = threadIdx.x; e < nc * D / 8; e += 256)
      reinterpret_cast<uint4*>(xs)[e] = reinterpret_cast<const uint4*>(x)[e];
    __syncthreads();
    int m = a.map ? a.map[i] : i;
    const bool bad = (unsigned)m >= (unsigned)a.map_rows;
    if (bad) m = -1;
    if (m != zm) {
#pragma unroll
      for (int q = 0; q < IT; ++q) {
        const int it = threadIdx.x + q * 256;
        if (it < items && m >= 0) {
          const int t = it / dv, d0 = (it - t * dv) * 8;
          const float* z = a.z + int64_t(m) * (int64_t(tc) * D) + int64_t(t) * D + d0;
          const float4 z0 = *reinterpret_cast<const float4*>(z);
          const float4 z1 = *reinterpret_cast<const float4*>(z + 4);
          zc[q][0] = z0.x; zc[q][1] = z0.y; zc[q][2] = z0.z; zc[q][3] = z0.w;
          zc[q][4] = z1.x; zc[q][5] = z1.y; zc[q][6] = z1.z; zc[q][7] = z1.w;
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) zc[q][j] = nan_f();
        }
      }
      zm = m;
    }
#pragma unroll
    for (int q = 0; q < IT; ++q) {
      const int it = threadIdx.x + q * 256;
      if (it >= items) continue;
      const int t = it / dv, d0 = (it - t * dv) * 8;
      float acc[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = 0.f;
      for (int k = 0; k < nc; ++k) {
        const float wk = to_f(ws[t * nc + k]);
        const uint4 u = *reinterpret_cast<const uint4*>(xs + k * D + d0);
        const bf16* xv = reinterpret_cast<const bf16*>(&u);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(wk, to_f(xv[j]), acc[j]);
      }
      bf16x8 pk;
#pragma unroll
      for (int j = 0; j < 8; ++j) pk[j] = to_bf(acc[j] + zc[q][j]);
      *reinterpret_cast<bf16x8*>(a.y_c + int64_t(i) * a.ldyc + int64_t(t) * D + d0) = pk;
    }
  }
}

// Request half on the matrix cores: per request, [T_R; Z] = [W_RR; W_CR]
// X_R[b], a [(t_r + t_c) x n_r] x [n_r x D] product (TB blocks of 32 output
// tokens, KS k-steps of 16 input tokens, zero-padded).  Wave w owns the 32
// dims d = 32w..32w+31 (A operand X_R[b]^T, gathered from memory; B operand
// the stacked weights).  Rows below t_r are T_R (bf16), the rest Z (fp32),
// stored straight from the MFMA layout: one workgroup per request, few of
// them, so the stores' row pattern does not matter.
template <int TB, int KS>
__global__ __launch_bounds__(256) void tok_request_mfma_kernel(TokLcbArgs a) {
  const int D = a.dim, nr = a.n_r, tr = a.t_r, tc = a.t_c, T = tr + tc;
  const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
  const int db = threadIdx.x >> 6;
  const int d = db * 32 + l32;
  const int b = blockIdx.x;
  const bf16* x = a.x_r + int64_t(b) * a.ldxr;
  bf16x8 xf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = ks * 16 + 8 * h + e;
      xf[ks][e] = k < nr ? x[k * D + d] : bf16(0.f);
    }
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int t = tb * 32 + l32;
    const bf16* w = t < tr ? a.w_rr + int64_t(t) * nr : a.w_cr + int64_t(t - tr) * nr;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 wf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = ks * 16 + 8 * h + e;
        wf[e] = (t < T && k < nr) ? w[k] : bf16(0.f);
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf[ks], wf, acc, 0, 0, 0);
    }
    if (t >= T) continue;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = db * 32 + 8 * g + 4 * h;
      if (t < tr) {
        bf16x4 pk = {to_bf(acc[4 * g]), to_bf(acc[4 * g + 1]), to_bf(acc[4 * g + 2]), to_bf(acc[4 * g + 3])};
        *reinterpret_cast<bf16x4*>(a.y_r + int64_t(b) * a.ldyr + int64_t(t) * D + d0) = pk;
      } else {
        *reinterpret_cast<float4*>(a.z + int64_t(b) * (int64_t(tc) * D) + int64_t(t - tr) * D + d0) =
            make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
      }
    }
  }
}

// Candidate half on the matrix cores: per candidate, T_C = W_CC X_C[i] is a
// [t_c x n_c] x [n_c x D] product, i.e. TB x (D / 32) blocks of
// v_mfma_f32_32x32x16_bf16 with KS k-steps of 16 input tokens (zero-padded).
// Wave w owns the 32 dims d = 32w..32w+31: its A operand is X_C[i]^T (row d,
// 8 consecutive input tokens per lane half, gathered straight from memory),
// its B operand W_CC (row t), so a lane ends with 4 consecutive d of one t.
// The fp32 request contribution Z[m] for those positions stays in registers
// while consecutive candidates share m.  The rounded block goes through an
// LDS stage and leaves as contiguous 16-byte chunks of the candidate's
// [t_c x D] output.
template <int TB, int KS>
__global__ __launch_bounds__(256) void tok_candidate_mfma_kernel(TokLcbArgs a, int cpw) {
  extern __shared__ uint4 smem_raw[];
  bf16* stage = reinterpret_cast<bf16*>(smem_raw);  // [t_c][D + 8]
  const int D = a.dim, nc = a.n_c, tc = a.t_c;
  const int SP = D + 8;
  const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
  const int db = threadIdx.x >> 6;
  const int d = db * 32 + l32;  // this lane's A-operand row
  bf16x8 wf[TB][KS];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = tb * 32 + l32, k = ks * 16 + 8 * h + e;
        wf[tb][ks][e] = (t < tc && k < nc) ? a.w_cc[t * nc + k] : bf16(0.f);
      }
  float zc[TB][4][4];
  int zm = -2;
  const int i0 = blockIdx.x * cpw;
  const int i1 = min(i0 + cpw, a.B_c);
  const int nch = tc * (D / 8);
  for (int i = i0; i < i1; ++i) {
    const bf16* x = a.x_c + int64_t(i) * a.ldxc;
    bf16x8 xf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = ks * 16 + 8 * h + e;
        xf[ks][e] = k < nc ? x[k * D + d] : bf16(0.f);
      }
    int m = a.map ? a.map[i] : i;
    if ((unsigned)m >= (unsigned)a.map_rows) m = -1;
    if (m != zm) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int t = tb * 32 + l32;
          float4 v = make_float4(nan_f(), nan_f(), nan_f(), nan_f());
          if (m >= 0 && t < tc)
            v = *reinterpret_cast<const float4*>(a.z + int64_t(m) * (int64_t(tc) * D) + int64_t(t) * D + db * 32 +
                                                 8 * g + 4 * h);
          zc[tb][g][0] = v.x; zc[tb][g][1] = v.y; zc[tb][g][2] = v.z; zc[tb][g][3] = v.w;
        }
      zm = m;
    }
    f32x16 acc[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf[ks], wf[tb][ks], acc[tb], 0, 0, 0);
    }
    __syncthreads();  // the previous candidate's stage has been read
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int t = tb * 32 + l32;
      if (t < tc)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 pk = {to_bf(acc[tb][4 * g] + zc[tb][g][0]), to_bf(acc[tb][4 * g + 1] + zc[tb][g][1]),
                       to_bf(acc[tb][4 * g + 2] + zc[tb][g][2]), to_bf(acc[tb][4 * g + 3] + zc[tb][g][3])};
          *reinterpret_cast<bf16x4*>(stage + t * SP + db * 32 + 8 * g + 4 * h) = pk;
        }
    }
    __syncthreads();
    bf16* y = a.y_c + int64_t(i) * a.ldyc;
    for (int c = threadIdx.x; c < nch; c += blockDim.x) {
      const int t = c / (D / 8), d8 = c - t * (D / 8);
      *reinterpret_cast<uint4*>(y + t * D + d8 * 8) = *reinterpret_cast<const uint4*>(stage + t * SP + d8 * 8);
    }
  }
}

}  // namespace

namespace {

using FmKernel = void (*)(FmArgs, int);

// fm_fast_kernel for NPB x NQB blocks and D = 32 KD, when instantiated.
template <int NPB>
FmKernel fm_fast_for(int nqb, int kd) {
  const int key = nqb * 16 + kd;
  switch (key) {
    case 1 * 16 + 2: return fm_fast_kernel<NPB, 1, 2>;
    case 2 * 16 + 2: return fm_fast_kernel<NPB, 2, 2>;
    case 3 * 16 + 2: return fm_fast_kernel<NPB, 3, 2>;
    case 4 * 16 + 2: return fm_fast_kernel<NPB, 4, 2>;
    case 1 * 16 + 4: return fm_fast_kernel<NPB, 1, 4>;
    case 2 * 16 + 4: return fm_fast_kernel<NPB, 2, 4>;
    case 3 * 16 + 4: return fm_fast_kernel<NPB, 3, 4>;
    case 4 * 16 + 4: return fm_fast_kernel<NPB, 4, 4>;
    default: return nullptr;
  }
}

FmKernel fm_kernel_for(int np, int nq, int dim) {
  if (dim % 32 != 0) return fm_kernel;
  const int npb = (np + 15) / 16, nqb = (nq + 15) / 16, kd = dim / 32;
  FmKernel k = nullptr;
  if (npb == 1) k = fm_fast_for<1>(nqb, kd);
  if (npb == 2) k = fm_fast_for<2>(nqb, kd);
  return k ? k : fm_kernel;
}

}  // namespace

hipError_t launch_fm(const FmArgs& a, hipStream_t s) {
  if (a.B_r > 0)
    hipLaunchKernelGGL(fm_kernel_for(a.n_r, a.n_r, a.dim), dim3((a.B_r + 3) / 4), dim3(256), 0, s, a, 1);
  if (a.B_c <= 0) return hipGetLastError();
  // candidates: the request-caching kernel for n_C <= 16, n_R in {16, 32, 48}
  // and D in {64, 128}; otherwise one item per wave
  const int nqr = a.n_r / 16;
  if (a.n_c <= 16 && a.n_r % 16 == 0 && nqr >= 1 && nqr <= 3 && (a.dim == 64 || a.dim == 128)) {
    const int ipw = 8;
    const dim3 grid((a.B_c + 4 * ipw - 1) / (4 * ipw)), block(256);
    const int key = nqr * 8 + a.dim / 32;
    switch (key) {
      case 1 * 8 + 2: hipLaunchKernelGGL((fm_cand_kernel<1, 2>), grid, block, 0, s, a, ipw); break;
      case 2 * 8 + 2: hipLaunchKernelGGL((fm_cand_kernel<2, 2>), grid, block, 0, s, a, ipw); break;
      case 3 * 8 + 2: hipLaunchKernelGGL((fm_cand_kernel<3, 2>), grid, block, 0, s, a, ipw); break;
      case 1 * 8 + 4: hipLaunchKernelGGL((fm_cand_kernel<1, 4>), grid, block, 0, s, a, ipw); break;
      case 2 * 8 + 4: hipLaunchKernelGGL((fm_cand_kernel<2, 4>), grid, block, 0, s, a, ipw); break;
      case 3 * 8 + 4: hipLaunchKernelGGL((fm_cand_kernel<3, 4>), grid, block, 0, s, a, ipw); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  hipLaunchKernelGGL(fm_kernel_for(a.n_c, a.n_r + a.n_c, a.dim), dim3((a.B_c + 3) / 4), dim3(256), 0, s, a, 0);
  return hipGetLastError();
}

hipError_t launch_token_lcb_request(const TokLcbArgs& a, hipStream_t s) {
  if (a.B_r <= 0) return hipSuccess;
  // Matrix-core path: D a multiple of 32 up to 128, up to 128 output and 32
  // input tokens, 8-byte aligned T_R rows.
  const int T = a.t_r + a.t_c;
  if (a.dim % 32 == 0 && a.dim <= 128 && T <= 128 && a.n_r <= 32 && (reinterpret_cast<uintptr_t>(a.y_r) & 7) == 0 &&
      a.ldyr % 4 == 0 && (reinterpret_cast<uintptr_t>(a.z) & 15) == 0) {
    const dim3 grid(a.B_r), block(64 * (a.dim / 32));
    const int key = ((T + 31) / 32) * 4 + (a.n_r + 15) / 16;
    switch (key) {
      case 1 * 4 + 1: hipLaunchKernelGGL((tok_request_mfma_kernel<1, 1>), grid, block, 0, s, a); break;
      case 1 * 4 + 2: hipLaunchKernelGGL((tok_request_mfma_kernel<1, 2>), grid, block, 0, s, a); break;
      case 2 * 4 + 1: hipLaunchKernelGGL((tok_request_mfma_kernel<2, 1>), grid, block, 0, s, a); break;
      case 2 * 4 + 2: hipLaunchKernelGGL((tok_request_mfma_kernel<2, 2>), grid, block, 0, s, a); break;
      case 3 * 4 + 1: hipLaunchKernelGGL((tok_request_mfma_kernel<3, 1>), grid, block, 0, s, a); break;
      case 3 * 4 + 2: hipLaunchKernelGGL((tok_request_mfma_kernel<3, 2>), grid, block, 0, s, a); break;
      case 4 * 4 + 1: hipLaunchKernelGGL((tok_request_mfma_kernel<4, 1>), grid, block, 0, s, a); break;
      case 4 * 4 + 2: hipLaunchKernelGGL((tok_request_mfma_kernel<4, 2>), grid, block, 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const size_t lds = size_t(a.n_r) * a.dim * 2;
  hipLaunchKernelGGL(tok_request_kernel, dim3(a.B_r), dim3(256), lds, s, a);
  return hipGetLastError();
}

namespace {

template <int TB>
hipError_t launch_tok_mfma(const TokLcbArgs& a, int ks, hipStream_t s) {
  const int cpw = 16;
  const size_t lds = size_t(TB * 32) * (a.dim + 8) * 2;
  const dim3 grid((a.B_c + cpw - 1) / cpw), block(64 * (a.dim / 32));
  switch (ks) {
    case 1: hipLaunchKernelGGL((tok_candidate_mfma_kernel<TB, 1>), grid, block, lds, s, a, cpw); break;
    case 2: hipLaunchKernelGGL((tok_candidate_mfma_kernel<TB, 2>), grid, block, lds, s, a, cpw); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_token_lcb_candidate(const TokLcbArgs& a, hipStream_t s) {
  if (a.B_c <= 0) return hipSuccess;
  // Matrix-core path: D a multiple of 32 up to 128 (one wave per 32 dims),
  // up to 128 output and 32 input tokens, 16-byte aligned output rows.
  const bool mfma_ok = a.dim % 32 == 0 && a.dim <= 128 && a.t_c <= 128 && a.n_c <= 32 &&
                       (reinterpret_cast<uintptr_t>(a.y_c) & 15) == 0 && a.ldyc % 8 == 0;
  if (mfma_ok) {
    const int tb = (a.t_c + 31) / 32, ks = (a.n_c + 15) / 16;
    switch (tb) {
      case 1: return launch_tok_mfma<1>(a, ks, s);
      case 2: return launch_tok_mfma<2>(a, ks, s);
      case 3: return launch_tok_mfma<3>(a, ks, s);
      case 4: return launch_tok_mfma<4>(a, ks, s);
      default: break;
    }
  }
  const int items = a.t_c * (a.dim / 8);
  const int it = (items + 255) / 256;
  const int cpw = 8;
  const size_t lds = size_t((a.t_c * a.n_c + 7) / 8) * 16 + size_t(a.n_c) * a.dim * 2;
  const dim3 grid((a.B_c + cpw - 1) / cpw), block(256);
  if (it <= 1)
    hipLaunchKernelGGL((tok_candidate_kernel<1>), grid, block, lds, s, a, cpw);
  else if (it <= 2)
    hipLaunchKernelGGL((tok_candidate_kernel<2>), grid, block, lds, s, a, cpw);
  else if (it <= 4)
    hipLaunchKernelGGL((tok_candidate_kernel<4>), grid, block, lds, s, a, cpw);
  else if (it <= 8)
    hipLaunchKernelGGL((tok_candidate_kernel<8>), grid, block, lds, s, a, cpw);
  else if (it <= 16)
    hipLaunchKernelGGL((tok_candidate_kernel<16>), grid, block, lds, s, a, cpw);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace rocs
