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

}  // namespace

hipError_t launch_fm(const FmArgs& a, hipStream_t s) {
  if (a.B_r > 0) hipLaunchKernelGGL(fm_kernel, dim3((a.B_r + 3) / 4), dim3(256), 0, s, a, 1);
  if (a.B_c > 0) hipLaunchKernelGGL(fm_kernel, dim3((a.B_c + 3) / 4), dim3(256), 0, s, a, 0);
  return hipGetLastError();
}

hipError_t launch_token_lcb_request(const TokLcbArgs& a, hipStream_t s) {
  if (a.B_r <= 0) return hipSuccess;
  const size_t lds = size_t(a.n_r) * a.dim * 2;
  hipLaunchKernelGGL(tok_request_kernel, dim3(a.B_r), dim3(256), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_token_lcb_candidate(const TokLcbArgs& a, hipStream_t s) {
  if (a.B_c <= 0) return hipSuccess;
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
