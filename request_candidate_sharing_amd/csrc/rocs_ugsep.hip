// UG-Separation TokenMixer ([U] "Compute Only Once: UG-Separation for
// Efficient Large Recommendation Models", xllm-io review, §3 core formulas,
// separation mask and information compensation).
//
// The U side (user tokens, n_u per request) is computed once per request;
// the G side (n_g tokens per candidate) reads its request's U tokens through
// the candidate -> request map, so no U token is copied per candidate.
//   ug_comp_kernel      Proj(U) = P U along the token axis, once per request
//                       (fp32, [B_r, n_g * dim]); the G side adds it by map.
//   mixup_norm_kernel   multi-head token mixing under the UG mask fused
//                       with the LayerNorm that follows it: one wave per
//                       output token row; U rows and G rows in one launch.
// The per-token FFN runs on the GEMM kernels (one launch per token).
#include <algorithm>

#include "rocs_device.h"

namespace rocs {

namespace {

// uc[b, g, e] = sum_u P[g, u] * x_u[b, u, e]  (fma chain over u in order).
template <typename T>
__global__ __launch_bounds__(256) void ug_comp_kernel(CompArgs a) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = int64_t(a.rows) * a.n_g * a.dim;
  if (idx >= total) return;
  const int e = int(idx % a.dim);
  const int64_t q = idx / a.dim;
  const int g = int(q % a.n_g);
  const int b = int(q / a.n_g);
  const T* x = reinterpret_cast<const T*>(a.xu) + int64_t(b) * a.ldxu + e;
  float s = 0.f;
  for (int u = 0; u < a.n_u; ++u) s = fmaf(a.P[g * a.n_u + u], to_f(x[int64_t(u) * a.dim]), s);
  a.uc[int64_t(b) * a.lduc + int64_t(g) * a.dim + e] = s;
}

// Output token h of a sample is the concatenation over input tokens t of
// chunk h (width cw = dim / T) of token t; in U outputs (h < n_u) the chunks
// of G tokens are zero.  G tokens are read compensated (+ uc of the
// request).  The mixed row is then layer-normalised over its dim features
// (fp32 two-pass statistics, the row held in registers).  Workgroups
// [0, nblk_u) take U rows (sample = request), the rest G rows (sample =
// candidate).  cw is a multiple of the 16-byte vector, so each vector lies
// inside one chunk.
template <typename T, int CH>
__global__ __launch_bounds__(256) void mixup_norm_kernel(MixupArgs a, int nblk_u) {
  constexpr int VEC = 16 / sizeof(T);
  const bool gside = int(blockIdx.x) >= nblk_u;
  const int lane = threadIdx.x & 63;
  const int row = (gside ? int(blockIdx.x) - nblk_u : int(blockIdx.x)) * 4 + (threadIdx.x >> 6);
  const int per = gside ? a.n_g : a.n_u;
  const int nrows = (gside ? a.rows_g : a.rows_u) * per;
  if (per == 0 || row >= nrows) return;
  const int s = row / per;
  const int h = (gside ? a.n_u : 0) + row % per;
  const int T_ = a.n_u + a.n_g;
  const int cw = a.dim / T_;
  const int b = gside ? (a.map ? a.map[s] : s) : s;  // no map: one U row per candidate
  const bool bad = (unsigned)b >= (unsigned)a.rows_u;
  const T* xu = reinterpret_cast<const T*>(a.xu) + int64_t(bad ? 0 : b) * a.ldxu;
  const T* xg = gside ? reinterpret_cast<const T*>(a.xg) + int64_t(s) * a.ldxg : nullptr;
  const float* uc = (gside && a.uc) ? a.uc + int64_t(bad ? 0 : b) * a.lduc : nullptr;
  // all loads of the row first (kept in flight together), then the sums
  // Branch-free: every lane loads from an address inside its sample's rows
  // (lanes past the row end, and U-output lanes on G chunks, load a valid U
  // vector instead) and keeps or drops the value by a select afterwards.
  // Chunks that start past the row are skipped by a uniform test.
  uint4 raw[CH];
  float4 cq[CH][VEC / 4];
  bool keep[CH], comp[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int e0 = (c * 64 + lane) * VEC;
    raw[c] = make_uint4(0, 0, 0, 0);
    keep[c] = comp[c] = false;
#pragma unroll
    for (int k = 0; k < VEC / 4; ++k) cq[c][k] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c * 64 * VEC < a.dim) {
      const int ec = min(e0, a.dim - VEC);
      const int t = ec / cw;
      const int col = h * cw + (ec - t * cw);
      const bool from_u = t < a.n_u, from_g = !from_u && gside;
      keep[c] = e0 < a.dim && (from_u || from_g);
      const int tg = max(t - a.n_u, 0);
      const T* src = from_g ? xg + tg * a.dim + col : xu + int64_t(from_u ? t : 0) * a.dim + col;
      raw[c] = *reinterpret_cast<const uint4*>(src);
      if (uc) {
        comp[c] = keep[c] && from_g;
#pragma unroll
        for (int k = 0; k < VEC / 4; ++k) cq[c][k] = *reinterpret_cast<const float4*>(uc + tg * a.dim + col + 4 * k);
      }
    }
  }
  float v[CH][VEC];
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const T* tw = reinterpret_cast<const T*>(&raw[c]);
#pragma unroll
    for (int j = 0; j < VEC; ++j) v[c][j] = keep[c] ? to_f(tw[j]) : 0.f;
    if (comp[c]) {
#pragma unroll
      for (int k = 0; k < VEC / 4; ++k) {
        v[c][4 * k] += cq[c][k].x;
        v[c][4 * k + 1] += cq[c][k].y;
        v[c][4 * k + 2] += cq[c][k].z;
        v[c][4 * k + 3] += cq[c][k].w;
      }
    }
#pragma unroll
    for (int j = 0; j < VEC; ++j) sum += v[c][j];
  }
  const float inv_w = 1.0f / float(a.dim);
  const float mean = wave_sum(sum) * inv_w;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    if ((c * 64 + lane) * VEC >= a.dim) continue;
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      const float d = v[c][j] - mean;
      q += d * d;
    }
  }
  const float scale = bad ? nan_f() : 1.0f / sqrtf(wave_sum(q) * inv_w + a.eps);
  const T* gam = reinterpret_cast<const T*>(a.gamma);
  const T* bet = reinterpret_cast<const T*>(a.beta);
  T* y = reinterpret_cast<T*>(gside ? a.pg : a.pu) + int64_t(s) * (gside ? a.ldpg : a.ldpu) +
         int64_t(h - (gside ? a.n_u : 0)) * a.dim;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int e0 = (c * 64 + lane) * VEC;
    if (e0 >= a.dim) continue;
    const uint4 gw = *reinterpret_cast<const uint4*>(gam + e0);
    const uint4 bw = *reinterpret_cast<const uint4*>(bet + e0);
    const T* tg = reinterpret_cast<const T*>(&gw);
    const T* tb = reinterpret_cast<const T*>(&bw);
    T out[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) out[j] = from_f<T>((v[c][j] - mean) * scale * to_f(tg[j]) + to_f(tb[j]));
    *reinterpret_cast<uint4*>(y + e0) = *reinterpret_cast<const uint4*>(out);
  }
}

template <typename T>
hipError_t mixup_dispatch(const MixupArgs& a, hipStream_t s) {
  constexpr int VEC = 16 / sizeof(T);
  const int ch = (a.dim + 64 * VEC - 1) / (64 * VEC);
  const int nu = (a.rows_u * a.n_u + 3) / 4;
  const int ng = (a.rows_g * a.n_g + 3) / 4;
  if (nu + ng == 0) return hipSuccess;
  const dim3 grid(nu + ng), block(256);
  switch (ch) {
    case 1: hipLaunchKernelGGL((mixup_norm_kernel<T, 1>), grid, block, 0, s, a, nu); break;
    case 2: hipLaunchKernelGGL((mixup_norm_kernel<T, 2>), grid, block, 0, s, a, nu); break;
    case 3: hipLaunchKernelGGL((mixup_norm_kernel<T, 3>), grid, block, 0, s, a, nu); break;
    case 4: hipLaunchKernelGGL((mixup_norm_kernel<T, 4>), grid, block, 0, s, a, nu); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int mixup_max_dim(DType dt) { return 4 * 64 * (dt == F32 ? 4 : 8); }

hipError_t launch_mixup_norm(DType dt, const MixupArgs& a, hipStream_t s) {
  if (a.dim > mixup_max_dim(dt)) return hipErrorInvalidValue;
  return dt == F32 ? mixup_dispatch<float>(a, s) : mixup_dispatch<bf16>(a, s);
}

hipError_t launch_ug_comp(DType dt, const CompArgs& a, hipStream_t s) {
  const int64_t total = int64_t(a.rows) * a.n_g * a.dim;
  if (total == 0) return hipSuccess;
  const dim3 grid(unsigned((total + 255) / 256)), block(256);
  if (dt == F32)
    hipLaunchKernelGGL(ug_comp_kernel<float>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(ug_comp_kernel<bf16>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace rocs
