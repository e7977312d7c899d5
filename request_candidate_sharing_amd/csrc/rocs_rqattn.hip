// Request-side DCA cross-attention computed from the encoder output itself.
//
// [R] §2.2, grouped cross-attention: the request query group attends to
// K^R = S W_K^R and V^R = S W_V^R of its own request's sequence S, one query
// row per request and head.  With one query per (request, head), projecting
// all L keys and values first is wasted work.  Re-associating the products
// gives the same attention from S directly (exact in real arithmetic):
//   score_h(l) = q_h . (W_K,h S_l) = (W_K,h^T q_h) . S_l = q'_h . S_l
//   A_h        = sum_l p_h(l) W_V,h S_l = W_V,h (sum_l p_h(l) S_l) = W_V,h u_h
// with W_K,h, W_V,h the 64 rows of head h ([out, in] weights).  Three
// launches, fp32 except S and the weights (bf16) and q' as an MFMA operand:
//   rq_fold     q'_h = scale log2(e) W_K,h^T q_h          per (request, head)
//   rq_attend   64 events per workgroup: scores of every head (MFMA, q' in
//               bf16), the chunk's maximum m_h, p = 2^(s - m_h), l_h = sum p,
//               u_h = sum p S_l
//   rq_combine  chunks merged per (request, head) in a fixed order,
//               A_h = W_V,h (u_h / l_h), rounded once to bf16
#include "rocs_device.h"

namespace rocs {

namespace {

constexpr int RQ_CHUNK = 64;  // events per workgroup
constexpr int RQ_WROWS = 16;  // events per wave

template <int H>
struct RowFrag;
template <>
struct RowFrag<8> {
  using T = uint4;
};
template <>
struct RowFrag<4> {
  using T = uint2;
};
template <>
struct RowFrag<2> {
  using T = uint32_t;
};
template <>
struct RowFrag<1> {
  using T = uint16_t;
};

template <int H>
__device__ __forceinline__ void unpack_row(const typename RowFrag<H>::T& u, float (&x)[H]) {
  const bf16* e = reinterpret_cast<const bf16*>(&u);
#pragma unroll
  for (int i = 0; i < H; ++i) x[i] = to_f(e[i]);
}

// Lane mask of the upper lanes of offset o ((lane & o) != 0), for the
// halving steps below.
template <int O>
constexpr uint64_t upper_lanes() {
  uint64_t m = 0;
  for (int l = 0; l < 64; ++l)
    if (l & O) m |= uint64_t(1) << l;
  return m;
}

// x where the lane's bit of mask is clear, y where it is set.  Written as one
// v_cndmask: as a C select between two elements of a register array the
// compiler turns it into an indexed read, which it lowers into a compare
// and select over every element.
__device__ __forceinline__ float lane_select(float x, float y, uint64_t mask) {
  float r;
  asm volatile("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "s"(mask));
  return r;
}

template <int O, int HALF, int H, bool MAX>
__device__ __forceinline__ void halving_step(float (&v)[H]) {
  constexpr uint64_t up = upper_lanes<O>();
#pragma unroll
  for (int j = 0; j < HALF; ++j) {
    const float mine = lane_select(v[j], v[HALF + j], up);
    const float other = lane_select(v[HALF + j], v[j], up);
    const float got = __shfl_xor(other, O, 64);
    v[j] = MAX ? fmaxf(mine, got) : mine + got;
  }
}

// Sum (or maximum) over the 64 lanes of H values per lane.  Each halving
// step exchanges half of the values with the lane at offset o (upper lanes
// keep the upper half), so log2(H) steps leave one value per lane, that of
// head head_of_lane<H>(lane); plain butterfly steps then finish.  The order
// of operations is fixed (deterministic).
template <int H, bool MAX>
__device__ __forceinline__ float transpose_reduce(float (&v)[H]) {
  constexpr int LOGH = H == 8 ? 3 : H == 4 ? 2 : H == 2 ? 1 : 0;
  if constexpr (LOGH >= 1) halving_step<32, H / 2, H, MAX>(v);
  if constexpr (LOGH >= 2) halving_step<16, H / 4, H, MAX>(v);
  if constexpr (LOGH >= 3) halving_step<8, H / 8, H, MAX>(v);
#pragma unroll
  for (int o = 32 >> LOGH; o >= 1; o >>= 1) {
    const float got = __shfl_xor(v[0], o, 64);
    v[0] = MAX ? fmaxf(v[0], got) : v[0] + got;
  }
  return v[0];
}

template <int H>
__device__ __forceinline__ int head_of_lane(int lane) {
  int h = 0;
#pragma unroll
  for (int s = 0, half = H >> 1; half >= 1; ++s, half >>= 1)
    if (lane & (32 >> s)) h += half;
  return h;
}

// q'_h[i] = scale_log2 * sum_e q[h*64 + e] W_K[h*64 + e][i] (d <= 512).
// Thread t takes eight consecutive features and a quarter of the 64 rows of
// head h, with all of its loads issued before the sums; the four quarters
// are then added in order.
__global__ __launch_bounds__(256) void rq_fold_kernel(RqAttnArgs a) {
  const int b = blockIdx.x / a.H, h = blockIdx.x - (blockIdx.x / a.H) * a.H;
  const int d = 64 * a.H;
  __shared__ float qs[64];
  __shared__ float part[4][512];
  if (threadIdx.x < 64) qs[threadIdx.x] = to_f(a.q[int64_t(b) * a.ldq + h * 64 + threadIdx.x]);
  __syncthreads();
  const int fq = threadIdx.x >> 6, i0 = (threadIdx.x & 63) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (i0 < d) {
    const bf16* w = a.wk + (int64_t(h) * 64 + fq * 16) * a.ldw + i0;
    uint4 rows[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) rows[e] = *reinterpret_cast<const uint4*>(w + int64_t(e) * a.ldw);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const bf16* x = reinterpret_cast<const bf16*>(&rows[e]);
      const float qe = qs[fq * 16 + e];
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = fmaf(qe, to_f(x[k]), acc[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) part[fq][i0 + k] = acc[k];
  __syncthreads();
  for (int i = threadIdx.x; i < d; i += 256)
    a.qf[(int64_t(b) * a.H + h) * d + i] = (((part[0][i] + part[1][i]) + part[2][i]) + part[3][i]) * a.scale_log2;
}

// Scores of a wave's 16 events for every head on v_mfma_f32_16x16x32_bf16:
// the event rows are the first operand (lane l supplies row l % 16, eight K
// elements at 8 (l / 16) of each 32-wide K step), q' rounded to bf16 the
// second (column l % 16 = head; heads past H are zero), so lane l ends with
// the scores of events 4 (l / 16) + j (j < 4) for head l % 16.  The
// contributions p S_l to u then run on the VALU with a lane owning H
// consecutive features (the rows are read again, from L2).
template <int H>
__global__ __launch_bounds__(256, 2) void rq_attend_kernel(RqAttnArgs a) {
  constexpr int D = 64 * H;
  constexpr int KB = D / 32;  // 32-wide K steps
  using Frag = typename RowFrag<H>::T;
  const int nch = (a.L + RQ_CHUNK - 1) / RQ_CHUNK;
  const int b = blockIdx.x / nch, ch = blockIdx.x - (blockIdx.x / nch) * nch;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, kg = lane >> 4;
  __shared__ float sc[RQ_CHUNK][H];
  __shared__ float mx[H];
  __shared__ float ured[H][D];
  __shared__ float lred[4][H];

  const int r0 = ch * RQ_CHUNK + wave * RQ_WROWS;
  const bf16* sb = a.s + (int64_t(b) * a.L) * a.lds;
  // MFMA operands: this lane's event row and q' row, all K steps requested up front
  uint4 sf[KB];
  {
    const int r = r0 + r16;
    const bf16* rp = sb + int64_t(r < a.L ? r : 0) * a.lds + kg * 8;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      sf[kb] = r < a.L ? *reinterpret_cast<const uint4*>(rp + kb * 32) : make_uint4(0, 0, 0, 0);
  }
  bf16x8 qf[KB];
  {
    const float* qp = a.qf + (int64_t(b) * H + (r16 < H ? r16 : 0)) * D + kg * 8;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const float4 lo = *reinterpret_cast<const float4*>(qp + kb * 32);
      const float4 hi = *reinterpret_cast<const float4*>(qp + kb * 32 + 4);
      const bool on = r16 < H;
      qf[kb] = bf16x8{to_bf(on ? lo.x : 0.f), to_bf(on ? lo.y : 0.f), to_bf(on ? lo.z : 0.f), to_bf(on ? lo.w : 0.f),
                      to_bf(on ? hi.x : 0.f), to_bf(on ? hi.y : 0.f), to_bf(on ? hi.z : 0.f), to_bf(on ? hi.w : 0.f)};
    }
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, sf[kb]), qf[kb], acc, 0, 0, 0);
  if (r16 < H) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rl = wave * RQ_WROWS + 4 * kg + j;
      sc[rl][r16] = (ch * RQ_CHUNK + rl < a.L) ? acc[j] : -INFINITY;
    }
  }
  // the rows again, one H-wide slice per lane, for the contributions to u
  Frag rows[RQ_WROWS];
#pragma unroll
  for (int j = 0; j < RQ_WROWS; ++j) {
    const int r = r0 + j;
    rows[j] = r < a.L ? *reinterpret_cast<const Frag*>(sb + int64_t(r) * a.lds + lane * H) : Frag{};
  }
  __syncthreads();
  const int hsel = head_of_lane<H>(lane);
  const bool writer = (lane & ((64 / H) - 1)) == 0;
  if (wave == 0) {
    float v[H];
#pragma unroll
    for (int h = 0; h < H; ++h) v[h] = sc[lane][h];
    const float m = transpose_reduce<H, true>(v);
    if (writer) mx[hsel] = m;
  }
  __syncthreads();

  // p = 2^(s - m_h) of the wave's events, each (event, head) once per wave
  // and in place (every lane needs all of them below); events past L have
  // score -inf (p = 0) and zero rows: they add nothing
#pragma unroll
  for (int t = 0; t < (RQ_WROWS * H + 63) / 64; ++t) {
    const int i = lane + 64 * t;
    if (i < RQ_WROWS * H) {
      const int j = i / H, h = i - (i / H) * H;
      float& e = sc[wave * RQ_WROWS + j][h];
      e = __builtin_amdgcn_exp2f(e - mx[h]);  // argument <= 0
    }
  }
  __syncthreads();

  float l[H], u[H][H];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < H; ++e) u[h][e] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < RQ_WROWS; ++j) {
    float x[H];
    unpack_row<H>(rows[j], x);
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const float p = sc[wave * RQ_WROWS + j][h];
      l[h] += p;
#pragma unroll
      for (int e = 0; e < H; ++e) u[h][e] = fmaf(p, x[e], u[h][e]);
    }
  }
  // waves combine in a fixed order: ((u3 + u2) + u1) + u0.  (A two-level
  // tree through a lane-contiguous layout measured slower: 27 vs 22 us.)
  if (lane == 0)
#pragma unroll
    for (int h = 0; h < H; ++h) lred[wave][h] = l[h];
  for (int w = 3; w >= 1; --w) {
    if (wave == w) {
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int e = 0; e < H; ++e) {
          float& slot = ured[h][lane * H + e];
          slot = (w == 3) ? u[h][e] : slot + u[h][e];
        }
    }
    __syncthreads();
  }
  if (wave != 0) return;
  const int64_t pbase = (int64_t(b) * nch + ch) * H;
#pragma unroll
  for (int h = 0; h < H; ++h) {
    float* up = a.part_u + (pbase + h) * D + lane * H;
#pragma unroll
    for (int e = 0; e < H; ++e) up[e] = ured[h][lane * H + e] + u[h][e];
  }
  if (lane < H) {
    const float lt = ((lred[3][lane] + lred[2][lane]) + lred[1][lane]) + lred[0][lane];
    a.part_ml[2 * (pbase + lane) + 0] = mx[lane];
    a.part_ml[2 * (pbase + lane) + 1] = lt;
  }
}

// out[h*64 + e] = W_V[h*64 + e] . (sum_c 2^(m_c - M) u_c / sum_c 2^(m_c - M) l_c),
// chunks summed in ascending order.  The chunk statistics go to LDS first;
// each wave then forms 16 outputs with one 16-byte weight load per lane per
// output, all issued before the products.
template <int H>
__global__ __launch_bounds__(256) void rq_combine_kernel(RqAttnArgs a) {
  constexpr int D = 64 * H;
  const int b = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  const int nch = (a.L + RQ_CHUNK - 1) / RQ_CHUNK;
  __shared__ float us[D];
  __shared__ float wc[1024];
  __shared__ float lc[1024];
  __shared__ float stats[2];
  const float* ml = a.part_ml + 2 * (int64_t(b) * nch * H + h);
  for (int c = threadIdx.x; c < nch; c += 256) {
    wc[c] = ml[2 * c * H];
    lc[c] = ml[2 * c * H + 1];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c) M = fmaxf(M, wc[c]);
    stats[0] = M;
  }
  __syncthreads();
  const float M = stats[0];
  for (int c = threadIdx.x; c < nch; c += 256) wc[c] = __builtin_amdgcn_exp2f(wc[c] - M);  // argument <= 0
  __syncthreads();
  if (threadIdx.x == 0) {
    float lsum = 0.f;
    for (int c = 0; c < nch; ++c) lsum = fmaf(wc[c], lc[c], lsum);
    stats[1] = 1.f / lsum;
  }
  __syncthreads();
  const float inv = stats[1];
  for (int i = threadIdx.x; i < D; i += 256) {
    const float* pu = a.part_u + (int64_t(b) * nch * H + h) * D + i;
    float acc = 0.f;
    int c = 0;
    for (; c + 4 <= nch; c += 4) {
      const float x0 = pu[int64_t(c) * H * D], x1 = pu[int64_t(c + 1) * H * D];
      const float x2 = pu[int64_t(c + 2) * H * D], x3 = pu[int64_t(c + 3) * H * D];
      acc = fmaf(wc[c], x0, acc);
      acc = fmaf(wc[c + 1], x1, acc);
      acc = fmaf(wc[c + 2], x2, acc);
      acc = fmaf(wc[c + 3], x3, acc);
    }
    for (; c < nch; ++c) acc = fmaf(wc[c], pu[int64_t(c) * H * D], acc);
    us[i] = acc * inv;
  }
  __syncthreads();
  using Frag = typename RowFrag<H>::T;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float x[H];
#pragma unroll
  for (int k = 0; k < H; ++k) x[k] = us[lane * H + k];
  Frag wrow[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
    wrow[j] = *reinterpret_cast<const Frag*>(a.wv + (int64_t(h) * 64 + wave * 16 + j) * a.ldw + lane * H);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float w[H];
    unpack_row<H>(wrow[j], w);
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < H; ++k) acc = fmaf(w[k], x[k], acc);
    acc = wave_sum(acc);
    if (lane == 0) a.o[int64_t(b) * a.ldo + h * 64 + wave * 16 + j] = to_bf(acc);
  }
}

}  // namespace

size_t rq_attn_ws_bytes(int B_r, int L, int H) {
  const size_t d = 64 * size_t(H);
  const size_t nch = (size_t(L) + RQ_CHUNK - 1) / RQ_CHUNK;
  const size_t qf = size_t(B_r) * H * d * 4;
  const size_t pu = size_t(B_r) * nch * H * d * 4;
  const size_t pm = size_t(B_r) * nch * H * 2 * 4;
  return ((qf + 255) / 256 + (pu + 255) / 256 + (pm + 255) / 256) * 256;
}

void rq_attn_carve(RqAttnArgs& a, void* ws) {
  const size_t d = 64 * size_t(a.H);
  const size_t nch = (size_t(a.L) + RQ_CHUNK - 1) / RQ_CHUNK;
  char* p = reinterpret_cast<char*>(ws);
  a.qf = reinterpret_cast<float*>(p);
  p += (size_t(a.B_r) * a.H * d * 4 + 255) / 256 * 256;
  a.part_u = reinterpret_cast<float*>(p);
  p += (size_t(a.B_r) * nch * a.H * d * 4 + 255) / 256 * 256;
  a.part_ml = reinterpret_cast<float*>(p);
}

// H heads of 64 (d <= 512 for rq_fold) and at most 1024 chunks of 64 events
// (the chunk weights of rq_combine live in LDS)
bool rq_attn_supported(int H, int L) {
  return (H == 1 || H == 2 || H == 4 || H == 8) && L > 0 && L <= 1024 * RQ_CHUNK;
}

hipError_t launch_rq_attn(const RqAttnArgs& a, hipStream_t s) {
  if (a.B_r <= 0) return hipSuccess;
  if (!rq_attn_supported(a.H, a.L)) return hipErrorInvalidValue;
  const int nch = (a.L + RQ_CHUNK - 1) / RQ_CHUNK;
  hipLaunchKernelGGL(rq_fold_kernel, dim3(a.B_r * a.H), dim3(256), 0, s, a);
  const dim3 g(unsigned(a.B_r * nch));
  switch (a.H) {
    case 8: hipLaunchKernelGGL(rq_attend_kernel<8>, g, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(rq_attend_kernel<4>, g, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(rq_attend_kernel<2>, g, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(rq_attend_kernel<1>, g, dim3(256), 0, s, a); break;
  }
  const dim3 gc(unsigned(a.B_r * a.H));
  switch (a.H) {
    case 8: hipLaunchKernelGGL(rq_combine_kernel<8>, gc, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(rq_combine_kernel<4>, gc, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(rq_combine_kernel<2>, gc, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(rq_combine_kernel<1>, gc, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace rocs
