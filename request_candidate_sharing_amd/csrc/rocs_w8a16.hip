// W8A16 linear layer ([U] "Compute Only Once: UG-Separation for Efficient
// Large Recommendation Models", xllm-io review, §3 stage 4 and the W8A16
// configuration): y = act(x (s . fp8(Wq))^T + b) with 8-bit E4M3 weight codes,
// one fp32 scale per output channel, bf16 activations and outputs.
//
// For the weight-bound shapes this serves (a few to 64 activation rows), the
// time is the weight stream: one byte per weight instead of two.  One
// workgroup owns 32 output channels; its 8 waves split K in 128-byte blocks
// (one cache line of each weight row per block).  A lane streams 64
// contiguous code bytes of one weight row per block, decodes them to bf16
// with v_cvt_pk_f32_fp8 (exact: every E4M3 value is a bf16 value) and feeds
// v_mfma_f32_32x32x16_bf16 with the weights as operand A and the activation
// rows as operand B.  In k-step s of a block, lane half h supplies the 8
// consecutive k at 64h + 8s, for both operands.  The 8 partial tiles are
// added in wave order through LDS; the scale, bias and ReLU follow.
#include "rocs_device.h"

namespace rocs {

namespace {

constexpr int W8_KB = 128;  // K per block
constexpr int W8_NW = 8;    // waves per workgroup

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(int(lo), false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(int(lo), true);
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(int(hi), false);
  const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(int(hi), true);
  bf16x8 r;
  r[0] = to_bf(a[0]);
  r[1] = to_bf(a[1]);
  r[2] = to_bf(b[0]);
  r[3] = to_bf(b[1]);
  r[4] = to_bf(c[0]);
  r[5] = to_bf(c[1]);
  r[6] = to_bf(d[0]);
  r[7] = to_bf(d[1]);
  return r;
}

template <int MT>  // 32-row tiles of activation rows (M <= 32 MT)
__global__ __launch_bounds__(W8_NW * 64) void w8a16_kernel(W8Args a) {
  __shared__ float part[W8_NW * MT * 16 * 64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 32;
  const int r = lane & 31, h = lane >> 5;
  const int nkb = a.K / W8_KB;
  const int kb_lo = wave * nkb / W8_NW, kb_hi = (wave + 1) * nkb / W8_NW;
  const uint8_t* wrow = a.wq + int64_t(n0 + r) * a.ldw + h * 64;
  f32x16_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;
  for (int kb = kb_lo; kb < kb_hi; ++kb) {
    uint4 w[4];
    const uint4* wp = reinterpret_cast<const uint4*>(wrow + int64_t(kb) * W8_KB);
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = wp[q];
    bf16x8 xb[MT][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 32 + r;
      const uint4* xp = reinterpret_cast<const uint4*>(a.x + int64_t(min(m, a.M - 1)) * a.ldx + kb * W8_KB + h * 64);
      // lanes past the last activation row load nothing (their operand is zero)
      if (m < a.M) {
#pragma unroll
        for (int s = 0; s < 8; ++s) xb[mt][s] = __builtin_bit_cast(bf16x8, xp[s]);
      } else {
#pragma unroll
        for (int s = 0; s < 8; ++s) xb[mt][s] = bf16x8{};
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint4 q = w[s >> 1];
      const bf16x8 af = (s & 1) ? e4m3x8_to_bf16(q.z, q.w) : e4m3x8_to_bf16(q.x, q.y);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, xb[mt][s], acc[mt], 0, 0, 0);
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) part[((wave * MT + mt) * 16 + i) * 64 + lane] = acc[mt][i];
  __syncthreads();
  const float* scale = a.scale;
  for (int idx = threadIdx.x; idx < MT * 16 * 64; idx += W8_NW * 64) {
    const int l = idx & 63, i = (idx >> 6) & 15, mt = idx >> 10;
    float v = part[(mt * 16 + i) * 64 + l];
#pragma unroll
    for (int wv = 1; wv < W8_NW; ++wv) v += part[((wv * MT + mt) * 16 + i) * 64 + l];
    // accumulator register i of lane l: weight row (i / 4) * 8 + (l / 32) * 4 + i % 4, activation row l % 32
    const int n = n0 + (i >> 2) * 8 + (l >> 5) * 4 + (i & 3);
    const int m = mt * 32 + (l & 31);
    if (m < a.M) {
      v *= scale[n];
      if (a.bias) v += to_f(a.bias[n]);
      if (a.act == 1) v = fmaxf(v, 0.f);
      a.y[int64_t(m) * a.ldy + n] = to_bf(v);
    }
  }
}

}  // namespace

hipError_t launch_w8a16(const W8Args& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.M > 64 || a.N % 32 != 0 || a.K <= 0 || a.K % W8_KB != 0) return hipErrorInvalidValue;
  const dim3 grid(a.N / 32), block(W8_NW * 64);
  if (a.M <= 32)
    hipLaunchKernelGGL(w8a16_kernel<1>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(w8a16_kernel<2>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace rocs
