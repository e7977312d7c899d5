// W8A16 linear layer ([U] "Compute Only Once: UG-Separation for Efficient
// Large Recommendation Models", xllm-io review, §3 stage 4 and the W8A16
// configuration): y = act(x (s . fp8(Wq))^T + b) with 8-bit E4M3 weight codes,
// one fp32 scale per output channel, bf16 activations and outputs.
//
// For the shapes this serves (1 to 64 activation rows) the weights are the
// bulk of the bytes, read once; the activations are small and re-read from
// L2 by every wave.  One workgroup owns 16 * CT output channels; its NW waves
// split K in 128-k blocks (one 128-byte line of each weight row per block).
//
// A wave computes CT x MT tiles of v_mfma_f32_16x16x32_bf16: channel tile c
// (16 weight rows, operand A) times row tile t (16 activation rows, operand
// B).  Lane l = 16 g + r streams 32 contiguous code bytes of weight row r of
// each channel tile per block and 64 bytes of activation row r of each row
// tile; in k-step s (0..3) lane group g supplies the 8 k at 32 g + 8 s, for
// both operands.  The codes are decoded to bf16 with
// v_cvt_scalef32_pk_bf16_fp8 at scale 1 (exact: every E4M3 value is a bf16
// value).  Each wave requests its next block before the current one's
// products, so two blocks are in flight per wave.  The NW partial tiles are
// added in wave order through LDS; the scale, bias, ReLU and an optional
// residual follow.  A batch of GEMMs of one shape runs as one launch
// (grid.y).
//
// Shape rule (measured: the activation loads, one fragment per wave and
// block, are what grows with M; more channels per wave re-read them less but
// leave fewer workgroups): MT = ceil(M / 16); 16 channels and 8 waves per
// workgroup while the launch has at most 320 tiles of 16 channels, else 32
// channels and 4 waves.
#include "rocs_device.h"

namespace rocs {

namespace {

constexpr int W8_KB = 128;  // K per block

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r;
  r[0] = a[0];
  r[1] = a[1];
  r[2] = b[0];
  r[3] = b[1];
  r[4] = c[0];
  r[5] = c[1];
  r[6] = d[0];
  r[7] = d[1];
  return r;
}

// Arguments of GEMM blockIdx.y of a batch.
__device__ __forceinline__ W8Args batch_member(const W8Args& a0) {
  W8Args a = a0;
  if (blockIdx.y > 0) {
    const int64_t i = blockIdx.y;
    a.x += i * a.sx;
    a.wq += i * a.sw;
    a.scale += i * a.sscale;
    if (a.bias) a.bias += i * a.sbias;
    if (a.res) a.res += i * a.sres;
    a.y += i * a.sy;
  }
  return a;
}

// Operands of one block for one lane: 32 code bytes of each channel tile's
// weight row, 64 bytes of each row tile's activation row.
template <int CT, int MT>
struct W8Block {
  uint4 w[CT][2];
  bf16x8 x[MT][4];
};

template <int CT, int MT>
__device__ __forceinline__ void w8_load(W8Block<CT, MT>& b, const uint8_t* w0, int64_t ldw, const bf16* x0,
                                        int64_t ldx, unsigned xvalid, int kb) {
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const uint4* p = reinterpret_cast<const uint4*>(w0 + int64_t(c) * 16 * ldw + int64_t(kb) * W8_KB);
    b.w[c][0] = p[0];
    b.w[c][1] = p[1];
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    // lanes past the last activation row load nothing (their operand is zero)
    if (xvalid & (1u << t)) {
      const uint4* p = reinterpret_cast<const uint4*>(x0 + int64_t(t) * 16 * ldx + kb * W8_KB);
#pragma unroll
      for (int s = 0; s < 4; ++s) b.x[t][s] = __builtin_bit_cast(bf16x8, p[s]);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) b.x[t][s] = bf16x8{};
    }
  }
}

template <int CT, int MT>
__device__ __forceinline__ void w8_mfma(const W8Block<CT, MT>& b, f32x4 (&acc)[CT][MT]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const uint4 q = b.w[c][s >> 1];
      const bf16x8 af = (s & 1) ? e4m3x8_to_bf16(q.z, q.w) : e4m3x8_to_bf16(q.x, q.y);
#pragma unroll
      for (int t = 0; t < MT; ++t)
        acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b.x[t][s], acc[c][t], 0, 0, 0);
    }
  }
}

template <int CT, int MT, int NW>
__global__ __launch_bounds__(NW * 64) void w8a16_kernel(W8Args a0) {
  constexpr int TILE = CT * MT * 4 * 64;  // accumulator floats of one wave
  __shared__ float part[NW * TILE];
  const W8Args a = batch_member(a0);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 16 * CT;
  const int r = lane & 15, g = lane >> 4;
  const int nkb = a.K / W8_KB;
  const int kb_lo = wave * nkb / NW, kb_hi = (wave + 1) * nkb / NW;
  const uint8_t* w0 = a.wq + int64_t(n0 + r) * a.ldw + g * 32;
  const bf16* x0 = a.x + int64_t(r) * a.ldx + g * 32;
  unsigned xvalid = 0;
#pragma unroll
  for (int t = 0; t < MT; ++t) xvalid |= (16 * t + r < a.M ? 1u : 0u) << t;
  f32x4 acc[CT][MT];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // one block ahead, in two named buffers used in alternation (no register
  // copies between blocks)
  W8Block<CT, MT> b0, b1;
  int kb = kb_lo;
  if (kb < kb_hi) w8_load<CT, MT>(b0, w0, a.ldw, x0, a.ldx, xvalid, kb);
  while (kb < kb_hi) {
    if (kb + 1 < kb_hi) w8_load<CT, MT>(b1, w0, a.ldw, x0, a.ldx, xvalid, kb + 1);
    w8_mfma<CT, MT>(b0, acc);
    if (++kb >= kb_hi) break;
    if (kb + 1 < kb_hi) w8_load<CT, MT>(b0, w0, a.ldw, x0, a.ldx, xvalid, kb + 1);
    w8_mfma<CT, MT>(b1, acc);
    ++kb;
  }
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) part[wave * TILE + ((c * MT + t) * 4 + j) * 64 + lane] = acc[c][t][j];
  __syncthreads();
  for (int idx = threadIdx.x; idx < TILE; idx += NW * 64) {
    float v = part[idx];
#pragma unroll
    for (int wv = 1; wv < NW; ++wv) v += part[wv * TILE + idx];
    // accumulator register j of lane l in tile (c, t): weight row 16 c + 4 (l / 16) + j,
    // activation row 16 t + l % 16
    const int l = idx & 63, j = (idx >> 6) & 3, t = (idx >> 8) % MT, c = (idx >> 8) / MT;
    const int m = 16 * t + (l & 15), n = n0 + 16 * c + 4 * (l >> 4) + j;
    if (m < a.M) {
      v *= a.scale[n];
      if (a.bias) v += to_f(a.bias[n]);
      if (a.act == 1) v = fmaxf(v, 0.f);
      if (a.res) v += to_f(a.res[int64_t(m) * a.ldres + n]);
      a.y[int64_t(m) * a.ldy + n] = to_bf(v);
    }
  }
}

template <int CT, int NW>
hipError_t launch_ct(const W8Args& a, int mt, hipStream_t s) {
  const dim3 grid(a.N / (16 * CT), a.batch > 1 ? a.batch : 1), block(NW * 64);
  switch (mt) {
    case 1:
      hipLaunchKernelGGL((w8a16_kernel<CT, 1, NW>), grid, block, 0, s, a);
      break;
    case 2:
      hipLaunchKernelGGL((w8a16_kernel<CT, 2, NW>), grid, block, 0, s, a);
      break;
    case 3:
      hipLaunchKernelGGL((w8a16_kernel<CT, 3, NW>), grid, block, 0, s, a);
      break;
    default:
      hipLaunchKernelGGL((w8a16_kernel<CT, 4, NW>), grid, block, 0, s, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace

bool w8a16_supported(int M, int N, int K) {
  return M >= 1 && M <= 64 && N >= 1 && N % 16 == 0 && K >= W8_KB && K % W8_KB == 0;
}

hipError_t launch_w8a16(const W8Args& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (!w8a16_supported(a.M, a.N, a.K)) return hipErrorInvalidValue;
  const int mt = (a.M + 15) / 16;
  const long tiles = long(a.N / 16) * (a.batch > 1 ? a.batch : 1);
  if (tiles <= 320 || a.N % 32 != 0) return launch_ct<1, 8>(a, mt, s);
  return launch_ct<2, 4>(a, mt, s);
}

}  // namespace rocs
