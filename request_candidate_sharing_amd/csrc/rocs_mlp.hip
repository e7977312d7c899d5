// Fused candidate-side GLM MLP block:
//   h = act1(x W1^T + Z1[m_i] + b1)          (GLM linear, [R] §2.4 epilogue)
//   o = act2(h W2^T + Z2[m_i] + b2) (+ x)     (GLM linear, residual)
//   y = group_norm(o)                          ([R] §2.1, Figure 2(b))
// for the candidate batch, with the request contributions Z1 = x_R W1_CR^T
// and Z2 = h_R W2_CR^T computed once per request beforehand.  The hidden
// activation never reaches HBM: per 128-row tile it is produced in 128-wide
// chunks into LDS and consumed at once by the second GEMM, whose
// accumulators (128 x d_out fp32, up to 256 registers per lane) stay in the
// accumulation registers across all chunks.  Per tile HBM sees x once and y
// once; the weights and the later x slabs come from L2.
//
// 4 waves, one per SIMD, 512 registers each.  Operands move global -> LDS by
// DMA (global_load_lds_dwordx4) through a two-slot ring of 64 KB slabs shared
// by both GEMMs, so the next slab is always in flight, across phase changes
// too:
//   A slab  x [128 x 128] | W1 chunk rows [128 x 128]   (K = 128 of d_in)
//   B slab  W2 rows [64*FNB x 64]                        (K = 64 of the chunk)
// Waves sit 2 (rows) x 2 (cols): in the first GEMM each owns 64 x 64 of the
// chunk, in the second 64 rows x 32*FNB output columns; the hidden chunk
// [128 x 128] bf16 (32 KB, its own LDS) is the second GEMM's B operand.  The
// K order of every MFMA is the library's (rocs_mfma.h), so with no norm fused
// the result is bit-identical to the two unfused GEMMs.  Norm statistics are
// fp32 with a fixed reduction order.
#include "rocs_mfma.h"

namespace rocs {

namespace {

constexpr int BM = 128;       // rows per tile
constexpr int HC = 128;       // hidden chunk
constexpr int NT = 256;       // threads per workgroup
constexpr int SLAB_U4 = 4096; // 64 KB slab in uint4

template <int FNB, bool Z2F>
__global__ __launch_bounds__(NT, 1) void mlp_block_kernel(MlpArgs a) {
  __shared__ uint4 ring[2][SLAB_U4];  // 128 KB
  __shared__ uint4 hs[BM * HC / 8];   // 32 KB: hidden chunk, 16 chunks per row

  constexpr int DOUT_PAD = 2 * FNB * 32;  // W2 rows covered by the two column waves
  static_assert(DOUT_PAD * 8 <= SLAB_U4, "W2 slab must fit one ring slot");
  const int ntiles = (a.M + BM - 1) / BM;
  const int tile = xcd_remap(blockIdx.x, ntiles);
  const int m0 = tile * BM;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: branches on it stay scalar
  const int hk = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  const int nA = a.d_in / 128;
  const int nchunks = (a.hidden + HC - 1) / HC;

  // ---- DMA of one slab into ring slot st
  // The lane index is made opaque at each issue so that the compiler
  // recomputes the slab addresses (a few ALU ops) instead of keeping 16
  // 64-bit addresses per slab kind live across the loops.
  auto issue_a = [&](int c, int k, int st) {
    uint4* dst = ring[st];
    int ln = lane;
    asm volatile("" : "+v"(ln));
    // 256 rows of 256 B: rows 0..127 x, 128..255 W1; 4 rows per wave-instruction
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int blk = wave * 16 + q;
      const int r = blk * 4 + (ln >> 4);
      const int ch = (ln & 15) ^ swz<16>(r);
      const bf16* src;
      if (r < BM)
        src = a.x + int64_t(min(m0 + r, a.M - 1)) * a.ldx + k * 128 + ch * 8;
      else
        src = a.w1 + int64_t(min(c * HC + r - BM, a.hidden - 1)) * a.d_in + k * 128 + ch * 8;
      dma16(src, dst + blk * 64);
    }
  };
  auto issue_b = [&](int c, int k, int st) {
    uint4* dst = ring[st];
    int ln = lane;
    asm volatile("" : "+v"(ln));
    // DOUT_PAD rows of 128 B; 8 rows per wave-instruction
#pragma unroll
    for (int q = 0; q < 2 * FNB; ++q) {
      const int blk = wave * 2 * FNB + q;
      const int r = blk * 8 + (ln >> 3);
      const int ch = (ln & 7) ^ swz<8>(r);
      const bf16* src = a.w2 + int64_t(min(r, a.d_out - 1)) * a.hidden + c * HC + k * 64 + ch * 8;
      dma16(src, dst + blk * 64);
    }
  };

  // request row of each of this lane's tile rows (wm*64 + 32i + l32)
  int zr[2];
  bool bad[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = min(m0 + wm * 64 + i * 32 + l32, a.M - 1);
    const int q = a.zmap ? a.zmap[m] : m;
    bad[i] = (unsigned)q >= (unsigned)a.zrows;
    zr[i] = bad[i] ? 0 : q;
  }

  f32x16 oacc[2][FNB];
  if constexpr (Z2F) {
    // the second GEMM accumulates onto Z2 (blocks past d_out start at 0)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < FNB; ++j) {
        const int cb = (wn * FNB + j) * 32;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 zz = cb < a.d_out
                                ? *reinterpret_cast<const float4*>(a.z2 + int64_t(zr[i]) * a.ldz2 + cb + 8 * g + 4 * hk)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
          oacc[i][j][4 * g + 0] = zz.x;
          oacc[i][j][4 * g + 1] = zz.y;
          oacc[i][j][4 * g + 2] = zz.z;
          oacc[i][j][4 * g + 3] = zz.w;
        }
      }
  } else {
    zero_acc(oacc);
  }

  int st = 0;
  issue_a(0, 0, 0);
  wait_dma();
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int hw = min(HC, a.hidden - c * HC);
    const int nB = hw / 64;
    // Z1 entries of this chunk, fetched while the first GEMM runs
    float4 z1v[2][2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = wn * 64 + j * 32 + 8 * g + 4 * hk;
          z1v[i][j][g] = col < hw ? *reinterpret_cast<const float4*>(a.z1 + int64_t(zr[i]) * a.ldz1 + c * HC + col)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
        }

    // first GEMM: hacc = x W1_chunk^T (onto Z1 when z1_first)
    f32x16 hacc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 zi = a.z1_first ? z1v[i][j][g] : make_float4(0.f, 0.f, 0.f, 0.f);
          hacc[i][j][4 * g + 0] = zi.x;
          hacc[i][j][4 * g + 1] = zi.y;
          hacc[i][j][4 * g + 2] = zi.z;
          hacc[i][j][4 * g + 3] = zi.w;
        }
    for (int k = 0; k < nA; ++k) {
      if (k + 1 < nA)
        issue_a(c, k + 1, st ^ 1);
      else
        issue_b(c, 0, st ^ 1);
      const uint4* s = ring[st];
      mfma_steps<2, 2, 8, 16, 16>(s, BM + wn * 64 + l32, s, wm * 64 + l32, 0, hk, hacc);
      wait_dma();
      __syncthreads();
      st ^= 1;
    }
    // hidden chunk epilogue: + Z1 + b1, act1, round to bf16 into hs
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wm * 64 + i * 32 + l32;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = wn * 64 + j * 32 + 8 * g + 4 * hk;
          float v[4] = {hacc[i][j][4 * g], hacc[i][j][4 * g + 1], hacc[i][j][4 * g + 2], hacc[i][j][4 * g + 3]};
          if (!a.z1_first) {
            v[0] += z1v[i][j][g].x;
            v[1] += z1v[i][j][g].y;
            v[2] += z1v[i][j][g].z;
            v[3] += z1v[i][j][g].w;
          }
          if (col < hw) {
            if (a.b1) {
              const bf16x4 bb = *reinterpret_cast<const bf16x4*>(a.b1 + c * HC + col);
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] += to_f(bb[e]);
            }
            if (a.act1 == 1)
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = fmaxf(v[e], 0.f);
            if (bad[i])
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = nan_f();
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = 0.f;
          }
          const bf16x4 pk = {to_bf(v[0]), to_bf(v[1]), to_bf(v[2]), to_bf(v[3])};
          reinterpret_cast<uint2*>(&hs[slot<16>(r, col >> 3)])[hk] = __builtin_bit_cast(uint2, pk);
        }
    }
    __syncthreads();
    // second GEMM: oacc += h_chunk W2_chunk^T
    for (int k = 0; k < nB; ++k) {
      if (k + 1 < nB)
        issue_b(c, k + 1, st ^ 1);
      else if (c + 1 < nchunks)
        issue_a(c + 1, 0, st ^ 1);
      const uint4* s = ring[st];
      mfma_steps<2, FNB, 4, 8, 16>(s, wn * FNB * 32 + l32, hs, wm * 64 + l32, k * 8, hk, oacc);
      wait_dma();
      __syncthreads();
      st ^= 1;
    }
  }

  // ---- epilogue: + Z2 + b2, act2, + residual, group norm, store.
  // The ring is free now.  Tile rows there keep their 16-byte chunks
  // XOR-swizzled inside aligned groups of up to 16 chunks, so that reads of
  // 32 rows of one column spread over the LDS banks.
  uint4* stage = &ring[0][0];
  const int ocpr = a.d_out / 8;  // 16-byte chunks per row (a multiple of 4)
  const int smask = (ocpr % 16 == 0) ? 15 : (ocpr % 8 == 0) ? 7 : 3;
  auto spos = [&](int r, int ch) { return r * ocpr + (ch ^ (r & smask)); };
  if (a.residual) {  // the residual is the block input x (d_in == d_out)
    for (int e = tid; e < BM * ocpr; e += NT) {
      const int r = e / ocpr, ch = e - r * ocpr;
      const int row = min(m0 + r, a.M - 1);
      stage[spos(r, ch)] = *reinterpret_cast<const uint4*>(a.x + int64_t(row) * a.ldx + ch * 8);
    }
    __syncthreads();
  }
  float s1[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = wm * 64 + i * 32 + l32;
#pragma unroll
    for (int j = 0; j < FNB; ++j) {
      // blocks past d_out (d_out not a multiple of 64*FNB) compute on column
      // 0..31 and are left out of the statistics and the store
      const int cb = (wn * FNB + j) * 32;
      const bool valid = cb < a.d_out;
      const float keep = valid ? 1.f : 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = (valid ? cb : 0) + 8 * g + 4 * hk;
        float v[4] = {oacc[i][j][4 * g], oacc[i][j][4 * g + 1], oacc[i][j][4 * g + 2], oacc[i][j][4 * g + 3]};
        if constexpr (!Z2F) {
          const float4 zz = *reinterpret_cast<const float4*>(a.z2 + int64_t(zr[i]) * a.ldz2 + col);
          v[0] += zz.x;
          v[1] += zz.y;
          v[2] += zz.z;
          v[3] += zz.w;
        }
        if (a.b2) {
          const bf16x4 bb = *reinterpret_cast<const bf16x4*>(a.b2 + col);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += to_f(bb[e]);
        }
        if (a.act2 == 1)
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = fmaxf(v[e], 0.f);
        if (a.residual) {
          const bf16x4 rv = reinterpret_cast<const bf16x4*>(&stage[spos(r, col >> 3)])[hk];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += to_f(rv[e]);
        }
        if (bad[i])
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = nan_f();
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          oacc[i][j][4 * g + e] = v[e];
          s1[i] += keep * ((a.norm == 1) ? v[e] * v[e] : v[e]);
        }
      }
      // keep the loads of one 32-column block from being hoisted above the
      // previous block (they would need 256 more registers)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // Row statistics: lane halves (l, l^32), then the two column waves in order.
  float(*red)[BM] = reinterpret_cast<float(*)[BM]>(&hs[0]);
  const float inv_d = 1.0f / float(a.d_out);
  float mean[2] = {0.f, 0.f}, scale[2] = {1.f, 1.f};
  if (a.norm >= 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) s1[i] += __shfl_xor(s1[i], 32, 64);
    if (hk == 0) {
      red[wn][wm * 64 + l32] = s1[0];
      red[wn][wm * 64 + 32 + l32] = s1[1];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wm * 64 + i * 32 + l32;
      const float t = red[0][r] + red[1][r];
      if (a.norm == 1)
        scale[i] = 1.0f / sqrtf(t * inv_d + a.eps);
      else
        mean[i] = t * inv_d;
    }
    if (a.norm == 0) {
      float s2[2] = {0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < FNB; ++j) {
          const float keep = (wn * FNB + j) * 32 < a.d_out ? 1.f : 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float dlt = oacc[i][j][e] - mean[i];
            s2[i] += keep * (dlt * dlt);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
      for (int i = 0; i < 2; ++i) s2[i] += __shfl_xor(s2[i], 32, 64);
      __syncthreads();
      if (hk == 0) {
        red[wn][wm * 64 + l32] = s2[0];
        red[wn][wm * 64 + 32 + l32] = s2[1];
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + l32;
        scale[i] = 1.0f / sqrtf((red[0][r] + red[1][r]) * inv_d + a.eps);
      }
    }
  }
  __syncthreads();  // residual reads done: the stage takes the output
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = wm * 64 + i * 32 + l32;
#pragma unroll
    for (int j = 0; j < FNB; ++j) {
      const int cb = (wn * FNB + j) * 32;
      const bool valid = cb < a.d_out;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = (valid ? cb : 0) + 8 * g + 4 * hk;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = oacc[i][j][4 * g + e];
        if (a.norm >= 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (v[e] - mean[i]) * scale[i];
          if (a.gamma) {
            const bf16x4 gg = *reinterpret_cast<const bf16x4*>(a.gamma + col);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] *= to_f(gg[e]);
          }
          if (a.beta) {
            const bf16x4 bb = *reinterpret_cast<const bf16x4*>(a.beta + col);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += to_f(bb[e]);
          }
        }
        const bf16x4 pk = {to_bf(v[0]), to_bf(v[1]), to_bf(v[2]), to_bf(v[3])};
        if (valid) reinterpret_cast<bf16x4*>(&stage[spos(r, col >> 3)])[hk] = pk;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();
  for (int e = tid; e < BM * ocpr; e += NT) {
    const int r = e / ocpr, ch = e - r * ocpr;
    if (m0 + r < a.M) *reinterpret_cast<uint4*>(a.y + int64_t(m0 + r) * a.ldy + ch * 8) = stage[spos(r, ch)];
  }
}

}  // namespace

bool mlp_block_supported(int d_in, int hidden, int d_out) {
  return d_in >= 128 && d_in % 128 == 0 && hidden >= 64 && hidden % 64 == 0 && d_out >= 32 && d_out <= 512 &&
         d_out % 32 == 0;
}

hipError_t launch_mlp_block(const MlpArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (!mlp_block_supported(a.d_in, a.hidden, a.d_out) || (a.residual && a.d_in != a.d_out))
    return hipErrorInvalidValue;
  const int ntiles = (a.M + BM - 1) / BM;
  // Z2 summed first or last is fixed per launch: a template parameter keeps
  // the unused path out of the register allocation
  if (a.d_out <= 128) {
    if (a.z2_first)
      hipLaunchKernelGGL((mlp_block_kernel<2, true>), dim3(ntiles), dim3(NT), 0, s, a);
    else
      hipLaunchKernelGGL((mlp_block_kernel<2, false>), dim3(ntiles), dim3(NT), 0, s, a);
  } else if (a.d_out <= 256) {
    if (a.z2_first)
      hipLaunchKernelGGL((mlp_block_kernel<4, true>), dim3(ntiles), dim3(NT), 0, s, a);
    else
      hipLaunchKernelGGL((mlp_block_kernel<4, false>), dim3(ntiles), dim3(NT), 0, s, a);
  } else {
    // 256 accumulators per lane leave no registers to start them at Z2: Z2 is
    // added last here, so with d_out > 256 the fused block and the unfused
    // layers agree to rounding rather than bit for bit when the unfused GEMM
    // sums Z first
    hipLaunchKernelGGL((mlp_block_kernel<8, false>), dim3(ntiles), dim3(NT), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace rocs
