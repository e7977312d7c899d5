// GLM linear GEMMs with the in-kernel broadcast epilogue.
//
// [R] §2.4 (IKBO for LCB): the candidate GEMM W_CC X_C[i] resolves m_i in its
// epilogue, loads the request contribution Z[m_i] and adds it in registers,
// writing only the final value; no broadcast tensor or GEMM intermediate
// reaches HBM.  The request half ([Y_R | Z] = X_R [W_RR; W_CR]^T) is the same
// kernel with a split output.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  The weight
// fragment is the MFMA "A" operand and the activation fragment the "B"
// operand, so each lane holds 4 consecutive output columns of one output row
// per register group.  Every bf16 shape runs gemm_bf16_big_kernel: operands
// move global->LDS by DMA (global_load_lds_dwordx4), with no register
// staging and a zero page for K tails; only the tile shape changes between
// request batches and candidate batches.  The accumulation order is fixed
// (64-wide K groups in ascending order, four k16 steps per group with the
// k-sets of kchunk in rocs_mfma.h), so every output element is reduced in the
// same order whichever tile shape computes it: results are bit-identical
// across batch sizes and batch compositions.
// Workgroup ids are remapped so that one XCD walks neighbouring tiles.
#include "rocs_gemm_tile.inc"

namespace rocs {

namespace {

// One tile per workgroup, tiles in XCD-aware order.  A batch of GEMMs is
// one flat grid of (GEMM, tile) pairs, remapped as a whole, so each XCD
// runs a contiguous range of one GEMM's tiles (its weights stay in that
// XCD's L2).
template <int BM, int BN, int WM, int WN, int NS = 2>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_bf16_big_kernel(GemmArgs a0) {
  __shared__ uint4 smem[NS * (BM + BN) * 8];
  const int ntn = (a0.N + BN - 1) / BN;
  const int ntm = (a0.M + BM - 1) / BM;
  const int tiles = ntm * ntn;
  const int logical = xcd_remap(blockIdx.x, tiles * (a0.batch > 1 ? a0.batch : 1));
  // the division runs on the vector unit; the member's pointers must stay scalar
  const int member = __builtin_amdgcn_readfirstlane(logical / tiles);
  const int t = logical - member * tiles;
  const GemmArgs a = batch_slice(a0, member);
  gemm_tile<BM, BN, WM, WN, NS>(a, (t / ntn) * BM, (t % ntn) * BN, smem);
}

// Two tile heights in one launch: rows [0, M1) in 256-row tiles (whole
// rounds of one workgroup per CU), then rows [M1, M) in H2-row tiles that
// fill one more round.  Workgroups are dispatched in order, so the short
// tiles run last and the final round is not left half empty.
template <int BN, int H2>
__global__ __launch_bounds__(512, 1) void gemm_bf16_mixed_kernel(GemmArgs a, int M1) {
  __shared__ uint4 smem[2 * (256 + BN) * 8];
  const int ntn = (a.N + BN - 1) / BN;
  const int n1 = (M1 / 256) * ntn;
  const int b = blockIdx.x;
  if (b < n1) {
    const int logical = xcd_remap(b, n1);
    gemm_tile<256, BN, 2, 4, 2>(a, (logical / ntn) * 256, (logical % ntn) * BN, smem);
  } else {
    const int logical = xcd_remap(b - n1, gridDim.x - n1);
    gemm_tile<H2, BN, 2, 4, 2>(a, M1 + (logical / ntn) * H2, (logical % ntn) * BN, smem);
  }
}

// Launches of fewer than 2,048 rows with a long K (K >= 1024; few output
// tiles, each a long chain of slabs), and request-side launches with fewer
// 32 x 32 tiles than CUs: one 32 x 32 tile per workgroup of four waves, K
// split in quarters (splitk_tile).  The result is deterministic; it is summed
// in a different order than the single-chain kernels.  The choice depends on
// the launch's shape only (uses_splitk).
template <int NS>
__global__ __launch_bounds__(256, 1) void gemm_bf16_splitk_kernel(GemmArgs a0) {
  const GemmArgs a = batch_slice(a0, blockIdx.y);  // GEMM blockIdx.y of a batch
  constexpr int SLOT = (32 + 32) * 8;
  __shared__ uint4 smem[4 * NS * SLOT];
  const int ntn = (a.N + 31) / 32;
  const int ntm = (a.M + 31) / 32;
  const int logical = xcd_remap(blockIdx.x, ntm * ntn);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  splitk_tile<NS>(a, (logical / ntn) * 32, (logical % ntn) * 32, smem, wave, threadIdx.x & 63, true);
}

// fp32 path: LDS-tiled SIMT GEMM, 64 x 64 tile, each thread 4 x 4 outputs,
// K reduced sequentially (one fused multiply-add per k, ascending k).
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  constexpr int T = 64, KB = 16;
  __shared__ float sA[KB][T + 4];
  __shared__ float sW[KB][T + 4];
  const int ntn = (a.N + T - 1) / T;
  const int ntm = (a.M + T - 1) / T;
  const int logical = xcd_remap(blockIdx.x, ntm * ntn);
  const int m0 = (logical / ntn) * T, n0 = (logical % ntn) * T;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const float* A = reinterpret_cast<const float*>(a.A);
  float acc[4][4] = {};
  for (int k0 = 0; k0 < a.K; k0 += KB) {
    for (int e = tid; e < T * KB; e += 256) {
      const int r = e / KB, kk = e % KB, k = k0 + kk;
      const int row = m0 + r, col = n0 + r;
      sA[kk][r] = (row < a.M && k < a.K) ? A[int64_t(row) * a.lda + k] : 0.0f;
      float wv = 0.0f;
      if (col < a.N && k < a.K) {
        int s = 0, base = 0;
        while (s + 1 < a.nseg && col >= a.seg_end[s]) base = a.seg_end[s++];
        wv = reinterpret_cast<const float*>(a.W[s])[int64_t(col - base) * a.ldw + k];
      }
      sW[kk][r] = wv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      float xa[4], wb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) wb[j] = sW[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xa[i], wb[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) epilogue4<float>(a, m0 + ty * 4 + i, n0 + tx * 4, acc[i]);
}

template <typename K>
hipError_t launch_tiles(K kernel, int bm, int bn, int threads, const GemmArgs& a, hipStream_t s) {
  const int nwg = ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn);
  hipLaunchKernelGGL(kernel, dim3(nwg, a.batch > 1 ? a.batch : 1), dim3(threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[16] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cus[dev];
}

// Launch plan for a candidate GEMM (one workgroup per CU, BN = 256): either
// one tile height for all rows, or 256-row tiles for whole rounds followed
// by one round of shorter tiles (gemm_bf16_mixed_kernel).  Cost model, in
// units of a 256-row tile's time, fitted to interleaved timings on the
// candidate shapes: a tile of h rows costs 0.52 + 0.48 h / 256 (the fixed
// part is the tile's start, operand traffic and epilogue), and a round of
// concurrent tiles costs its tile's time.  Measured: N = 1024 (4 column
// tiles) takes 256-row tiles for 4 rounds and a round of 128-row tiles
// (116 vs 121 us for 256 rows throughout); N = 512 takes 192-row tiles
// (109 vs 111 us mixed, 125 us with 256 rows).
CandPlan cand_plan(int M, int ntn) {
  const int cus = device_cus();
  const auto tile_cost = [](int h) { return 0.52 + 0.48 * h / 256.0; };
  CandPlan best{256, 0, 0, 0};
  double best_cost = 1e30;
  for (int h : {256, 192, 128}) {
    const long tiles = long((M + h - 1) / h) * ntn;
    const double cost = double((tiles + cus - 1) / cus) * tile_cost(h);
    if (cost < best_cost - 1e-9) {
      best = CandPlan{h, 0, 0, 0};
      best_cost = cost;
    }
  }
  const int per_round = (cus / ntn) * 256;
  if (per_round > 0 && M > per_round && M % per_round != 0) {
    const int M1 = (M / per_round) * per_round, rest = M - M1, slots = cus / ntn;
    for (int h2 : {64, 128, 192}) {
      if ((rest + h2 - 1) / h2 > slots) continue;
      const double cost = double(M1 / per_round) + tile_cost(h2);
      if (cost < best_cost - 1e-9) {
        best = CandPlan{0, M1, h2, (M1 / 256) * ntn + ((rest + h2 - 1) / h2) * ntn};
        best_cost = cost;
      }
      break;  // the smallest height that fits one round is the cheapest
    }
  }
  return best;
}

template <int BN>
hipError_t launch_mixed(const GemmArgs& a, int M1, int h2, int grid, hipStream_t s) {
  switch (h2) {
    case 64: hipLaunchKernelGGL((gemm_bf16_mixed_kernel<BN, 64>), dim3(grid), dim3(512), 0, s, a, M1); break;
    case 128: hipLaunchKernelGGL((gemm_bf16_mixed_kernel<BN, 128>), dim3(grid), dim3(512), 0, s, a, M1); break;
    case 192: hipLaunchKernelGGL((gemm_bf16_mixed_kernel<BN, 192>), dim3(grid), dim3(512), 0, s, a, M1); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Epilogue variant of a launch: one of the specialised ones when the terms
// match (at most one of ReLU and a residual) and every offset fits 32 bits,
// else EPI_ANY.
int epilogue_variant(const GemmArgs& a) {
  if (a.out0_f32 || a.act > 1 || (a.act == 1 && a.res != nullptr)) return EPI_ANY;
  const int64_t lim = int64_t(1) << 31;
  if (int64_t(a.M) * a.ld0 >= lim) return EPI_ANY;
  if (a.res != nullptr && int64_t(a.M) * a.ldres >= lim) return EPI_ANY;
  const int tail = (a.bias ? EPI_BIAS : 0) | (a.act == 1 ? EPI_RELU : 0) | (a.res ? EPI_RES : 0);
  if (a.z == nullptr) return EPI_SPEC | tail;
  if (int64_t(a.zrows) * a.ldz >= lim) return EPI_ANY;
  // Z goes into the accumulators at tile start when no tile takes the edge
  // path (which adds Z itself): N a multiple of every tile width, one output.
  // Mapped and unmapped Z (the dense-broadcast comparator's copied rows) then
  // sum in the same order.
  const bool zacc = a.N % 256 == 0 && a.n_split >= a.N;
  if (a.zmap == nullptr && !zacc) return EPI_ANY;
  return EPI_Z | tail | (zacc ? EPI_ZACC : 0);
}

// bf16 launches below the candidate-size threshold that take the split-K
// kernel (its partial sums start at zero; Z is added last).  Short chains
// split only for request-side launches (no Z input), so candidate rows keep
// the single-chain K order.
bool uses_splitk(const GemmArgs& a) {
  if (a.M >= 2048) return false;
  const long tiles32 = long((a.M + 31) / 32) * ((a.N + 31) / 32);
  return a.K >= 1024 || (a.z == nullptr && a.K >= 256 && tiles32 < device_cus());
}

bool gemm_z_in_accumulators(const GemmArgs& a) { return !uses_splitk(a) && (epilogue_variant(a) & EPI_ZACC) != 0; }

hipError_t launch_gemm(DType dt, const GemmArgs& args, hipStream_t s) {
  GemmArgs a = args;
  a.epi = epilogue_variant(a);
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  // A batch runs as one launch (grid.y = GEMM) on the split-K kernel, whose
  // few tiles per GEMM leave most of the chip idle; any other kernel choice
  // runs the GEMMs one launch each.
  const bool big_batch = dt == BF16 && a.M >= 2048 && a.N > 128;
  if (a.batch > 1 && !(dt == BF16 && uses_splitk(a)) && !big_batch) {
    for (int i = 0; i < a.batch; ++i) {
      GemmArgs b = batch_slice(args, i);
      b.batch = 1;
      const hipError_t e = launch_gemm(dt, b, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (dt == F32) return launch_tiles(gemm_f32_kernel, 64, 64, 256, a, s);
  // All bf16 variants compute every element identically; the choice only
  // trades tile size against the number of workgroups.  Measured on the
  // candidate shapes (M = 73,704; K, N = 512/1024 both ways, interleaved
  // medians): 256-wide tiles beat 128x128 ones (139 vs 164 us for N =
  // 1024): half the operand traffic from L2 per FLOP.  One workgroup fits
  // per CU, so the tile heights are chosen to fill the rounds (cand_plan).
  if (a.M >= 2048) {
    if (a.N > 128 && a.batch > 1) {  // one flat grid of every GEMM's 256 x 256 tiles
      const long nwg = long((a.M + 255) / 256) * ((a.N + 255) / 256) * a.batch;
      hipLaunchKernelGGL((gemm_bf16_big_kernel<256, 256, 2, 4>), dim3(nwg), dim3(512), 0, s, a);
      return hipGetLastError();
    }
    if (a.N > 128) {
      const CandPlan p = cand_plan(a.M, (a.N + 255) / 256);
      switch (p.h) {
        case 0: return launch_mixed<256>(a, p.M1, p.h2, p.grid, s);
        case 192: return launch_tiles(gemm_bf16_big_kernel<192, 256, 2, 4>, 192, 256, 512, a, s);
        case 128: return launch_tiles(gemm_bf16_big_kernel<128, 256, 2, 4>, 128, 256, 512, a, s);
        default: return launch_tiles(gemm_bf16_big_kernel<256, 256, 2, 4>, 256, 256, 512, a, s);
      }
    }
    return launch_tiles(gemm_bf16_big_kernel<256, 128, 4, 2>, 256, 128, 512, a, s);
  }
  // Request batches (M <= a few hundred): the weights stream from HBM once
  // and K/64 slabs run in sequence, so the time is slab latency.  One-wave
  // 32x32 tiles put enough workgroups on the chip (B_r = 256, N = 1024:
  // 256 of them), each with seven slabs (56 KB) in flight.  Longer chains
  // split K over four waves per tile (measured, M = 128, N = 2048, K = 8960:
  // 62 -> 25 us; M = 256, N = 1024, K = 1024: 8.3 -> 5.2 us; at K = 512 the
  // single chain is faster, 6.1 vs 7.6 us), and so do short chains when there
  // are fewer tiles than CUs (M = 32, N = 4096, K = 512: 5.8 -> 4.6 us; M =
  // 64, N = 512, K = 256: 4.9 -> 4.1 us).
  if (uses_splitk(a)) return launch_tiles(gemm_bf16_splitk_kernel<4>, 32, 32, 256, a, s);
  return launch_tiles(gemm_bf16_big_kernel<32, 32, 1, 1, 8>, 32, 32, 64, a, s);
}

}  // namespace rocs
