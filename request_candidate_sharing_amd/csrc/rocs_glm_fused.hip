// Both halves of one GLM linear in one launch.
//
// [R] §2.4 (IKBO for LCB, the mega-kernel step of the kernel ladder in
// §3.5 Table 4): the request tiles ([Y_R | Z] = X_R [W_RR; W_CR]^T) and the
// candidate tiles (Y_C = act(Z[m_i] + X_C W_CC^T + b_C) (+ res)) share one
// grid, and a candidate tile waits on completion counters of the request rows
// it reads instead of a kernel boundary.
//
// Order and progress.  The request tiles take the lowest workgroup ids.
// Workgroups are dispatched in id order, so a candidate tile that is running
// has every request tile already dispatched, and request tiles wait for
// nothing: every wait ends.  A wait is bounded all the same (kSpinLimit
// polls); one that gives up sets *err and the tile writes NaN.
//
// Counters.  One int per 32-row block of request rows counts the request
// tiles of that block that have stored their outputs (`target` of them
// cover the block).  A request tile publishes with an agent-scope release
// fence on every wave, a workgroup barrier, then one relaxed agent-scope
// atomic add per block; a candidate tile polls with relaxed agent-scope
// atomic loads, takes one agent-scope acquire fence and a workgroup barrier,
// so the Z rows it loads are the ones the request tiles wrote, whichever XCD
// (and L2) they ran on.
//
// Bits.  The request tiles follow the kernel the separate request launch
// would run: the one-chain K order of the DMA GEMMs (64 x 128 tiles here, the
// order does not depend on the tile shape) or the split-K order of four K
// quarters (32 x 32 tiles on four waves); the candidate tiles run the
// candidate launch's tile plan with its accumulators started at Z.  Every
// output is bit-identical to the two-launch path.
#include <cstdlib>

#include "rocs_gemm_tile.inc"

namespace rocs {

namespace {

constexpr int kSpinLimit = 1 << 18;  // polls of one counter before a wait gives up

struct FusedArgs {
  GemmArgs req, cand;
  int* flags;    // one counter per 32-row block of request rows, zero at launch
  int* err;      // set to 1 by a wait that gave up
  int req_kind;  // 0: 64 x 128 one-chain request tiles; 1: 32 x 32 split-K tiles on four waves
  int req_wg;    // workgroups of request tiles (ids 0 .. req_wg - 1)
  int target;    // request tiles that cover one 32-row block
  int rblocks;   // 32-row blocks of request rows
  int M1;        // mixed candidate plan: rows in 256-row tiles
  int polls;     // polls of one counter before a wait gives up
};

// The candidate tile's wait: the request rows it reads are those its map
// entries name (any candidate order); wave 0 reduces their range and lane 0
// polls the counters of the 32-row blocks in it.
struct ZRowsReady {
  const int32_t* zmap;
  int M, zrows;
  const int* flags;
  int target, polls;
  int* err;
  __device__ __forceinline__ bool operator()(int m0, int rows) const {
    __shared__ int ready_s;
    const int lane = threadIdx.x & 63;
    if ((threadIdx.x >> 6) == 0) {
      int lo = 0x7fffffff, hi = -1;
      for (int r = lane; r < rows; r += 64) {
        const int m = m0 + r;
        if (m < M) {
          const int z = zmap[m];
          if ((unsigned)z < (unsigned)zrows) {
            lo = min(lo, z);
            hi = max(hi, z);
          }
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        lo = min(lo, __shfl_xor(lo, o, 64));
        hi = max(hi, __shfl_xor(hi, o, 64));
      }
      if (lane == 0) {
        bool gave_up = false;
        for (int rb = lo >> 5; rb <= (hi >> 5) && !gave_up; ++rb) {  // none when hi < 0
          int n_polls = 0;
          while (__hip_atomic_load(flags + rb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (++n_polls > polls) {
              __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              gave_up = true;
              break;
            }
            __builtin_amdgcn_s_sleep(2);
          }
        }
        ready_s = gave_up ? 0 : 1;
      }
      // One acquire per workgroup: it invalidates this CU's L1 and the stale
      // lines of the XCD's L2, and the barrier orders every wave's Z loads
      // after it (an acquire on every wave measured 70 us slower per launch).
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    return ready_s != 0;
  }
};

// Makes this workgroup's request outputs visible device-wide, then counts
// them in the counters of 32-row blocks [rb, rb + n) (one lane per tile).
__device__ __forceinline__ void publish(const FusedArgs& f, bool lead, int rb, int n) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (lead)
    for (int i = 0; i < n; ++i)
      if (rb + i < f.rblocks) __hip_atomic_fetch_add(f.flags + rb + i, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void request_tiles(const FusedArgs& f, int b, uint4* smem) {
  const GemmArgs& a = f.req;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (f.req_kind == 0) {
    const int ntn = (a.N + 127) / 128;
    const int t = xcd_remap(b, f.req_wg);
    const int m0 = (t / ntn) * 64, n0 = (t % ntn) * 128;
    gemm_tile<64, 128, 2, 4, 5>(a, m0, n0, smem);
    publish(f, threadIdx.x == 0, m0 / 32, 2);
  } else {
    // waves 0-3 run the tile with the request launch's four-slab rings (two
    // tiles per workgroup on two-slab rings measured 50 us slower per launch:
    // the chains are latency-bound); waves 4-7 only pass the barriers
    const int ntn = (a.N + 31) / 32;
    const int t = xcd_remap(b, f.req_wg);
    const int m0 = (t / ntn) * 32, n0 = (t % ntn) * 32;
    splitk_tile<4>(a, m0, n0, smem, wave & 3, lane, wave < 4);
    publish(f, threadIdx.x == 0, m0 / 32, 1);
  }
}

// H: candidate tile height; H2 > 0: the mixed plan (rows [0, M1) in 256-row
// tiles, then H2-row tiles, dispatched last).
template <int H, int H2>
__global__ __launch_bounds__(512, 1) void glm_fused_kernel(FusedArgs f) {
  __shared__ uint4 smem[2 * (256 + 256) * 8];
  const int b = blockIdx.x;
  if (b < f.req_wg) {
    request_tiles(f, b, smem);
    return;
  }
  const GemmArgs& a = f.cand;
  const ZRowsReady ready{a.zmap, a.M, a.zrows, f.flags, f.target, f.polls, f.err};
  const int cb = b - f.req_wg, nc = gridDim.x - f.req_wg;
  const int ntn = (a.N + 255) / 256;
  if constexpr (H2 == 0) {
    const int logical = xcd_remap(cb, nc);
    gemm_tile<H, 256, 2, 4, 2, ZRowsReady, true>(a, (logical / ntn) * H, (logical % ntn) * 256, smem, ready);
  } else {
    const int n1 = (f.M1 / 256) * ntn;
    if (cb < n1) {
      const int logical = xcd_remap(cb, n1);
      gemm_tile<256, 256, 2, 4, 2, ZRowsReady, true>(a, (logical / ntn) * 256, (logical % ntn) * 256, smem, ready);
    } else {
      const int logical = xcd_remap(cb - n1, nc - n1);
      gemm_tile<H2, 256, 2, 4, 2, ZRowsReady, true>(a, f.M1 + (logical / ntn) * H2, (logical % ntn) * 256, smem,
                                                    ready);
    }
  }
}

}  // namespace

int glm_fused_flag_count(const GemmArgs& req) { return (req.M + 31) / 32; }

bool glm_fused_supported(DType dt, const GemmArgs& req_in, const GemmArgs& cand_in) {
  if (dt != BF16) return false;
  GemmArgs req = req_in, cand = cand_in;
  req.epi = epilogue_variant(req);
  cand.epi = epilogue_variant(cand);
  if (req.M <= 0 || req.M >= 2048 || req.N <= 0 || req.batch > 1 || cand.batch > 1) return false;
  if (req.out1 == nullptr || req.n_split >= req.N) return false;  // the request tiles write Z
  if (cand.M < 2048 || cand.N <= 128 || cand.zmap == nullptr || cand.z != req.out1 || cand.ldz != req.ld1 ||
      cand.zrows != req.M)
    return false;
  if ((cand.epi & (EPI_Z | EPI_ZACC)) != (EPI_Z | EPI_ZACC)) return false;
  const CandPlan p = cand_plan(cand.M, (cand.N + 255) / 256);
  if (p.h == 0) return p.h2 == 64 || p.h2 == 128 || p.h2 == 192;
  return p.h == 256 || p.h == 192 || p.h == 128;
}

hipError_t launch_glm_fused(DType dt, const GemmArgs& req, const GemmArgs& cand, int* flags, int* err,
                            hipStream_t s) {
  if (!glm_fused_supported(dt, req, cand) || flags == nullptr || err == nullptr) return hipErrorNotSupported;
  FusedArgs f{};
  f.req = req;
  f.cand = cand;
  f.req.epi = epilogue_variant(req);
  f.cand.epi = epilogue_variant(cand);
  f.flags = flags;
  f.err = err;
  f.rblocks = glm_fused_flag_count(req);
  if (uses_splitk(req)) {
    const int tiles = f.rblocks * ((req.N + 31) / 32);
    f.req_kind = 1;
    f.req_wg = tiles;
    f.target = (req.N + 31) / 32;
  } else {
    f.req_kind = 0;
    f.req_wg = ((req.M + 63) / 64) * ((req.N + 127) / 128);
    f.target = (req.N + 127) / 128;
  }
  f.polls = kSpinLimit;
  // Failure injection for tests of the bounded wait: ROCS_TEST_FUSED_GIVE_UP=n
  // sets a target no counter reaches and n polls, so every candidate tile
  // gives up after n polls (its outputs NaN, *err set) and the grid drains.
  if (const char* e = std::getenv("ROCS_TEST_FUSED_GIVE_UP")) {
    const int n = std::atoi(e);
    if (n > 0) {
      f.polls = n;
      f.target = 0x7fffffff;
    }
  }
  const int ntn = (cand.N + 255) / 256;
  const CandPlan p = cand_plan(cand.M, ntn);
  int nc = 0;
  if (p.h == 0) {
    f.M1 = p.M1;
    nc = p.grid;
  } else {
    nc = ((cand.M + p.h - 1) / p.h) * ntn;
  }
  const dim3 grid(unsigned(f.req_wg + nc)), block(512);
  switch (p.h) {
    case 256: hipLaunchKernelGGL((glm_fused_kernel<256, 0>), grid, block, 0, s, f); break;
    case 192: hipLaunchKernelGGL((glm_fused_kernel<192, 0>), grid, block, 0, s, f); break;
    case 128: hipLaunchKernelGGL((glm_fused_kernel<128, 0>), grid, block, 0, s, f); break;
    default:
      switch (p.h2) {
        case 64: hipLaunchKernelGGL((glm_fused_kernel<256, 64>), grid, block, 0, s, f); break;
        case 128: hipLaunchKernelGGL((glm_fused_kernel<256, 128>), grid, block, 0, s, f); break;
        case 192: hipLaunchKernelGGL((glm_fused_kernel<256, 192>), grid, block, 0, s, f); break;
        default: return hipErrorNotSupported;
      }
  }
  return hipGetLastError();
}

}  // namespace rocs
