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
#include "rocs_mfma.h"

namespace rocs {

namespace {

// Weight rows of the (up to four) segments.  The segment table is copied
// out of the argument struct through an opaque asm into SGPRs and selected
// as plain values: selected as struct fields or argument memory, the choice
// becomes a per-lane indexed load (from argument memory, or from a private
// copy of the table that the compiler then places in LDS).
struct WeightSegs {
  const bf16 *w0, *w1, *w2, *w3;
  int e0, e1, e2;
};

__device__ __forceinline__ WeightSegs weight_segs(const GemmArgs& a) {
  const bf16* x0 = reinterpret_cast<const bf16*>(a.W[0]);
  const bf16* x1 = reinterpret_cast<const bf16*>(a.nseg > 1 ? a.W[1] : a.W[0]);
  const bf16* x2 = reinterpret_cast<const bf16*>(a.nseg > 2 ? a.W[2] : a.W[0]);
  const bf16* x3 = reinterpret_cast<const bf16*>(a.nseg > 3 ? a.W[3] : a.W[0]);
  int y0 = a.nseg > 1 ? a.seg_end[0] : 0x7fffffff;
  int y1 = a.nseg > 2 ? a.seg_end[1] : 0x7fffffff;
  int y2 = a.nseg > 3 ? a.seg_end[2] : 0x7fffffff;
  asm volatile("" : "+s"(x0), "+s"(x1), "+s"(x2), "+s"(x3), "+s"(y0), "+s"(y1), "+s"(y2));
  return WeightSegs{x0, x1, x2, x3, y0, y1, y2};
}

__device__ __forceinline__ const bf16* weight_row(const bf16* w0, const bf16* w1, const bf16* w2, const bf16* w3,
                                                  int e0, int e1, int e2, int64_t ldw, int n) {
  const bf16* p = n >= e2 ? w3 : n >= e1 ? w2 : n >= e0 ? w1 : w0;
  const int base = n >= e2 ? e2 : n >= e1 ? e1 : n >= e0 ? e0 : 0;
  return p + int64_t(n - base) * ldw;
}

__device__ __forceinline__ const bf16* weight_row(const GemmArgs& a, int n) {
  const WeightSegs t = weight_segs(a);
  return weight_row(t.w0, t.w1, t.w2, t.w3, t.e0, t.e1, t.e2, a.ldw, n);
}

template <typename T>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
  return to_f(reinterpret_cast<const T*>(p)[i]);
}

// Epilogue for one output row m and four consecutive columns n..n+3:
//   v = acc + Z[zrow(m)][n] + bias[n];  v = act(v);  v += res[m][n];  store
// (columns >= n_split go raw to out1 instead).
template <typename T>
__device__ __forceinline__ void epilogue4(const GemmArgs& a, int m, int n, const float* acc) {
  if (m >= a.M) return;
  int zrow = m;
  bool bad = false;
  if (a.z != nullptr && a.zmap != nullptr) {
    zrow = a.zmap[m];
    bad = (unsigned)zrow >= (unsigned)a.zrows;
  }
  const bool full = (n + 4 <= a.N) && (n + 4 <= a.n_split);
  if (full) {
    float v[4] = {acc[0], acc[1], acc[2], acc[3]};
    if (a.z != nullptr) {
      if (bad) {
        v[0] = v[1] = v[2] = v[3] = nan_f();
      } else {
        const float4 zz = *reinterpret_cast<const float4*>(a.z + int64_t(zrow) * a.ldz + n);
        v[0] += zz.x; v[1] += zz.y; v[2] += zz.z; v[3] += zz.w;
      }
    }
    if (a.bias != nullptr) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] += load_elem<T>(a.bias, n + j);
    }
    if (a.act == 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = fmaxf(v[j], 0.0f);
    }
    if (a.res != nullptr) {
      const T* r = reinterpret_cast<const T*>(a.res) + int64_t(m) * a.ldres + n;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] += to_f(r[j]);
    }
    if (a.out0_f32) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out0) + int64_t(m) * a.ld0 + n) =
          make_float4(v[0], v[1], v[2], v[3]);
    } else {
      T* o = reinterpret_cast<T*>(a.out0) + int64_t(m) * a.ld0 + n;
      if constexpr (sizeof(T) == 2) {
        bf16x4 pk = {to_bf(v[0]), to_bf(v[1]), to_bf(v[2]), to_bf(v[3])};
        *reinterpret_cast<bf16x4*>(o) = pk;
      } else {
        *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
    return;
  }
  for (int j = 0; j < 4; ++j) {
    const int c = n + j;
    if (c >= a.N) break;
    float v = acc[j];
    if (c < a.n_split) {
      if (a.z != nullptr) v = bad ? nan_f() : v + a.z[int64_t(zrow) * a.ldz + c];
      if (a.bias != nullptr) v += load_elem<T>(a.bias, c);
      if (a.act == 1) v = fmaxf(v, 0.0f);
      if (a.res != nullptr) v += load_elem<T>(a.res, int64_t(m) * a.ldres + c);
      if (a.out0_f32)
        reinterpret_cast<float*>(a.out0)[int64_t(m) * a.ld0 + c] = v;
      else
        reinterpret_cast<T*>(a.out0)[int64_t(m) * a.ld0 + c] = from_f<T>(v);
    } else if (a.out1 != nullptr) {
      a.out1[int64_t(m) * a.ld1 + (c - a.n_split)] = v;
    }
  }
}

// Epilogue of one element (m, c), same arithmetic as epilogue4.
template <typename T>
__device__ __forceinline__ void epilogue1(const GemmArgs& a, int m, int c, float v) {
  if (m >= a.M || c >= a.N) return;
  if (c < a.n_split) {
    if (a.z != nullptr) {
      const int zrow = a.zmap != nullptr ? a.zmap[m] : m;
      v = (unsigned)zrow >= (unsigned)a.zrows ? nan_f() : v + a.z[int64_t(zrow) * a.ldz + c];
    }
    if (a.bias != nullptr) v += load_elem<T>(a.bias, c);
    if (a.act == 1) v = fmaxf(v, 0.0f);
    if (a.res != nullptr) v += load_elem<T>(a.res, int64_t(m) * a.ldres + c);
    if (a.out0_f32)
      reinterpret_cast<float*>(a.out0)[int64_t(m) * a.ld0 + c] = v;
    else
      reinterpret_cast<T*>(a.out0)[int64_t(m) * a.ld0 + c] = from_f<T>(v);
  } else if (a.out1 != nullptr) {
    a.out1[int64_t(m) * a.ld1 + (c - a.n_split)] = v;
  }
}

// Per-wave LDS stage of the transposing epilogue: 32 rows of up to 64 fp32
// accumulators (two 32x32 blocks), rows padded by 16 bytes (conflict-free
// both ways).  Wider wave tiles go through it two blocks at a time.
template <int FN, int JWM = 2>
constexpr int stage_blocks() { return FN > JWM ? JWM : FN; }
template <int FN, int JWM = 2>
constexpr int stage_pitch() { return stage_blocks<FN, JWM>() * 32 + 4; }
template <int FN, int JWM = 2>
constexpr int stage_floats() { return 32 * stage_pitch<FN, JWM>(); }
template <int FN, int JWM = 2>
__device__ __forceinline__ int stage_at(int r, int c) { return r * stage_pitch<FN, JWM>() + c; }

// Epilogue variants.  EPI_ANY tests every optional term at run time; the
// others are fixed at compile time (request contribution gathered through
// the map or none, bias or none, then ReLU, a residual or neither), with
// 32-bit row offsets (launch_gemm checks the ranges).
enum : int {
  EPI_ANY = 0,
  EPI_Z = 1,     // z with zmap
  EPI_BIAS = 2,
  EPI_RELU = 4,
  EPI_RES = 8,
  EPI_ZACC = 16,  // with EPI_Z: the tile's accumulators started at Z[m_i] (zinit_acc)
  EPI_SPEC = 32,  // without EPI_Z: a fixed variant with no request contribution
};

// Writes one 32-row block-row of a wave's tile through the epilogue.  Block
// j: lane holds row mrow0 + lane%32 and columns nb + 32j + 8g +
// 4*(lane/32) + 0..3 in registers 4g..4g+3.  Stored directly, every
// instruction would touch 32 rows (half the achievable write bandwidth), so
// interior blocks pass through the wave's LDS stage and come back
// row-contiguous (JW*8 lanes per row, 4 columns each), JW column blocks at a
// time.  All loads of a pass (map entries, Z rows, residual) are issued
// before its arithmetic and stores.  The arithmetic is the edge path's:
// acc + Z + bias, act, + residual, one rounding.
template <int FN, int EPI = EPI_ANY, int JWM = 2>
__device__ __forceinline__ void store_row_staged(const GemmArgs& a, int mrow0, int nb, int lane,
                                                 const f32x16 (&row)[FN], float* stage) {
  constexpr bool ANY = EPI == EPI_ANY;
  constexpr int JW = stage_blocks<FN, JWM>();
  static_assert(FN % JW == 0, "column blocks must pair up");
  constexpr int LPR = JW * 8;     // lanes per row
  constexpr int RPI = 64 / LPR;   // rows per pass
  constexpr int NP = 32 / RPI;    // passes per block-row
  const int hk = lane >> 5;
  const float* __restrict__ z = a.z;
  const bf16* __restrict__ bias = reinterpret_cast<const bf16*>(a.bias);
  const bf16* __restrict__ res = reinterpret_cast<const bf16*>(a.res);
  bf16* __restrict__ out = reinterpret_cast<bf16*>(a.out0);
  const bool has_z = ANY ? z != nullptr : (EPI & EPI_Z) != 0 && (EPI & EPI_ZACC) == 0;
  const bool has_map = ANY ? a.zmap != nullptr : (EPI & EPI_Z) != 0 && (EPI & EPI_ZACC) == 0;
  const bool has_bias = ANY ? bias != nullptr : (EPI & EPI_BIAS) != 0;
  const bool relu = ANY ? a.act == 1 : (EPI & EPI_RELU) != 0;
  const bool has_res = ANY ? res != nullptr : (EPI & EPI_RES) != 0;
  const int rl = lane / LPR;
#pragma unroll
  for (int jg = 0; jg < FN / JW; ++jg) {
    const int n = nb + jg * JW * 32 + (lane % LPR) * 4;
    // map entries and residuals of this lane's NP rows, issued before the LDS round trip
    int zrow[NP];
    bf16x4 rr[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int m = min(mrow0 + p * RPI + rl, a.M - 1);
      zrow[p] = (has_z && has_map) ? a.zmap[m] : m;
      if (has_res) {
        const bf16* rp = ANY ? res + int64_t(m) * a.ldres + n : res + (uint32_t(m) * uint32_t(a.ldres) + n);
        rr[p] = *reinterpret_cast<const bf16x4*>(rp);
      }
    }
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if (has_bias) {
      const bf16x4 bb = *reinterpret_cast<const bf16x4*>(bias + n);
#pragma unroll
      for (int e = 0; e < 4; ++e) bv[e] = to_f(bb[e]);
    }
#pragma unroll
    for (int jj = 0; jj < JW; ++jj)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& c = row[jg * JW + jj];
        *reinterpret_cast<f32x4*>(stage + stage_at<FN, JWM>(lane & 31, jj * 32 + 8 * g + 4 * hk)) =
            f32x4{c[4 * g], c[4 * g + 1], c[4 * g + 2], c[4 * g + 3]};
      }
    __builtin_amdgcn_wave_barrier();
    float4 zz[NP];
    bool bad[NP];
    if (has_z) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        bad[p] = (unsigned)zrow[p] >= (unsigned)a.zrows;
        const int zr = bad[p] ? 0 : zrow[p];
        const float* zp = ANY ? z + int64_t(zr) * a.ldz + n : z + (uint32_t(zr) * uint32_t(a.ldz) + n);
        zz[p] = *reinterpret_cast<const float4*>(zp);
      }
    }
    f32x4 sv[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p)
      sv[p] = *reinterpret_cast<const f32x4*>(stage + stage_at<FN, JWM>(p * RPI + rl, (lane % LPR) * 4));
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int m = mrow0 + p * RPI + rl;
      float v[4] = {sv[p][0], sv[p][1], sv[p][2], sv[p][3]};
      if (has_z) {
        v[0] = bad[p] ? nan_f() : v[0] + zz[p].x;
        v[1] = bad[p] ? nan_f() : v[1] + zz[p].y;
        v[2] = bad[p] ? nan_f() : v[2] + zz[p].z;
        v[3] = bad[p] ? nan_f() : v[3] + zz[p].w;
      }
      if (has_bias)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += bv[e];
      if (relu)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaxf(v[e], 0.f);
      if (has_res)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += to_f(rr[p][e]);
      if (m < a.M) {
        bf16x4 pk = {to_bf(v[0]), to_bf(v[1]), to_bf(v[2]), to_bf(v[3])};
        bf16* op = ANY ? out + int64_t(m) * a.ld0 + n : out + (uint32_t(m) * uint32_t(a.ld0) + n);
        *reinterpret_cast<bf16x4*>(op) = pk;
      }
    }
  }
}

// Edge block-rows (N tail, the split between the two outputs, fp32 output):
// the block-row goes through the LDS stage too, then one element per lane
// at a time through epilogue1 (no register array is indexed at run time).
template <int FN, int JWM = 2>
__device__ __forceinline__ void store_row_edge(const GemmArgs& a, int mrow0, int nb, int lane,
                                               const f32x16 (&row)[FN], float* stage) {
  constexpr int JW = stage_blocks<FN, JWM>();
  constexpr int W = JW * 32;
  const int hk = lane >> 5;
#pragma unroll
  for (int jg = 0; jg < FN / JW; ++jg) {
#pragma unroll
    for (int jj = 0; jj < JW; ++jj)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& c = row[jg * JW + jj];
        *reinterpret_cast<f32x4*>(stage + stage_at<FN, JWM>(lane & 31, jj * 32 + 8 * g + 4 * hk)) =
            f32x4{c[4 * g], c[4 * g + 1], c[4 * g + 2], c[4 * g + 3]};
      }
    __builtin_amdgcn_wave_barrier();
    for (int e = lane; e < 32 * W; e += 64) {
      const int r = e / W, c = e % W;
      epilogue1<bf16>(a, mrow0 + r, nb + jg * W + c, stage[stage_at<FN, JWM>(r, c)]);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int FN, int EPI, int JWM>
__device__ __forceinline__ void store_row(const GemmArgs& a, int mrow0, int nb, int lane, const f32x16 (&row)[FN],
                                          float* stage) {
  const bool interior = (nb + FN * 32 <= a.N) && (nb + FN * 32 <= a.n_split) && !a.out0_f32;
  if (interior)
    store_row_staged<FN, EPI, JWM>(a, mrow0, nb, lane, row, stage);
  else
    store_row_edge<FN, JWM>(a, mrow0, nb, lane, row, stage);
}

template <int EPI, int JWM, int FM, int FN>
__device__ __forceinline__ void store_blocks_as(const GemmArgs& a, int mb, int nb, int lane,
                                                const f32x16 (&acc)[FM][FN], float* stage) {
#pragma unroll
  for (int i = 0; i < FM; ++i) store_row<FN, EPI, JWM>(a, mb + i * 32, nb, lane, acc[i], stage);
}

// The epilogue variant is uniform per launch: one switch, then straight-line
// code without per-element feature tests.
template <int JWM = 2, int FM, int FN>
__device__ __forceinline__ void store_blocks(const GemmArgs& a, int mb, int nb, int lane, const f32x16 (&acc)[FM][FN],
                                             float* stage) {
#define ROCS_EPI_CASE(V) \
  case (V): store_blocks_as<(V), JWM>(a, mb, nb, lane, acc, stage); break;
#define ROCS_EPI_TAILS(P) \
  ROCS_EPI_CASE(P) ROCS_EPI_CASE(P | EPI_RELU) ROCS_EPI_CASE(P | EPI_RES) ROCS_EPI_CASE(P | EPI_BIAS) \
  ROCS_EPI_CASE(P | EPI_BIAS | EPI_RELU) ROCS_EPI_CASE(P | EPI_BIAS | EPI_RES)
  switch (a.epi) {
    ROCS_EPI_TAILS(EPI_Z)
    ROCS_EPI_TAILS(EPI_Z | EPI_ZACC)
    ROCS_EPI_TAILS(EPI_SPEC)
    default: store_blocks_as<EPI_ANY, JWM>(a, mb, nb, lane, acc, stage); break;
  }
#undef ROCS_EPI_TAILS
#undef ROCS_EPI_CASE
}

// ----------------------------------------------------------------- DMA-staged bf16 GEMM
// For the candidate-batch GEMMs (M = B_c in the tens of thousands).  A
// BM x BN tile per workgroup of WM x WN waves; each wave owns a
// (BM/WM) x (BN/WN) sub-tile of 32x32 blocks.  Operand slabs (64 wide in K)
// move global -> LDS with global_load_lds_dwordx4 (no register staging)
// through a ring of NS slab buffers: NS-1 slabs are in flight while one is
// multiplied, which hides the HBM latency of the activation rows (each slab
// of a 512-deep K is a fresh HBM read).  Each wave-instruction fills 1 KB of
// LDS (8 rows of 128 B); lane i fetches the global chunk that the row
// swizzle places at its LDS slot.  Chunks past K come from a zero page, so K
// tails need no masking (K is a multiple of 8: weight and activation rows
// are 16-byte aligned).
__device__ uint4 g_zero_page[4];

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt with vmcnt(N), expcnt and lgkmcnt left at their maxima (gfx9
// encoding: vmcnt bits [3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Wait until at most `newer` slabs of PER instructions each are outstanding
// (0 <= newer <= MAXN; the immediate must be a compile-time constant).
template <int PER, int MAXN>
__device__ __forceinline__ void wait_slabs(int newer) {
  if constexpr (MAXN > 0) {
    if (newer >= MAXN) {
      wait_vmcnt<PER * MAXN>();
      return;
    }
    wait_slabs<PER, MAXN - 1>(newer);
  } else {
    wait_vmcnt<0>();
  }
}

// This wave's share of the slab DMA for one BM x BN tile: PER
// wave-instructions per 64-wide slab, each filling 1 KB of the ring (8 rows
// of 128 B); lane i fetches the global chunk that the row swizzle places at
// its LDS slot.  Chunks past K come from the zero page.
template <int BM, int BN, int NW>
struct SlabFeed {
  static constexpr int CPR = 8, RPI = 8;
  static constexpr int RB = (BM + BN) / RPI;
  static_assert(RB % NW == 0, "row blocks must divide among waves");
  static constexpr int PER = RB / NW;
  const bf16* src[PER];
  int kofs[PER];
  __device__ __forceinline__ void init(const GemmArgs& a, const WeightSegs& ws, int m0, int n0, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int r = (wave * PER + j) * RPI + lane / CPR;
      const int chunk = (lane % CPR) ^ swz<CPR>(r);
      kofs[j] = chunk * 8;
      if (r < BM)
        src[j] = reinterpret_cast<const bf16*>(a.A) + int64_t(min(m0 + r, a.M - 1)) * a.lda + chunk * 8;
      else
        src[j] = weight_row(ws.w0, ws.w1, ws.w2, ws.w3, ws.e0, ws.e1, ws.e2, a.ldw, min(n0 + r - BM, a.N - 1)) +
                 chunk * 8;
    }
  }
  __device__ __forceinline__ void issue(int K, const void* zero, int k0, uint4* slot, int wave) const {
    if (k0 + CPR * 8 <= K) {  // a whole slab inside K (a wave-uniform branch): no per-lane select
#pragma unroll
      for (int j = 0; j < PER; ++j)
        __builtin_amdgcn_global_load_lds(src[j] + k0, (lds_ptr_t)(slot + (wave * PER + j) * 64), 16, 0, 0);
      return;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const void* p = (k0 + kofs[j] < K) ? static_cast<const void*>(src[j] + k0) : zero;
      __builtin_amdgcn_global_load_lds(p, (lds_ptr_t)(slot + (wave * PER + j) * 64), 16, 0, 0);
    }
  }
};

// The zero page's address comes from the GOT.  Loaded inside a loop, that
// scalar load (out of order with LDS reads on the same counter) would turn
// every fragment wait into a full lgkmcnt(0); pinned in SGPRs by the caller,
// it is loaded once.
__device__ __forceinline__ const void* pinned_zero_page() {
  const void* zero = g_zero_page;
  asm volatile("" : "+s"(zero));
  return zero;
}

// Starts a wave's accumulators at the request contribution Z[m_i] of its
// rows (EPI_ZACC launches), so the epilogue has nothing left to gather and
// the Z loads overlap the first slab's DMA: acc = Z[m] + the products, in
// that order.  A row whose map entry is out of range starts at NaN.  Block
// (i, j): lane holds row mb + 32i + lane%32 and columns nb + 32j + 8g +
// 4*(lane/32) + 0..3 in registers 4g..4g+3.  Offsets are 32-bit (checked
// when the variant is chosen).
template <int FM, int FN>
__device__ __forceinline__ void zinit_acc(const GemmArgs& a, int mb, int nb, int lane, f32x16 (&acc)[FM][FN]) {
  const int hk = lane >> 5;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row = min(mb + i * 32 + (lane & 31), a.M - 1);
    const int zr = a.zmap ? a.zmap[row] : row;  // no map: Z has one row per output row
    const bool bad = (unsigned)zr >= (unsigned)a.zrows;
    const float* zp = a.z + (uint32_t(bad ? 0 : zr) * uint32_t(a.ldz) + uint32_t(nb + 4 * hk));
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 v = *reinterpret_cast<const float4*>(zp + j * 32 + 8 * g);
        acc[i][j][4 * g + 0] = bad ? nan_f() : v.x;
        acc[i][j][4 * g + 1] = bad ? nan_f() : v.y;
        acc[i][j][4 * g + 2] = bad ? nan_f() : v.z;
        acc[i][j][4 * g + 3] = bad ? nan_f() : v.w;
      }
  }
}

// One BM x BN output tile at (m0, n0) on a workgroup of WM x WN waves, with
// the ring (NS slots of BM + BN rows of one 64-wide slab) at smem; slab kb
// lives in slot kb % NS.
template <int BM, int BN, int WM, int WN, int NS>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, int m0, int n0, uint4* smem) {
  constexpr int BK = 64;
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int CPR = BK / 8;
  constexpr int SLOT = (BM + BN) * CPR;
  static_assert(NW * stage_floats<FN>() * 4 <= NS * SLOT * 16, "epilogue stage exceeds the ring");
  using Feed = SlabFeed<BM, BN, NW>;
  static_assert(NS >= 2 && Feed::PER * (NS - 2) < 64, "ring depth");
  // the wave index is uniform: the LDS slot addresses of the DMA stay scalar
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const void* zero = pinned_zero_page();
  const WeightSegs ws = weight_segs(a);
  auto slot = [&](int kb) { return smem + (kb % NS) * SLOT; };

  Feed feed;
  feed.init(a, ws, m0, n0, wave, lane);
  f32x16 acc[FM][FN];

  const int nk = (a.K + BK - 1) / BK;
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) feed.issue(a.K, zero, s * BK, slot(s), wave);
  if (a.epi & EPI_ZACC)
    zinit_acc(a, m0 + wm * WTM, n0 + wn * WTN, lane, acc);
  else
    zero_acc(acc);

  const int xr0 = wm * WTM + (lane & 31);
  const int wr0 = BM + wn * WTN + (lane & 31);
  Frags<FM, FN> fr;
  for (int kb = 0; kb < nk - 1; ++kb) {
    // Slab kb has landed once at most min(NS-2, nk-1-kb) newer slabs (PER
    // instructions each, returned in order) are still outstanding.
    wait_slabs<Feed::PER, NS - 2>(min(NS - 2, nk - 1 - kb));
    // every wave's part of slab kb is in LDS, and every wave is done with
    // slab kb-1 (its last step's fragments are in registers), whose slot
    // the next issue refills
    __syncthreads();
    if (kb + NS - 1 < nk) feed.issue(a.K, zero, (kb + NS - 1) * BK, slot(kb + NS - 1), wave);
    const uint4* sl = slot(kb);
    mfma_slab_carry<FM, FN, CPR, CPR>(fr, kb > 0, sl, wr0, sl, xr0, lane >> 5, acc);
  }
  if (nk > 0) {  // the last slab, then the carried step
    wait_vmcnt<0>();
    __syncthreads();
    const uint4* sl = slot(nk - 1);
    mfma_slab_carry<FM, FN, CPR, CPR>(fr, nk > 1, sl, wr0, sl, xr0, lane >> 5, acc);
    mfma_frags(fr, 1, acc);
  }
  __syncthreads();  // every wave is done reading the ring: the epilogue stages in it
  store_blocks(a, m0 + wm * WTM, n0 + wn * WTN, lane, acc, reinterpret_cast<float*>(smem) + wave * stage_floats<FN>());
}

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
// 32 x 32 tiles than CUs: 32 x 32 output tiles, four waves per tile, wave w reducing the
// contiguous K quarter [w nk / 4, (w + 1) nk / 4) through a ring of its own
// (no workgroup barrier in the loop).  The four fp32 partial tiles are then
// added in a fixed order, ((p0 + p1) + p2) + p3, and wave 0 runs the
// epilogue.  The result is deterministic; it is summed in a different order
// than the single-chain kernels.  The choice depends on the launch's shape
// only (uses_splitk).
template <int NS>
__global__ __launch_bounds__(256, 1) void gemm_bf16_splitk_kernel(GemmArgs a0) {
  const GemmArgs a = batch_slice(a0, blockIdx.y);  // GEMM blockIdx.y of a batch
  constexpr int BM = 32, BN = 32, BK = 64, CPR = 8, SLOT = (BM + BN) * CPR, SPLIT = 4;
  __shared__ uint4 smem[SPLIT * NS * SLOT];
  using Feed = SlabFeed<BM, BN, 1>;
  static_assert(Feed::PER * (NS - 2) < 64, "ring depth");
  const int ntn = (a.N + BN - 1) / BN;
  const int ntm = (a.M + BM - 1) / BM;
  const int logical = xcd_remap(blockIdx.x, ntm * ntn);
  const int m0 = (logical / ntn) * BM, n0 = (logical % ntn) * BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const void* zero = pinned_zero_page();
  const WeightSegs ws = weight_segs(a);
  uint4* ring = smem + wave * NS * SLOT;
  auto slot = [&](int i) { return ring + (i % NS) * SLOT; };

  const int nk = (a.K + BK - 1) / BK;
  const int k_lo = (wave * nk) / SPLIT, k_hi = ((wave + 1) * nk) / SPLIT;
  const int n = k_hi - k_lo;  // slabs of this wave
  Feed feed;
  feed.init(a, ws, m0, n0, 0, lane);
  f32x16 acc[1][1];
  zero_acc(acc);
#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (i < n) feed.issue(a.K, zero, (k_lo + i) * BK, slot(i), 0);
  Frags<1, 1> fr;
  for (int i = 0; i < n; ++i) {
    wait_slabs<Feed::PER, NS - 2>(min(NS - 2, n - 1 - i));
    __builtin_amdgcn_wave_barrier();
    if (i + NS - 1 < n) feed.issue(a.K, zero, (k_lo + i + NS - 1) * BK, slot(i + NS - 1), 0);
    const uint4* sl = slot(i);
    mfma_slab_carry<1, 1, CPR, CPR>(fr, i > 0, sl, BM + (lane & 31), sl, lane & 31, lane >> 5, acc);
  }
  if (n > 0) mfma_frags(fr, 1, acc);
  __syncthreads();  // every wave is done with its ring: the partials go there
  float* part = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int r = 0; r < 16; ++r) part[(wave * 16 + r) * 64 + lane] = acc[0][0][r];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float v = part[r * 64 + lane];
#pragma unroll
    for (int w = 1; w < SPLIT; ++w) v += part[(w * 16 + r) * 64 + lane];
    acc[0][0][r] = v;
  }
  // The partial sums started at zero, so the epilogue adds Z: the mapped
  // variant without EPI_ZACC, or the generic one when Z has no map (only
  // EPI_ZACC variants accept an unmapped Z).
  GemmArgs e = a;
  if (e.epi & EPI_ZACC) e.epi = a.zmap ? (e.epi & ~EPI_ZACC) : EPI_ANY;
  store_blocks(e, m0, n0, lane, acc, part + SPLIT * 16 * 64);
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
struct CandPlan {
  int h;             // uniform tile height, or 0 for the mixed plan
  int M1, h2, grid;  // mixed plan
};

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
