// Grouped attention for DCA ([R] §2.2 grouped cross-attention; [R] §2.4
// IKBO-DCA): keys/values stay at request-batch size and every query tile is
// made of queries of ONE request, so each staged key/value tile in LDS is
// shared by all the queries of the workgroup, and the tiles of one request
// run back to back on one XCD (shared L2).  The same kernel runs the
// request-only encoder's self-attention (group = one request's sequence).
//
// Per workgroup: 4 waves x 32 queries = 128 queries of one group and one
// head (head_dim 64).  Keys and values stream in 64-key slabs, as they are
// stored (row-major key rows), global -> LDS by DMA through a 3-stage ring
// (two slabs in flight).  Each wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16, so each lane holds scores of a single query:
// the online-softmax max needs one exchange between lanes l and l ^ 32 per
// slab (v_permlane32_swap).  The row sums of P come from the matrix cores:
// one more 32 x 32 accumulator takes ones x P^T next to the PV product, so
// every register of lane l holds the sum of its query's bf16 P (the
// softmax is VALU-issue bound and the MFMA pipe has room).  P^T is fed back as the B operand of
// O^T = V^T P^T in the register order the S^T accumulator produced; the
// V^T operand is read from the row-major value tile with transposing LDS
// reads (ds_read_b64_tr_b16) in that same key order.  Softmax in fp32 with
// exp2 and the scale folded into one multiply-add; the running maximum is
// only moved when a score exceeds it by more than 2^8 in exp2 units (lazy
// rescaling).
#include <cstdlib>
#include "rocs_device.h"

namespace rocs {

namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One wave-instruction of global -> LDS DMA: lane i's 16 bytes land at
// dst + 16*i (dst wave-uniform).  Written as asm so that the compiler, which
// would otherwise wait for every LDS DMA in flight before any LDS read, leaves
// the ring's waits to the explicit vmcnt counts below.  No register receives
// data (the load writes LDS only); the wait state after the M0 write is the
// one LDS DMA needs.
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  const uint32_t m0 = uint32_t(uintptr_t((lds_ptr_t)dst));
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}
// The same DMA from a wave-uniform base held in SGPRs plus a 32-bit per-lane
// byte offset: no 64-bit address arithmetic on the vector unit per load.  The
// base is copied by the scalar unit first: a vector-memory read of an SGPR
// written by a VALU instruction (v_readfirstlane, v_readlane) needs five wait
// states, which the compiler does not insert for inline asm.
__device__ __forceinline__ void dma16_s(const char* base, uint32_t off, void* dst) {
  const uint32_t m0 = uint32_t(uintptr_t((lds_ptr_t)dst));
  uint64_t b;
  asm volatile("s_mov_b64 %0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %0"
               : "=&s"(b)
               : "s"(base), "v"(off), "{m0}"(m0)
               : "memory");
}
// A pointer whose value is the same in every lane, moved to SGPRs.
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(u >> 32));
  return reinterpret_cast<const char*>((uint64_t(hi) << 32) | lo);
}
// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt bits [3:0] and [15:14]; expcnt,
// lgkmcnt at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

constexpr int TQ = 128;  // queries per workgroup
constexpr int KC = 64;   // keys per slab
constexpr int DH = 64;   // head dim

// Tiles hold 8 16-byte chunks per 128-byte row; chunk c of row r sits at
// c ^ swz(r), with swz(r) = (r1 << 2) | ((r0 ^ r3) << 1) | r2 for the bits
// r0..r3 of r.  Both LDS read patterns then hit distinct banks whether the
// LDS serves 128 or 256 bytes per clock: the K fragment reads (32
// consecutive rows, one chunk column; swz is a permutation over any 8
// aligned rows, and over the 8 rows of one parity in 16) and the transposed
// V reads (4 consecutive rows x 2 chunks per 16 lanes; swz bits 1-2 differ
// between the 4 rows, and bit 2 flips between rows 2 apart).
__device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) << 2) | (((r ^ (r >> 3)) & 1) << 1) | ((r >> 2) & 1); }
// K and V tiles: [64 keys][64 dh] bf16.
__device__ __forceinline__ int k_off(int key, int chunk) { return key * 8 + (chunk ^ swz(key)); }

// Query tile of one workgroup: group (request / sequence), rows [rbeg, rend)
// of the query batch, head h.  Returns false when the workgroup has no tile.
struct QTile {
  int group, rbeg, rend, h;
};
// (tile, head) pairs of a launch: tiles of the plan (or of the uniform
// groups) times heads; a plan's count is an upper bound (max_tiles).
__device__ __forceinline__ int attn_total(const AttnArgs& a) {
  const int tiles = a.q_rows_per_group > 0 ? a.n_groups * ((a.q_rows_per_group + TQ - 1) / TQ) : a.max_tiles;
  return tiles * a.n_heads;
}

// Tile and head of logical pair `logical`; false past the plan's tile count.
__device__ __forceinline__ bool decode_tile(const AttnArgs& a, int logical, QTile& t) {
  const int H = a.n_heads;
  int n_tiles;
  if (a.q_rows_per_group > 0)
    n_tiles = a.n_groups * ((a.q_rows_per_group + TQ - 1) / TQ);
  else
    n_tiles = *a.n_tiles_dev;
  const int tile = logical / H;
  t.h = logical - tile * H;
  if (tile >= n_tiles) return false;
  if (a.q_rows_per_group > 0) {
    const int tpg = (a.q_rows_per_group + TQ - 1) / TQ;
    t.group = tile / tpg;
    t.rbeg = t.group * a.q_rows_per_group + (tile - t.group * tpg) * TQ;
    t.rend = min(t.rbeg + TQ, (t.group + 1) * a.q_rows_per_group);
  } else {
    t.group = a.tile_info[3 * tile + 0];
    t.rbeg = a.tile_info[3 * tile + 1];
    t.rend = a.tile_info[3 * tile + 2];
  }
  return true;
}

// Per-lane query state: the Q^T fragments (B operand; lane holds query
// q_local, dh 16*ks + 8*hl + 0..7), the output accumulators O^T and the
// online-softmax reference and sum.
struct QState {
  bf16x8 qf[4];
  f32x16 o_acc[2];
  f32x16 l_acc;  // every register: the running sum of this lane's query's P
  float m_run;
};

// Candidates whose request id was out of range get NaN rows.
__device__ __forceinline__ void write_nan_row(const AttnArgs& a, int64_t q_phys, int h, int hl) {
  bf16* o = a.o + q_phys * a.ldo + h * DH;
  for (int e = hl * 32; e < hl * 32 + 32; ++e) o[e] = to_bf(nan_f());
}

__device__ __forceinline__ void load_q(const AttnArgs& a, int64_t q_phys, bool q_ok, int h, int hl, QState& st) {
  const bf16* qp = a.q + q_phys * a.ldq + h * DH;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (q_ok) u = *reinterpret_cast<const uint4*>(qp + ks * 16 + hl * 8);
    st.qf[ks] = __builtin_bit_cast(bf16x8, u);
  }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < 16; ++j) st.o_acc[t][j] = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) st.l_acc[j] = 0.f;
  st.m_run = -INFINITY;
}

// max of x over lanes l and l ^ 32 (v_permlane32_swap gives every lane both
// values: a VALU exchange, no LDS round trip).
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element i % 4 of the 4 x 16-bit words that lanes
// 4k + i / 4 (k = 0..3) address, in that order of k.
__device__ __forceinline__ v4s read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)((__attribute__((address_space(3))) const char*)p));
}

// Byte offset, in a row-major [64 keys][64 dh] tile (k_off layout), of the
// 4 x 16-bit word this lane addresses for the transposed V reads of head-dim
// block dt (32 dh) and key run j.  Source lane 4k + g of 16-lane group G
// addresses keys 8j + 4 hl + k (hl = G / 2) and dh 32 dt + 16 (G % 2) + 4g
// .. +3, so output lane i of the group holds dh 32 dt + 16 (G % 2) + i for
// the four keys 8j + 4 hl + 0..3: the A operand of O^T = V^T P^T for MFMA
// rows (lane % 32) and the key order the P^T registers come in.  A slab's
// key tile (32 kt + 16 sp) adds a multiple of 16 rows, which keeps the row
// swizzle.
__device__ __forceinline__ int vrow_off(int lane, int dt, int j) {
  const int G = lane >> 4, k = (lane >> 2) & 3, g = lane & 3;
  const int row = 8 * j + 4 * (G >> 1) + k;
  const int chunk = 4 * dt + 2 * (G & 1) + (g >> 1);
  return row * 128 + (chunk ^ swz(row)) * 16 + (g & 1) * 8;
}

// One 64-key slab for the wave's 32 queries: S^T = K Q^T, online softmax,
// O^T += V^T P^T.  tK, tV: [64 keys][8 chunks] (k_off); tV is read
// transposed (vo: vrow_off per dt, j).  key0 = first key of the slab.
__device__ __forceinline__ void attend_slab(const uint4* tK, const uint4* tV, int key0, int L, float c, int lane,
                                            QState& st, const int (&vo)[2][2]) {
  const int hl = lane >> 5;
  // All 8 K fragments first (their LDS latency overlaps), then the S MFMAs.
  uint4 kf[8];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kf[kt * 4 + ks] = tK[k_off(kt * 32 + (lane & 31), ks * 2 + hl)];
  __builtin_amdgcn_sched_barrier(0);
  // S^T tiles: keys kt*32 + row, queries = lane columns
  f32x16 s[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
    for (int j = 0; j < 16; ++j) s[kt][j] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[kt * 4 + ks]), st.qf[ks], s[kt],
                                                      0, 0, 0);
  }
  // V^T fragments next: read while the softmax below runs.
  // keys kt*32 + 16*sp + 8*(q/4) + 4*hl + q%4 = chunk 4*kt + 2*sp + hl
  uint4 vf[8];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        const char* tb = reinterpret_cast<const char*>(tV) + (kt * 32 + 16 * sp) * 128;
        const v4s lo = read_tr16(tb + vo[dt][0]), hi = read_tr16(tb + vo[dt][1]);
        vf[dt * 4 + kt * 2 + sp] = __builtin_bit_cast(uint4, v8s(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)));
      }
  __builtin_amdgcn_sched_barrier(0);
  // mask keys beyond L (last slab only)
  if (key0 + KC > L) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = key0 + kt * 32 + 8 * (j >> 2) + 4 * hl + (j & 3);
        if (key >= L) s[kt][j] = -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kt][j]);
  mx = halves_max(mx);
  // Lazy rescaling: the running reference m_run moves only when some query of
  // the wave sees a score more than 2^8 above it (in exp2 units); otherwise
  // P may reach 2^8, which fp32 sums and bf16 P hold as well as values <= 1.
  // O and l always share one reference, so O / l is unchanged.
  if (__builtin_amdgcn_ballot_w64((mx - st.m_run) * c > 8.f)) {
    const float m_new = fmaxf(st.m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f((st.m_run - m_new) * c);  // 0 on the first slab
#pragma unroll
    for (int j = 0; j < 16; ++j) st.l_acc[j] *= alpha;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) st.o_acc[t][j] *= alpha;
    st.m_run = m_new;
  }
  const float mc = st.m_run * c;
  bf16x8 pf[4];  // B operand for the PV step: [kt*2 + step]
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int sp = 0; sp < 2; ++sp)
#pragma unroll
      for (int q = 0; q < 8; ++q) pf[kt * 2 + sp][q] = to_bf(__builtin_amdgcn_exp2f(fmaf(s[kt][sp * 8 + q], c, -mc)));

  // O^T[dh][query] += V^T[dh][keys] P^T[keys][query]
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int sp = 0; sp < 2; ++sp)
        st.o_acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf[dt * 4 + kt * 2 + sp]),
                                                               pf[kt * 2 + sp], st.o_acc[dt], 0, 0, 0);
  // l += ones x P^T: the sum over the slab's 64 keys of the bf16 P the PV
  // product uses, for this lane's query, in every register
  const bf16 one = to_bf(1.f);
  const bf16x8 ones = {one, one, one, one, one, one, one, one};
#pragma unroll
  for (int t = 0; t < 4; ++t) st.l_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pf[t], st.l_acc, 0, 0, 0);
}

__device__ __forceinline__ void write_out(const AttnArgs& a, int64_t q_phys, int h, int hl, const QState& st) {
  const float inv = 1.0f / st.l_acc[0];
  bf16* o = a.o + q_phys * a.ldo + h * DH;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // registers 4g..4g+3 hold dh = dt*32 + 8g + 4*hl + 0..3
      bf16x4 pk = {to_bf(st.o_acc[dt][4 * g + 0] * inv), to_bf(st.o_acc[dt][4 * g + 1] * inv),
                   to_bf(st.o_acc[dt][4 * g + 2] * inv), to_bf(st.o_acc[dt][4 * g + 3] * inv)};
      *reinterpret_cast<bf16x4*>(o + dt * 32 + 8 * g + 4 * hl) = pk;
    }
}

// K and V slabs move global -> LDS by DMA (global_load_lds_dwordx4) through
// a ring of NST stages, so two slabs are in flight while one is consumed and
// no registers hold staged data.  Both tiles are row-major key rows in the
// k_off layout (V is read transposed by the PV step).  Each wave fills 2 of
// the 8 1-KB pieces of each tile; lane i fetches the 16-byte chunk that the
// row swizzle places at its LDS slot.
constexpr int NST = 3;
template <int S>
struct Stage {
  static constexpr int value = S;
};
constexpr int DMA_PER_SLAB = 4;  // wave-instructions per slab per wave (2 K + 2 V)

typedef uint4 AttnRing[NST][KC * 8];

// One (tile, head) pair on the workgroup's K and V rings.
__device__ __forceinline__ void attn_tile(const AttnArgs& a, int logical, AttnRing& sK, AttnRing& sV) {
  QTile t;
  if (!decode_tile(a, logical, t)) return;
  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q_local = t.rbeg + wave * 32 + (lane & 31);
  const bool q_ok = q_local < t.rend;
  const int64_t q_phys = q_ok ? (a.perm ? a.perm[q_local] : q_local) : 0;
  if (t.group >= a.n_groups) {
    if (q_ok) write_nan_row(a, q_phys, t.h, hl);
    return;
  }
  const int L = a.L;
  const int nslab = (L + KC - 1) / KC;

  // LDS entry (2*wave + j)*64 + lane of a tile is row r = (2*wave + j)*8 +
  // lane/8, slot lane%8, which holds global chunk (lane%8) ^ swz(r) of that
  // row.  Each lane's source is a fixed byte offset from the slab's base
  // (kept in SGPRs; the launcher checks that 64 key rows span less than
  // 2 GiB).  K and V rows share the stride and offsets.
  const int row0 = wave * 16 + (lane >> 3);  // j = 0; j = 1 adds 8
  int chunk[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) chunk[j] = (lane & 7) ^ swz(row0 + 8 * j);
  const int64_t gofs = int64_t(t.group) * a.kv_group_stride + t.h * DH;
  const bf16* kbase = a.k + gofs;
  const bf16* vbase = a.v + gofs;
  const char* kb_s = uniform_ptr(kbase);
  const char* vb_s = uniform_ptr(vbase);
  const int64_t kslab = int64_t(KC) * a.ldkv * 2;  // bytes between slabs of key rows
  uint32_t koff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) koff[j] = uint32_t(((row0 + 8 * j) * a.ldkv + chunk[j] * 8) * 2);
  int vo[2][2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int j = 0; j < 2; ++j) vo[dt][j] = vrow_off(lane, dt, j);
  auto issue = [&](int slab, auto stage) {
    constexpr int S = decltype(stage)::value;
    if ((slab + 1) * KC <= L) {
      const int64_t so = slab * kslab;
#pragma unroll
      for (int j = 0; j < 2; ++j) dma16_s(kb_s + so, koff[j], &sK[S][(2 * wave + j) * 64]);
#pragma unroll
      for (int j = 0; j < 2; ++j) dma16_s(vb_s + so, koff[j], &sV[S][(2 * wave + j) * 64]);
    } else {
      // the ragged last slab: keys past L read row L-1 (their scores are
      // masked, so their P is 0 and the finite V row adds nothing)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t o = int64_t(min(slab * KC + row0 + 8 * j, L - 1)) * a.ldkv + chunk[j] * 8;
        dma16(kbase + o, &sK[S][(2 * wave + j) * 64]);
        dma16(vbase + o, &sV[S][(2 * wave + j) * 64]);
      }
    }
  };

  // Every step issues one slab (the last one again once past the end), so
  // "this wave's DMA for slab sb has landed" is always vmcnt <= one slab.
  issue(0, Stage<0>{});
  issue(min(1, nslab - 1), Stage<1>{});
  QState st;
  load_q(a, q_phys, q_ok, t.h, hl, st);
  // The compiler does not see the DMA on the load counter: make it wait for
  // the Q fragments here, once, rather than inside the loop at their first use.
  asm volatile("" : : "v"(st.qf[0]), "v"(st.qf[1]), "v"(st.qf[2]), "v"(st.qf[3]));
  // Slab sb lives in stage sb % 3.  The loop is unrolled over the stages so
  // that every LDS address is a lane offset plus a constant.
  auto step = [&](int sb, auto stage) {
    constexpr int CUR = decltype(stage)::value, NXT = (CUR + 2) % NST;
    wait_vmcnt<DMA_PER_SLAB>();
    __syncthreads();  // slab sb is in LDS for all waves; stage NXT (slab sb-1) is free
    issue(min(sb + 2, nslab - 1), Stage<NXT>{});
    attend_slab(sK[CUR], sV[CUR], sb * KC, L, a.scale_log2, lane, st, vo);
  };
  for (int sb = 0; sb < nslab; sb += NST) {
    step(sb, Stage<0>{});
    if (sb + 1 < nslab) step(sb + 1, Stage<1>{});
    if (sb + 2 < nslab) step(sb + 2, Stage<2>{});
  }
  wait_vmcnt<0>();  // no DMA may still write this workgroup's LDS when it exits
  if (q_ok) write_out(a, q_phys, t.h, hl, st);
}

__global__ __launch_bounds__(256, 3) void attn_dma_kernel(AttnArgs a) {
  __shared__ AttnRing sK, sV;
  attn_tile(a, xcd_remap(blockIdx.x, attn_total(a)), sK, sV);
}

// The persistent grid ([R] §2.4, the persistent attention kernel across short
// query tiles): one round of workgroups (three per CU), each walking the
// (tile, head) pairs of its XCD's contiguous range, the range the one-pair-
// per-workgroup grid gives that XCD, so a request's tiles still share that
// XCD's L2.  The workgroup's LDS rings are reused from pair to pair; a
// barrier separates pairs (a fast wave may not refill a stage that a slow
// wave still reads).  Every pair is computed as in attn_dma_kernel, so the
// outputs are the same bits.  Measured slower than one workgroup per pair on
// the ranking-scale stack (the barrier holds all four waves until the
// slowest ends the pair, where a new workgroup would start beside the CU's
// other two), so only the one-launch schedule uses it.
__global__ __launch_bounds__(256, 3) void attn_persist_kernel(AttnArgs a) {
  __shared__ AttnRing sK, sV;
  const int total = attn_total(a);
  const int q = total >> 3, r = total & 7;
  const int x = blockIdx.x & 7, px = gridDim.x >> 3;  // gridDim.x is a multiple of 8
  const int start = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
  const int size = q + (x < r ? 1 : 0);
  for (int k = blockIdx.x >> 3; k < size; k += px) {
    if (k >= px) __syncthreads();
    attn_tile(a, start + k, sK, sV);
  }
}

// ----------------------------------------------------------------- planning
// Per-request query tiles.  Bucket B_r collects candidates whose request id
// is out of range (their outputs become NaN).
struct PlanWs {
  int32_t* cnt;      // [B_r + 2]
  int32_t* offs;     // [B_r + 2]
  int32_t* cursor;   // [B_r + 1]
  int32_t* n_tiles;  // [1]
  int32_t* perm;     // [B_c]
  int32_t* tiles;    // [3 * max_tiles]
};

__host__ __device__ inline int plan_max_tiles(int B_r, int B_c) { return (B_c + TQ - 1) / TQ + B_r + 1; }

__host__ inline PlanWs plan_carve(void* ws, int B_r, int B_c) {
  int32_t* p = reinterpret_cast<int32_t*>(ws);
  PlanWs w;
  w.cnt = p;
  p += B_r + 2;
  w.offs = p;
  p += B_r + 2;
  w.cursor = p;
  p += B_r + 1;
  w.n_tiles = p;
  p += 1;
  w.perm = p;
  p += B_c;
  w.tiles = p;
  return w;
}

__global__ void plan_clear(int32_t* cnt, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) cnt[i] = 0;
}

__global__ void plan_hist(const int32_t* cand2req, int B_c, int B_r, int32_t* cnt) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= B_c) return;
  int m = cand2req[i];
  if ((unsigned)m >= (unsigned)B_r) m = B_r;
  atomicAdd(&cnt[m], 1);
}

__global__ void plan_scatter(const int32_t* cand2req, int B_c, int B_r, int32_t* cursor, int32_t* perm) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= B_c) return;
  int m = cand2req[i];
  if ((unsigned)m >= (unsigned)B_r) m = B_r;
  perm[atomicAdd(&cursor[m], 1)] = i;
}

// The same counting sort with the counts privatized per workgroup in LDS
// (up to PLAN_LDS_BUCKETS buckets): one global atomic per (workgroup,
// bucket present) instead of one per candidate, which serializes hundreds of
// candidates of one request on one counter.  The order of a request's
// candidates within its bucket is the order the atomics happen to run in;
// the attention of one query does not depend on it.
constexpr int PLAN_IT = 4;                // candidates per thread
constexpr int PLAN_LDS_BUCKETS = 8000;    // B_r + 1 limit of the LDS path (the scatter holds 2 ints per bucket)

__global__ __launch_bounds__(256) void plan_hist_lds(const int32_t* cand2req, int B_c, int B_r, int32_t* cnt) {
  extern __shared__ int32_t h[];  // [B_r + 1]
  const int nb = B_r + 1;
  for (int b = threadIdx.x; b < nb; b += 256) h[b] = 0;
  __syncthreads();
  const int base = blockIdx.x * 256 * PLAN_IT;
#pragma unroll
  for (int k = 0; k < PLAN_IT; ++k) {
    const int i = base + k * 256 + threadIdx.x;
    if (i < B_c) {
      int m = cand2req[i];
      if ((unsigned)m >= (unsigned)B_r) m = B_r;
      atomicAdd(&h[m], 1);
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < nb; b += 256)
    if (h[b]) atomicAdd(&cnt[b], h[b]);
}

__global__ __launch_bounds__(256) void plan_scatter_lds(const int32_t* cand2req, int B_c, int B_r, int32_t* cursor,
                                                        int32_t* perm) {
  extern __shared__ int32_t h[];  // [B_r + 1] local counts, then local cursors; [B_r + 1] bases
  const int nb = B_r + 1;
  int32_t* first = h + nb;
  for (int b = threadIdx.x; b < nb; b += 256) h[b] = 0;
  __syncthreads();
  const int base = blockIdx.x * 256 * PLAN_IT;
  int mk[PLAN_IT];
#pragma unroll
  for (int k = 0; k < PLAN_IT; ++k) {
    const int i = base + k * 256 + threadIdx.x;
    mk[k] = -1;
    if (i < B_c) {
      int m = cand2req[i];
      if ((unsigned)m >= (unsigned)B_r) m = B_r;
      mk[k] = m;
      atomicAdd(&h[m], 1);
    }
  }
  __syncthreads();
  // reserve this workgroup's range in every bucket it touches
  for (int b = threadIdx.x; b < nb; b += 256) {
    if (h[b]) first[b] = atomicAdd(&cursor[b], h[b]);
    h[b] = 0;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < PLAN_IT; ++k)
    if (mk[k] >= 0) perm[first[mk[k]] + atomicAdd(&h[mk[k]], 1)] = base + k * 256 + threadIdx.x;
}

// Single workgroup: prefix sums over requests and the tile table.
// offsets_in (nullable): contiguous batch; otherwise counts in cnt.
__global__ __launch_bounds__(1024) void plan_tiles(const int32_t* offsets_in, int B_r, int B_c, PlanWs w) {
  __shared__ int32_t part[1024];
  __shared__ int32_t tpart[1024];
  const int nb = offsets_in ? B_r : B_r + 1;  // buckets
  const int t = threadIdx.x;
  const int per = (nb + 1023) / 1024;
  const int b0 = min(t * per, nb), b1 = min(b0 + per, nb);
  const int max_tiles = plan_max_tiles(B_r, B_c);
  // Row range of bucket b, clamped to [0, B_c] so that inconsistent offsets
  // can never address rows or tiles outside the buffers.
  auto range = [&](int b, int& beg, int& n) {
    if (offsets_in) {
      beg = min(max(offsets_in[b], 0), B_c);
      n = min(max(offsets_in[b + 1], beg), B_c) - beg;
    } else {
      beg = 0;
      n = w.cnt[b];
    }
  };
  int s = 0, ts = 0;
  for (int b = b0; b < b1; ++b) {
    int beg, n;
    range(b, beg, n);
    s += n;
    ts += (n + TQ - 1) / TQ;
  }
  part[t] = s;
  tpart[t] = ts;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int a = t >= o ? part[t - o] : 0;
    const int b = t >= o ? tpart[t - o] : 0;
    __syncthreads();
    part[t] += a;
    tpart[t] += b;
    __syncthreads();
  }
  int run = part[t] - s, trun = tpart[t] - ts;
  for (int b = b0; b < b1; ++b) {
    int beg, n;
    range(b, beg, n);
    if (!offsets_in) beg = run;
    w.offs[b] = beg;
    w.cursor[b] = beg;
    const int nt = (n + TQ - 1) / TQ;
    for (int k = 0; k < nt && trun + k < max_tiles; ++k) {
      w.tiles[3 * (trun + k) + 0] = b;
      w.tiles[3 * (trun + k) + 1] = beg + k * TQ;
      w.tiles[3 * (trun + k) + 2] = min(beg + (k + 1) * TQ, beg + n);
    }
    run += n;
    trun += nt;
  }
  if (t == 1023) {
    w.offs[nb] = part[1023];
    w.n_tiles[0] = min(tpart[1023], max_tiles);
  }
}

}  // namespace

int attn_tile_rows() { return TQ; }

size_t attn_plan_ws_bytes(int B_r, int B_c) {
  const size_t ints = size_t(B_r + 2) * 2 + size_t(B_r + 1) + 1 + size_t(B_c) + 3 * size_t(plan_max_tiles(B_r, B_c));
  return ints * sizeof(int32_t) + 256;
}

hipError_t launch_attn_plan(int B_r, int B_c, const int32_t* offsets, const int32_t* cand2req, void* ws,
                            int32_t** tile_info, int32_t** n_tiles, int32_t** perm, int* max_tiles, hipStream_t s) {
  PlanWs w = plan_carve(ws, B_r, B_c);
  *tile_info = w.tiles;
  *n_tiles = w.n_tiles;
  *max_tiles = plan_max_tiles(B_r, B_c);
  if (offsets) {
    *perm = nullptr;
    hipLaunchKernelGGL(plan_tiles, dim3(1), dim3(1024), 0, s, offsets, B_r, B_c, w);
    return hipGetLastError();
  }
  *perm = w.perm;
  const bool lds = B_r + 1 <= PLAN_LDS_BUCKETS;
  const int g = (B_c + 256 * PLAN_IT - 1) / (256 * PLAN_IT);
  const size_t hb = size_t(B_r + 1) * sizeof(int32_t);
  hipLaunchKernelGGL(plan_clear, dim3((B_r + 2 + 255) / 256), dim3(256), 0, s, w.cnt, B_r + 2);
  if (B_c > 0) {
    if (lds)
      hipLaunchKernelGGL(plan_hist_lds, dim3(g), dim3(256), hb, s, cand2req, B_c, B_r, w.cnt);
    else
      hipLaunchKernelGGL(plan_hist, dim3((B_c + 255) / 256), dim3(256), 0, s, cand2req, B_c, B_r, w.cnt);
  }
  hipLaunchKernelGGL(plan_tiles, dim3(1), dim3(1024), 0, s, nullptr, B_r, B_c, w);
  if (B_c > 0) {
    if (lds)
      hipLaunchKernelGGL(plan_scatter_lds, dim3(g), dim3(256), 2 * hb, s, cand2req, B_c, B_r, w.cursor, w.perm);
    else
      hipLaunchKernelGGL(plan_scatter, dim3((B_c + 255) / 256), dim3(256), 0, s, cand2req, B_c, B_r, w.cursor,
                         w.perm);
  }
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  int tiles = a.q_rows_per_group > 0 ? a.n_groups * ((a.q_rows_per_group + TQ - 1) / TQ) : a.max_tiles;
  if (tiles <= 0 || a.n_heads <= 0) return hipSuccess;
  if (a.L <= 0) return hipErrorInvalidValue;
  // the kernel addresses 64 key rows by 32-bit byte offsets
  if (a.ldkv >= kMaxAttnLdkv) return hipErrorInvalidValue;
  const int total = tiles * a.n_heads;
  int round = 3 * device_cus() / 8 * 8;  // three workgroups per CU, a multiple of the 8 XCDs
  // For tests of the pair walk at small sizes: ROCS_TEST_ATTN_ROUND=n sets a
  // round of n workgroups (rounded down to a multiple of 8).
  if (a.persistent)
    if (const char* e = std::getenv("ROCS_TEST_ATTN_ROUND")) {
      const int n = std::atoi(e) / 8 * 8;
      if (n >= 8) round = n;
    }
  if (a.persistent && total > round && round >= 8)
    hipLaunchKernelGGL(attn_persist_kernel, dim3(round), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attn_dma_kernel, dim3(total), dim3(256), 0, s, a);
  return hipGetLastError();
}


}  // namespace rocs
