// Grouped attention for DCA ([R] §2.2 grouped cross-attention; [R] §2.4
// IKBO-DCA): keys/values stay at request-batch size and every query tile is
// made of queries of ONE request, so each staged key/value tile in LDS is
// shared by all the queries of the workgroup, and the tiles of one request
// run back to back on one XCD (shared L2).  The same kernels run the
// request-only encoder's self-attention (group = one request's sequence).
//
// Per workgroup: 4 waves x 32 queries = 128 queries of one group and one
// head (head_dim 64).  Keys stream in 64-key slabs through LDS (K row-major,
// V transposed).  Each wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16, so each lane holds scores of a single query:
// the online-softmax max/sum need one exchange between lanes l and l ^ 32
// per slab (v_permlane32_swap).  P^T is fed back as the B operand of
// O^T = V^T P^T in the register order the S^T accumulator produced (the key
// order inside one MFMA k-step only has to agree between the two operands;
// the V^T rows are stored in that order).  Softmax in fp32 with exp2 and the
// scale folded into one multiply-add; the running maximum is only moved when
// a score exceeds it by more than 2^8 in exp2 units (lazy rescaling).
//
// With V^T staged once per call (vtrans_kernel), attn_vt_kernel feeds K and
// V^T slabs by LDS DMA through a 3-stage ring (two slabs in flight); without
// it, attn_kernel stages through registers and transposes V into LDS.
#include "rocs_device.h"

namespace rocs {

namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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
// c ^ swz(r).  A fragment read (32 consecutive rows, one chunk column) then
// hits distinct banks in every group of 16 lanes (256 B of banks per clock),
// and in every group of 8.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// K tile: [64 keys][64 dh] bf16.
__device__ __forceinline__ int k_off(int key, int chunk) { return key * 8 + (chunk ^ swz(key)); }
// V^T tile: [64 dh][64 keys] bf16.  Inside a row the keys sit in the order
// the PV step consumes them: position = key with bits 2 and 3 exchanged, so
// the 8 keys one lane feeds to one MFMA k-step (two runs of 4 keys, 8 apart)
// are one 16-byte chunk.
__device__ __forceinline__ int vt_pos(int key) { return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1); }
__device__ __forceinline__ int vt_chunk(int dh, int chunk) { return dh * 8 + (chunk ^ swz(dh)); }

// Query tile of one workgroup: group (request / sequence), rows [rbeg, rend)
// of the query batch, head h.  Returns false when the workgroup has no tile.
struct QTile {
  int group, rbeg, rend, h;
};
__device__ __forceinline__ bool decode_tile(const AttnArgs& a, QTile& t) {
  const int H = a.n_heads;
  int n_tiles;
  if (a.q_rows_per_group > 0)
    n_tiles = a.n_groups * ((a.q_rows_per_group + TQ - 1) / TQ);
  else
    n_tiles = *a.n_tiles_dev;
  const int total = (a.q_rows_per_group > 0 ? n_tiles : a.max_tiles) * H;
  const int logical = xcd_remap(blockIdx.x, total);
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
  float m_run, l_run;
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
  st.m_run = -INFINITY;
  st.l_run = 0.f;
}

// max / sum of x over lanes l and l ^ 32 (v_permlane32_swap gives every lane
// both values: a VALU exchange, no LDS round trip).
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One 64-key slab for the wave's 32 queries: S^T = K Q^T, online softmax,
// O^T += V^T P^T.  tK: [64 keys][8 chunks] (k_off), tV: [64 dh][8 chunks]
// (vt_chunk, keys in vt_pos order); key0 = first key of the slab.
__device__ __forceinline__ void attend_slab(const uint4* tK, const uint4* tV, int key0, int L, float c, int lane,
                                            QState& st) {
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
      for (int sp = 0; sp < 2; ++sp) vf[dt * 4 + kt * 2 + sp] = tV[vt_chunk(dt * 32 + (lane & 31), 4 * kt + 2 * sp + hl)];
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
    st.l_run *= alpha;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) st.o_acc[t][j] *= alpha;
    st.m_run = m_new;
  }
  const float mc = st.m_run * c;
  float psum = 0.f;
  bf16x8 pf[4];  // B operand for the PV step: [kt*2 + step]
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
#pragma unroll
      for (int q = 0; q < 8; ++q) pf[kt * 2 + sp][q] = to_bf(__builtin_amdgcn_exp2f(fmaf(s[kt][sp * 8 + q], c, -mc)));
      // l sums the bf16 P the PV product uses, two at a time (v_dot2_f32_bf16 with ones)
#pragma unroll
      for (int q = 0; q < 8; q += 2) {
        const bf16x2 pp = {pf[kt * 2 + sp][q], pf[kt * 2 + sp][q + 1]};
        psum = __builtin_amdgcn_fdot2_f32_bf16(pp, bf16x2{to_bf(1.f), to_bf(1.f)}, psum, false);
      }
    }
  psum = halves_sum(psum);
  st.l_run += psum;

  // O^T[dh][query] += V^T[dh][keys] P^T[keys][query]
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int sp = 0; sp < 2; ++sp)
        st.o_acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf[dt * 4 + kt * 2 + sp]),
                                                               pf[kt * 2 + sp], st.o_acc[dt], 0, 0, 0);
}

__device__ __forceinline__ void write_out(const AttnArgs& a, int64_t q_phys, int h, int hl, const QState& st) {
  const float inv = 1.0f / st.l_run;
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

// V read row-major from the K/V rows and transposed into LDS on the way in
// (register-staged, one slab ahead).
__global__ __launch_bounds__(256, 3) void attn_kernel(AttnArgs a) {
  __shared__ uint4 sK[2][KC * 8];
  __shared__ uint4 sV[2][DH * 8];
  QTile t;
  if (!decode_tile(a, t)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hl = lane >> 5;
  const int q_local = t.rbeg + wave * 32 + (lane & 31);
  const bool q_ok = q_local < t.rend;
  const int64_t q_phys = q_ok ? (a.perm ? a.perm[q_local] : q_local) : 0;
  if (t.group >= a.n_groups) {
    if (q_ok) write_nan_row(a, q_phys, t.h, hl);
    return;
  }
  QState st;
  load_q(a, q_phys, q_ok, t.h, hl, st);
  const bf16* kbase = a.k + int64_t(t.group) * a.kv_group_stride + t.h * DH;
  const bf16* vbase = a.v + int64_t(t.group) * a.kv_group_stride + t.h * DH;
  const int L = a.L;
  const int nslab = (L + KC - 1) / KC;

  // each thread stages 2 K chunks and 2 V chunks (16 B) per slab; keys past L
  // are zeros
  uint4 rk[2], rv[2];
  auto gload = [&](int slab) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int id = tid + i * 256;
      const int key = id >> 3, cc = id & 7;
      const int gk = slab * KC + key;
      rk[i] = gk < L ? *reinterpret_cast<const uint4*>(kbase + int64_t(gk) * a.ldkv + cc * 8) : make_uint4(0, 0, 0, 0);
      rv[i] = gk < L ? *reinterpret_cast<const uint4*>(vbase + int64_t(gk) * a.ldkv + cc * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int id = tid + i * 256;
      const int key = id >> 3, cc = id & 7;
      sK[buf][k_off(key, cc)] = rk[i];
      // transpose V: dh = cc*8 + e
      const uint16_t* e16 = reinterpret_cast<const uint16_t*>(&rv[i]);
      uint16_t* vt = reinterpret_cast<uint16_t*>(sV[buf]);
      const int pos = vt_pos(key);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dh = cc * 8 + e;
        vt[vt_chunk(dh, pos >> 3) * 8 + (pos & 7)] = e16[e];
      }
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int sb = 0; sb < nslab; ++sb) {
    const int cur = sb & 1;
    const bool more = sb + 1 < nslab;
    if (more) gload(sb + 1);
    attend_slab(sK[cur], sV[cur], sb * KC, L, a.scale_log2, lane, st);
    if (more) sstore(cur ^ 1);
    __syncthreads();
  }
  if (q_ok) write_out(a, q_phys, t.h, hl, st);
}

// V^T staged by vtrans_kernel (rows of keys in vt_pos order, zero-padded to
// a multiple of 64).  K and V^T slabs move global -> LDS by DMA
// (global_load_lds_dwordx4) through a ring of NST stages, so two slabs are in
// flight while one is consumed and no registers hold staged data.  Each wave
// fills 2 of the 8 1-KB pieces of each tile; lane i fetches the 16-byte
// chunk that the row swizzle places at its LDS slot.
constexpr int NST = 3;
constexpr int DMA_PER_SLAB = 4;  // wave-instructions per slab per wave (2 K + 2 V)

__global__ __launch_bounds__(256, 3) void attn_vt_kernel(AttnArgs a) {
  __shared__ uint4 sK[NST][KC * 8];
  __shared__ uint4 sV[NST][DH * 8];
  QTile t;
  if (!decode_tile(a, t)) return;
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
  // row; swz(r) = (lane/8) ^ j.
  const int row0 = wave * 16 + (lane >> 3);  // j = 0; j = 1 adds 8
  const int chunk0 = (lane & 7) ^ ((lane >> 3) & 7);
  const bf16* kbase = a.k + int64_t(t.group) * a.kv_group_stride + t.h * DH;
  const bf16* vsrc = a.vt + ((int64_t(t.group) * a.n_heads + t.h) * DH + row0) * a.ldvt;
  const int64_t vstep = 8 * a.ldvt;
  auto issue = [&](int slab, int stage) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // keys past L read row L-1: their scores are masked and their P is 0
      const int key = min(slab * KC + row0 + 8 * j, L - 1);
      dma16(kbase + int64_t(key) * a.ldkv + (chunk0 ^ j) * 8, &sK[stage][(2 * wave + j) * 64]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
      dma16(vsrc + j * vstep + slab * KC + (chunk0 ^ j) * 8, &sV[stage][(2 * wave + j) * 64]);
  };

  // Every step issues one slab (the last one again once past the end), so
  // "this wave's DMA for slab sb has landed" is always vmcnt <= one slab.
  issue(0, 0);
  issue(min(1, nslab - 1), 1);
  QState st;
  load_q(a, q_phys, q_ok, t.h, hl, st);
  // The compiler does not see the DMA on the load counter: make it wait for
  // the Q fragments here, once, rather than inside the loop at their first use.
  asm volatile("" : : "v"(st.qf[0]), "v"(st.qf[1]), "v"(st.qf[2]), "v"(st.qf[3]));
  int cur = 0, nxt = 2;
  for (int sb = 0; sb < nslab; ++sb) {
    wait_vmcnt<DMA_PER_SLAB>();
    __syncthreads();  // slab sb is in LDS for all waves; stage nxt (slab sb-1) is free
    issue(min(sb + 2, nslab - 1), nxt);
    attend_slab(sK[cur], sV[cur], sb * KC, L, a.scale_log2, lane, st);
    cur = cur == NST - 1 ? 0 : cur + 1;
    nxt = nxt == NST - 1 ? 0 : nxt + 1;
  }
  wait_vmcnt<0>();  // no DMA may still write this workgroup's LDS when it exits
  if (q_ok) write_out(a, q_phys, t.h, hl, st);
}

// ----------------------------------------------------------------- V^T staging
// The PV product takes V^T (keys contiguous per head dimension) as its A
// operand.  Transposed once per call here (one 64-key block of one head of
// one sequence per workgroup), every query tile then loads V^T rows with
// 16-byte loads instead of transposing the same V in LDS again.
__global__ __launch_bounds__(256) void vtrans_kernel(const bf16* __restrict__ v, int64_t ldv, int64_t gstride, int L,
                                                     int H, int64_t Lp, bf16* __restrict__ vt) {
  __shared__ uint16_t t[KC][DH + 2];  // [key][e]
  const int kb = blockIdx.x, h = blockIdx.y, g = blockIdx.z;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int id = tid + i * 256;
    const int key = id >> 3, c = id & 7;
    const int gk = kb * KC + key;
    const uint4 u = gk < L ? *reinterpret_cast<const uint4*>(v + g * gstride + int64_t(gk) * ldv + h * DH + c * 8)
                           : make_uint4(0, 0, 0, 0);
    const uint16_t* e16 = reinterpret_cast<const uint16_t*>(&u);
#pragma unroll
    for (int e = 0; e < 8; ++e) t[key][c * 8 + e] = e16[e];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int id = tid + i * 256;
    const int e = id >> 3, c = id & 7;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = uint32_t(t[vt_pos(c * 8 + 2 * j)][e]) | (uint32_t(t[vt_pos(c * 8 + 2 * j + 1)][e]) << 16);
    *reinterpret_cast<uint4*>(vt + ((int64_t(g) * H + h) * DH + e) * Lp + kb * KC + c * 8) =
        make_uint4(w[0], w[1], w[2], w[3]);
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
  if (a.vt != nullptr)
    hipLaunchKernelGGL(attn_vt_kernel, dim3(tiles * a.n_heads), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attn_kernel, dim3(tiles * a.n_heads), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_vtrans(const bf16* v, int64_t ldv, int64_t gstride, int G, int H, int L, bf16* vt, hipStream_t s) {
  if (G <= 0 || H <= 0 || L <= 0) return hipSuccess;
  const int64_t Lp = vt_pad(L);
  hipLaunchKernelGGL(vtrans_kernel, dim3(unsigned(Lp / KC), unsigned(H), unsigned(G)), dim3(256), 0, s, v, ldv,
                     gstride, L, H, Lp, vt);
  return hipGetLastError();
}

}  // namespace rocs
