// Grouped attention for DCA ([R] §2.2 grouped cross-attention; [R] §2.4
// IKBO-DCA): keys/values stay at request-batch size and every query tile is
// made of queries of ONE request, so each staged key/value tile in LDS is
// shared by all the queries of the workgroup, and the tiles of one request
// run back to back on one XCD (shared L2).  The same kernel runs the
// request-only encoder's self-attention (group = one request's sequence).
//
// Per workgroup: 4 waves x 32 queries = 128 queries of one group and one
// head (head_dim 64).  Keys stream in 64-key slabs through double-buffered
// LDS (K row-major, V transposed).  Each wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16, so each lane holds scores of a single query:
// the online-softmax max/sum need one cross-lane exchange (lane ^ 32) per
// slab.  P^T is fed back as the B operand of O^T = V^T P^T in the register
// order the S^T accumulator produced (the key order inside one MFMA k-step
// only has to agree between the two operands).  Softmax in fp32 with exp2
// and the scale folded into one multiply-add.
#include "rocs_device.h"

namespace rocs {

namespace {

constexpr int TQ = 128;  // queries per workgroup
constexpr int KC = 64;   // keys per slab
constexpr int DH = 64;   // head dim

// K tile: [64 keys][64 dh] bf16, 16-byte chunks swizzled by key.
__device__ __forceinline__ int k_off(int key, int chunk) { return key * 8 + (chunk ^ (key & 7)); }
// V^T tile: [64 dh][64 keys] bf16 in 8-byte units (16 per row), swizzled by dh.
__device__ __forceinline__ int vt_off(int dh, int unit) { return dh * 16 + (unit ^ (dh & 15)); }

template <bool VT>
__global__ __launch_bounds__(256, 3) void attn_kernel(AttnArgs a) {
  __shared__ uint4 sK[2][KC * 8];
  __shared__ uint2 sV[2][DH * 16];

  const int H = a.n_heads;
  int n_tiles;
  if (a.q_rows_per_group > 0)
    n_tiles = a.n_groups * ((a.q_rows_per_group + TQ - 1) / TQ);
  else
    n_tiles = *a.n_tiles_dev;
  const int total = (a.q_rows_per_group > 0 ? n_tiles : a.max_tiles) * H;
  const int logical = xcd_remap(blockIdx.x, total);
  const int tile = logical / H;
  const int h = logical - tile * H;
  if (tile >= n_tiles) return;

  int group, rbeg, rend;
  if (a.q_rows_per_group > 0) {
    const int tpg = (a.q_rows_per_group + TQ - 1) / TQ;
    group = tile / tpg;
    rbeg = group * a.q_rows_per_group + (tile - group * tpg) * TQ;
    rend = min(rbeg + TQ, (group + 1) * a.q_rows_per_group);
  } else {
    group = a.tile_info[3 * tile + 0];
    rbeg = a.tile_info[3 * tile + 1];
    rend = a.tile_info[3 * tile + 2];
  }

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5;  // half of the wave
  const int q_local = rbeg + wave * 32 + (lane & 31);
  const bool q_ok = q_local < rend;
  const int64_t q_phys = q_ok ? (a.perm ? a.perm[q_local] : q_local) : 0;

  if (group >= a.n_groups) {  // candidates whose request id was out of range
    if (q_ok) {
      bf16* o = a.o + q_phys * a.ldo + h * DH;
      for (int e = hl * 32; e < hl * 32 + 32; ++e) o[e] = to_bf(nan_f());
    }
    return;
  }

  // Q^T fragments (B operand): lane holds query q_local, dh 16*ks + 8*hl + 0..7
  bf16x8 qf[4];
  {
    const bf16* qp = a.q + q_phys * a.ldq + h * DH;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (q_ok) u = *reinterpret_cast<const uint4*>(qp + ks * 16 + hl * 8);
      qf[ks] = __builtin_bit_cast(bf16x8, u);
    }
  }

  const bf16* kbase = a.k + int64_t(group) * a.kv_group_stride + h * DH;
  const bf16* vbase = a.v + int64_t(group) * a.kv_group_stride + h * DH;
  const bf16* vtbase = VT ? a.vt + (int64_t(group) * H + h) * DH * a.ldvt : nullptr;
  const int L = a.L;
  const int nslab = (L + KC - 1) / KC;

  // each thread stages 2 K chunks and 2 V chunks (16 B) per slab
  uint4 rk[2], rv[2];
  auto gload = [&](int slab) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int id = tid + i * 256;
      const int key = id >> 3, c = id & 7;
      const int gk = slab * KC + key;
      rk[i] = gk < L ? *reinterpret_cast<const uint4*>(kbase + int64_t(gk) * a.ldkv + c * 8) : make_uint4(0, 0, 0, 0);
      if constexpr (VT) {
        // V^T row dh = id / 8, keys slab*64 + 8c .. +7 (padded with zeros up to ldvt)
        rv[i] = *reinterpret_cast<const uint4*>(vtbase + int64_t(key) * a.ldvt + slab * KC + c * 8);
      } else {
        rv[i] = gk < L ? *reinterpret_cast<const uint4*>(vbase + int64_t(gk) * a.ldkv + c * 8) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int id = tid + i * 256;
      const int key = id >> 3, c = id & 7;
      sK[buf][k_off(key, c)] = rk[i];
      if constexpr (VT) {
        // already transposed: row dh = id / 8 holds keys 8c .. 8c+7 = units 2c, 2c+1
        sV[buf][vt_off(key, 2 * c)] = make_uint2(rv[i].x, rv[i].y);
        sV[buf][vt_off(key, 2 * c + 1)] = make_uint2(rv[i].z, rv[i].w);
      } else {
        // transpose V: dh = c*8 + e, key -> unit key/4, lane-in-unit key%4
        const uint16_t* e16 = reinterpret_cast<const uint16_t*>(&rv[i]);
        uint16_t* vt = reinterpret_cast<uint16_t*>(sV[buf]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int dh = c * 8 + e;
          vt[vt_off(dh, key >> 2) * 4 + (key & 3)] = e16[e];
        }
      }
    }
  };

  f32x16 o_acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < 16; ++j) o_acc[t][j] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.scale_log2;

  gload(0);
  sstore(0);
  __syncthreads();

  for (int sb = 0; sb < nslab; ++sb) {
    const int cur = sb & 1;
    const bool more = sb + 1 < nslab;
    if (more) gload(sb + 1);

    // S^T tiles: keys kt*32 + row, queries = lane columns
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int j = 0; j < 16; ++j) s[kt][j] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 u = sK[cur][k_off(kt * 32 + (lane & 31), ks * 2 + hl)];
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u), qf[ks], s[kt], 0, 0, 0);
      }
    }
    // mask keys beyond L (last slab only)
    if ((sb + 1) * KC > L) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = sb * KC + kt * 32 + 8 * (j >> 2) + 4 * hl + (j & 3);
          if (key >= L) s[kt][j] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kt][j]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);  // v_exp_f32
    const float mc = m_new * c;
    float psum = 0.f;
    bf16x8 pf[4];  // B operand for the PV step: [kt*2 + step]
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][st * 8 + q], c, -mc));
          psum += p;
          pf[kt * 2 + st][q] = to_bf(p);
        }
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) o_acc[t][j] *= alpha;

    // O^T[dh][query] += V^T[dh][keys] P^T[keys][query]
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const int dh = dt * 32 + (lane & 31);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          // keys kt*32 + 16*st + 8*(q/4) + 4*hl + q%4 -> 8-byte units
          const int u0 = (kt * 32 + 16 * st + 4 * hl) >> 2;
          const uint2 lo = sV[cur][vt_off(dh, u0)];
          const uint2 hi = sV[cur][vt_off(dh, u0 + 2)];
          const uint4 vv = make_uint4(lo.x, lo.y, hi.x, hi.y);
          o_acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pf[kt * 2 + st],
                                                              o_acc[dt], 0, 0, 0);
        }
    }
    if (more) sstore(cur ^ 1);
    __syncthreads();
  }

  if (!q_ok) return;
  const float inv = 1.0f / l_run;
  bf16* o = a.o + q_phys * a.ldo + h * DH;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // registers 4g..4g+3 hold dh = dt*32 + 8g + 4*hl + 0..3
      bf16x4 pk = {to_bf(o_acc[dt][4 * g + 0] * inv), to_bf(o_acc[dt][4 * g + 1] * inv),
                   to_bf(o_acc[dt][4 * g + 2] * inv), to_bf(o_acc[dt][4 * g + 3] * inv)};
      *reinterpret_cast<bf16x4*>(o + dt * 32 + 8 * g + 4 * hl) = pk;
    }
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
    for (int j = 0; j < 4; ++j) w[j] = uint32_t(t[c * 8 + 2 * j][e]) | (uint32_t(t[c * 8 + 2 * j + 1][e]) << 16);
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
  hipLaunchKernelGGL(plan_clear, dim3((B_r + 2 + 255) / 256), dim3(256), 0, s, w.cnt, B_r + 2);
  if (B_c > 0) hipLaunchKernelGGL(plan_hist, dim3((B_c + 255) / 256), dim3(256), 0, s, cand2req, B_c, B_r, w.cnt);
  hipLaunchKernelGGL(plan_tiles, dim3(1), dim3(1024), 0, s, nullptr, B_r, B_c, w);
  if (B_c > 0)
    hipLaunchKernelGGL(plan_scatter, dim3((B_c + 255) / 256), dim3(256), 0, s, cand2req, B_c, B_r, w.cursor,
                       w.perm);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  int tiles = a.q_rows_per_group > 0 ? a.n_groups * ((a.q_rows_per_group + TQ - 1) / TQ) : a.max_tiles;
  if (tiles <= 0 || a.n_heads <= 0) return hipSuccess;
  if (a.vt != nullptr)
    hipLaunchKernelGGL(attn_kernel<true>, dim3(tiles * a.n_heads), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attn_kernel<false>, dim3(tiles * a.n_heads), dim3(256), 0, s, a);
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
