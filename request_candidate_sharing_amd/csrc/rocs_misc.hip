// Group-local norms, the scalar score head, the explicit broadcast used by
// the dense-broadcast comparator, and batch validation.
#include <algorithm>
#include <type_traits>

#include "rocs_device.h"

namespace rocs {

namespace {

// ----------------------------------------------------------------- group-local norm
// [R] §2.1, Figure 2(b): statistics inside one group's slice of a row.  One
// wave per row, RPW consecutive rows per wave: every 16-byte load of the
// wave's rows (and residuals) is issued before any is used, so a wave keeps
// RPW x CH loads per lane in flight.  A row stays in registers between the
// statistics and the normalisation, so each element is read once and
// written once.  LayerNorm: two-pass mean / biased variance in fp32;
// RMSNorm: mean square.  One launch can normalize two independent row groups
// (the request and the candidate part of a stack layer): workgroups
// [0, nblk_a) take group pa, the rest group pb.
// RES: some group of the launch adds a residual (the other may not).
template <typename T, int CH, bool RES, int RPW>
__global__ __launch_bounds__(256) void norm_kernel(NormArgs pa, NormArgs pb, int nblk_a) {
  constexpr int VEC = 16 / sizeof(T);
  const bool second = int(blockIdx.x) >= nblk_a;
  const NormArgs a = second ? pb : pa;
  const int lane = threadIdx.x & 63;
  const int row0 = ((second ? int(blockIdx.x) - nblk_a : int(blockIdx.x)) * 4 + (threadIdx.x >> 6)) * RPW;
  if (row0 >= a.rows) return;
  // head weights of this lane's chunks (the same for every row)
  const T* hw = reinterpret_cast<const T*>(a.head_w);
  uint4 hwv[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int e0 = (c * 64 + lane) * VEC;
    hwv[c] = (hw && e0 + VEC <= a.width) ? *reinterpret_cast<const uint4*>(hw + e0) : make_uint4(0, 0, 0, 0);
  }
  // every chunk's loads of every row, issued before any is used (one uniform
  // branch around all of them: a lane whose vector is not whole in the row
  // loads the row's last whole vector instead and ignores it; rows narrower
  // than one vector take the element path below).  With RES the residual is
  // loaded unconditionally (from x when this group has none) and added by a
  // select, so no branch separates the loads.
  const bool has_r = RES && a.res != nullptr;
  const int64_t ldr = a.ldres ? a.ldres : a.ldx;
  const int last_vec = (a.width / VEC - 1) * VEC;
  uint4 xq[RPW][CH], rq[RPW][CH];
  float hz[RPW];
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int row = min(row0 + j, a.rows - 1);  // rows past the end repeat the last one and store nothing
    hz[j] = 0.f;
    if (a.head_w && a.head_z) {
      const int m = a.head_zmap ? a.head_zmap[row] : row;
      hz[j] = ((unsigned)m < (unsigned)a.head_zrows) ? a.head_z[m] : nan_f();
    }
    const T* x = reinterpret_cast<const T*>(a.x) + int64_t(row) * a.ldx;
    const T* rp = has_r ? reinterpret_cast<const T*>(a.res) + int64_t(row) * ldr : x;
#pragma unroll
    for (int c = 0; c < CH; ++c) xq[j][c] = rq[j][c] = make_uint4(0, 0, 0, 0);
    if (a.width >= VEC) {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int e0 = (c * 64 + lane) * VEC;
        const int el = e0 + VEC <= a.width ? e0 : last_vec;
        xq[j][c] = *reinterpret_cast<const uint4*>(x + el);
        if (RES) rq[j][c] = *reinterpret_cast<const uint4*>(rp + el);
      }
    }
  }
  // Each loaded value is consumed here, in order, after the last load was
  // issued: the compiler may not move a load down next to its use.
  if constexpr (CH * RPW > 1) {
#pragma unroll
    for (int j = 0; j < RPW; ++j)
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        asm volatile("" ::"v"(xq[j][c].x), "v"(xq[j][c].y), "v"(xq[j][c].z), "v"(xq[j][c].w) : "memory");
        if (RES) asm volatile("" ::"v"(rq[j][c].x), "v"(rq[j][c].y), "v"(rq[j][c].z), "v"(rq[j][c].w) : "memory");
      }
  }
  const T* g = reinterpret_cast<const T*>(a.gamma);
  const T* b = reinterpret_cast<const T*>(a.beta);
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int row = row0 + j;
    if (row >= a.rows) continue;  // uniform across the wave
    const T* x = reinterpret_cast<const T*>(a.x) + int64_t(row) * a.ldx;
    const T* r = a.res ? reinterpret_cast<const T*>(a.res) + int64_t(row) * ldr : nullptr;
    float v[CH][VEC];
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int e0 = (c * 64 + lane) * VEC;
#pragma unroll
      for (int k = 0; k < VEC; ++k) v[c][k] = 0.f;
      if (e0 + VEC <= a.width) {
        const T* t = reinterpret_cast<const T*>(&xq[j][c]);
#pragma unroll
        for (int k = 0; k < VEC; ++k) v[c][k] = to_f(t[k]);
        if (RES) {
          const T* tr = reinterpret_cast<const T*>(&rq[j][c]);
#pragma unroll
          for (int k = 0; k < VEC; ++k) v[c][k] = has_r ? v[c][k] + to_f(tr[k]) : v[c][k];
        }
      } else {
        for (int k = 0; k < VEC; ++k)
          if (e0 + k < a.width) v[c][k] = to_f(x[e0 + k]) + (r ? to_f(r[e0 + k]) : 0.f);
      }
#pragma unroll
      for (int k = 0; k < VEC; ++k) s += (a.kind == 0) ? v[c][k] : v[c][k] * v[c][k];
    }
    const float inv_w = 1.0f / float(a.width);
    float mean = 0.f, scale;
    if (a.kind == 0) {
      mean = wave_sum(s) * inv_w;
      float q = 0.f;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int e0 = (c * 64 + lane) * VEC;
#pragma unroll
        for (int k = 0; k < VEC; ++k)
          if (e0 + k < a.width) {
            const float dd = v[c][k] - mean;
            q += dd * dd;
          }
      }
      scale = 1.0f / sqrtf(wave_sum(q) * inv_w + a.eps);
    } else {
      scale = 1.0f / sqrtf(wave_sum(s) * inv_w + a.eps);
    }
    T* y = reinterpret_cast<T*>(a.y) + int64_t(row) * a.ldy;
    float hs = 0.f;  // fused head: the same chunks and order as rowdot_kernel
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int e0 = (c * 64 + lane) * VEC;
      if (e0 >= a.width) continue;
      // affine parameters of this chunk in 16-byte loads (gamma and beta are
      // 16-byte aligned); the ragged last chunk reads them element by element
      T gv[VEC], bv[VEC];
      if (e0 + VEC <= a.width) {
        if (g) *reinterpret_cast<uint4*>(gv) = *reinterpret_cast<const uint4*>(g + e0);
        if (b) *reinterpret_cast<uint4*>(bv) = *reinterpret_cast<const uint4*>(b + e0);
      } else {
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          const int e = min(e0 + k, a.width - 1);
          if (g) gv[k] = g[e];
          if (b) bv[k] = b[e];
        }
      }
      T out[VEC];
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        float t = (v[c][k] - mean) * scale;
        if (g) t *= to_f(gv[k]);
        if (b) t += to_f(bv[k]);
        if (a.act == 1) t = fmaxf(t, 0.f);
        out[k] = from_f<T>(t);
      }
      if (e0 + VEC <= a.width) {
        *reinterpret_cast<uint4*>(y + e0) = *reinterpret_cast<const uint4*>(out);
        if (hw) {
          const T* tw = reinterpret_cast<const T*>(&hwv[c]);
#pragma unroll
          for (int k = 0; k < VEC; ++k) hs = fmaf(to_f(out[k]), to_f(tw[k]), hs);
        }
      } else {
        for (int k = 0; k < VEC; ++k)
          if (e0 + k < a.width) y[e0 + k] = out[k];
        if (hw)
          for (int k = 0; k < VEC && e0 + k < a.width; ++k) hs = fmaf(to_f(out[k]), to_f(hw[e0 + k]), hs);
      }
    }
    if (hw) {
      hs = wave_sum(hs);
      if (lane == 0) {
        if (a.head_z) hs = hs + hz[j];  // NaN for a map entry out of range
        hs += a.head_bias;
        if (a.head_bias_dev) hs += to_f(reinterpret_cast<const T*>(a.head_bias_dev)[0]);
        a.head_out[row] = hs;
      }
    }
  }
}

// Rows per wave.  One: measured on the GLM MLP stack (512-wide rows, 74k of
// them) four rows per wave with all their loads in flight took 44 us against
// 36 us for one row per wave (more registers per wave, fewer waves in flight),
// and 12 vs 5 us for 256 rows.
template <int CH>
constexpr int norm_rpw() { return 1; }

template <typename T, bool RES>
hipError_t norm_launch(int ch, const NormArgs& a, const NormArgs& b, hipStream_t s) {
  const dim3 block(256);
  auto go = [&](auto chc) -> hipError_t {
    constexpr int CH = decltype(chc)::value;
    constexpr int RPW = norm_rpw<CH>();
    const int na = (a.rows + 4 * RPW - 1) / (4 * RPW);
    const dim3 grid(na + (b.rows + 4 * RPW - 1) / (4 * RPW));
    if (grid.x == 0) return hipSuccess;
    hipLaunchKernelGGL((norm_kernel<T, CH, RES, RPW>), grid, block, 0, s, a, b, na);
    return hipGetLastError();
  };
  switch (ch <= 1 ? 1 : ch <= 2 ? 2 : ch <= 3 ? 3 : ch <= 4 ? 4 : ch <= 8 ? 8 : ch <= 16 ? 16 : 0) {
    case 1: return go(std::integral_constant<int, 1>{});
    case 2: return go(std::integral_constant<int, 2>{});
    case 3: return go(std::integral_constant<int, 3>{});
    case 4: return go(std::integral_constant<int, 4>{});
    case 8: return go(std::integral_constant<int, 8>{});
    case 16: return go(std::integral_constant<int, 16>{});
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t norm_dispatch(const NormArgs& a, const NormArgs& b, hipStream_t s) {
  constexpr int VEC = 16 / sizeof(T);
  const int per = 64 * VEC;
  const int ch = std::max((a.width + per - 1) / per, (b.width + per - 1) / per);
  return (a.res || b.res) ? norm_launch<T, true>(ch, a, b, s) : norm_launch<T, false>(ch, a, b, s);
}

// ----------------------------------------------------------------- row dot (score head)
// out[i] = w . x[i] + z[map[i]] + bias, one wave per row, fixed reduction order.
template <typename T>
__global__ __launch_bounds__(256) void rowdot_kernel(DotArgs a) {
  constexpr int VEC = 16 / sizeof(T);
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const T* x = reinterpret_cast<const T*>(a.x) + int64_t(row) * a.ldx;
  const T* w = reinterpret_cast<const T*>(a.w);
  float s = 0.f;
  for (int e0 = lane * VEC; e0 < a.width; e0 += 64 * VEC) {
    if (e0 + VEC <= a.width) {
      const uint4 ux = *reinterpret_cast<const uint4*>(x + e0);
      const uint4 uw = *reinterpret_cast<const uint4*>(w + e0);
      const T* tx = reinterpret_cast<const T*>(&ux);
      const T* tw = reinterpret_cast<const T*>(&uw);
#pragma unroll
      for (int j = 0; j < VEC; ++j) s = fmaf(to_f(tx[j]), to_f(tw[j]), s);
    } else {
      for (int j = 0; j < VEC && e0 + j < a.width; ++j) s = fmaf(to_f(x[e0 + j]), to_f(w[e0 + j]), s);
    }
  }
  s = wave_sum(s);
  if (lane == 0) {
    if (a.z) {
      const int m = a.zmap ? a.zmap[row] : row;
      s = ((unsigned)m < (unsigned)a.zrows) ? s + a.z[m] : nan_f();
    }
    s += a.bias;
    if (a.bias_dev) s += to_f(reinterpret_cast<const T*>(a.bias_dev)[0]);
    a.out[row] = s;
  }
}

// ----------------------------------------------------------------- zero padding
// dst[r][c] = src[r][c] for c < w and 0 for w <= c < wpad (rows of es-byte
// elements, any strides).  With src == NULL only [w, wpad) is written (the
// zero tail after a view of width w).  Element by element: for weights,
// staged inputs and outputs of widths that break 16-byte rows.
template <typename E>
__global__ __launch_bounds__(256) void pad_rows_kernel(int64_t rows, int w, int wpad, const E* __restrict__ src,
                                                       int64_t lds, E* __restrict__ dst, int64_t ldd) {
  const int c0 = src ? 0 : w;
  const int span = wpad - c0;
  const int64_t total = rows * span;
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < total; e += int64_t(gridDim.x) * 256) {
    const int64_t r = e / span;
    const int c = c0 + int(e - r * span);
    dst[r * ldd + c] = c < w ? src[r * lds + c] : E(0);
  }
}

// ----------------------------------------------------------------- explicit broadcast
// dst[i] = src[map[i]] byte for byte; 16 bytes per thread.
__global__ __launch_bounds__(256) void bcast_kernel(int64_t rows, const int32_t* map, int map_rows, int64_t chunks,
                                                     const uint4* src, int64_t src_stride, uint4* dst,
                                                     int64_t dst_stride, int inner) {
  const int64_t total = rows * chunks;
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < total; e += int64_t(gridDim.x) * 256) {
    const int64_t r = e / chunks, c = e - r * chunks;
    const int64_t i = r / inner, l = r - i * inner;
    const int m = map ? map[i] : int(i);
    uint4 v = make_uint4(0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu);
    if ((unsigned)m < (unsigned)map_rows) v = src[(int64_t(m) * inner + l) * src_stride + c];
    dst[r * dst_stride + c] = v;
  }
}

// ----------------------------------------------------------------- batch validation
__device__ int g_batch_flag;

__global__ void clear_flag_kernel() { g_batch_flag = 0; }

__global__ __launch_bounds__(256) void validate_kernel(int B_r, int B_c, const int32_t* offsets,
                                                        const int32_t* cand2req) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < B_c) {
    const int m = cand2req[i];
    bool bad = (unsigned)m >= (unsigned)B_r;
    if (!bad && offsets) bad = !(offsets[m] <= i && i < offsets[m + 1]);
    if (bad) atomicOr(&g_batch_flag, 1);
  }
  if (offsets && i <= B_r) {
    bool bad = false;
    if (i == 0) bad = offsets[0] != 0;
    if (i == B_r) bad = bad || offsets[B_r] != B_c;
    if (i < B_r) bad = bad || offsets[i] > offsets[i + 1];
    if (bad) atomicOr(&g_batch_flag, 2);
  }
}

}  // namespace

hipError_t launch_norm(DType dt, const NormArgs& a, hipStream_t s) {
  if (a.rows <= 0 || a.width <= 0) return hipSuccess;
  const NormArgs none{};
  return dt == F32 ? norm_dispatch<float>(a, none, s) : norm_dispatch<bf16>(a, none, s);
}

hipError_t launch_norm2(DType dt, const NormArgs& a, const NormArgs& b, hipStream_t s) {
  const bool ua = a.rows > 0 && a.width > 0, ub = b.rows > 0 && b.width > 0;
  if (!ua || !ub) return ua ? launch_norm(dt, a, s) : launch_norm(dt, b, s);
  return dt == F32 ? norm_dispatch<float>(a, b, s) : norm_dispatch<bf16>(a, b, s);
}

hipError_t launch_rowdot(DType dt, const DotArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  const dim3 grid((a.rows + 3) / 4), block(256);
  if (dt == F32)
    hipLaunchKernelGGL(rowdot_kernel<float>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(rowdot_kernel<bf16>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_broadcast_rows(int rows, const int32_t* map, int map_rows, int64_t row_bytes, const void* src,
                                 int64_t src_stride, void* dst, int64_t dst_stride, hipStream_t s, int inner) {
  if (rows <= 0 || row_bytes <= 0 || inner <= 0) return hipSuccess;
  const int64_t chunks = row_bytes / 16;
  const int64_t all_rows = int64_t(rows) * inner;
  const int64_t total = all_rows * chunks;
  const int64_t want = (total + 255) / 256;
  const int grid = int(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(bcast_kernel, dim3(grid), dim3(256), 0, s, all_rows, map, map_rows, chunks,
                     reinterpret_cast<const uint4*>(src), src_stride / 16, reinterpret_cast<uint4*>(dst),
                     dst_stride / 16, inner);
  return hipGetLastError();
}

hipError_t launch_pad_rows(int64_t rows, int w, int wpad, int es, const void* src, int64_t lds, void* dst,
                           int64_t ldd, hipStream_t s) {
  const int64_t total = rows * (wpad - (src ? 0 : w));
  if (rows <= 0 || total <= 0) return hipSuccess;
  const int64_t g = std::min<int64_t>((total + 255) / 256, 8192);
  if (es == 2)
    hipLaunchKernelGGL(pad_rows_kernel<uint16_t>, dim3(unsigned(g)), dim3(256), 0, s, rows, w, wpad,
                       static_cast<const uint16_t*>(src), lds, static_cast<uint16_t*>(dst), ldd);
  else
    hipLaunchKernelGGL(pad_rows_kernel<uint32_t>, dim3(unsigned(g)), dim3(256), 0, s, rows, w, wpad,
                       static_cast<const uint32_t*>(src), lds, static_cast<uint32_t*>(dst), ldd);
  return hipGetLastError();
}

hipError_t launch_validate_batch(int B_r, int B_c, const int32_t* offsets, const int32_t* cand2req, int32_t* flag,
                                 hipStream_t s) {
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(1), 0, s);
  const int n = (B_c > B_r + 1 ? B_c : B_r + 1);
  hipLaunchKernelGGL(validate_kernel, dim3((n + 255) / 256), dim3(256), 0, s, B_r, B_c, offsets, cand2req);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbolAsync(flag, HIP_SYMBOL(g_batch_flag), sizeof(int32_t), 0, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(s);
}

}  // namespace rocs
