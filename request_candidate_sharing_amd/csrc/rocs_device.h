// Device-side helpers shared by the librocs kernels (gfx950).
#pragma once

#include "rocs_internal.h"

namespace rocs {

__device__ __forceinline__ float to_f(bf16 h) { return (float)h; }
__device__ __forceinline__ float to_f(float h) { return h; }
__device__ __forceinline__ bf16 to_bf(float f) { return (bf16)f; }  // v_cvt_pk_bf16_f32, round to nearest even

template <typename T>
__device__ __forceinline__ T from_f(float f);
template <>
__device__ __forceinline__ float from_f<float>(float f) { return f; }
template <>
__device__ __forceinline__ bf16 from_f<bf16>(float f) { return to_bf(f); }

__device__ __forceinline__ float nan_f() { return __builtin_nanf(""); }

// Workgroups are dispatched round-robin over the 8 XCDs (wg i -> XCD i % 8).
// Remap so that each XCD receives one contiguous range of logical tile ids:
// neighbouring tiles (which share operand panels) then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
  const int q = nwg >> 3, r = nwg & 7;
  const int x = wg & 7, i = wg >> 3;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// Wave-wide sum (64 lanes) with a fixed butterfly order: every lane ends with
// the same, run-to-run deterministic value.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace rocs
