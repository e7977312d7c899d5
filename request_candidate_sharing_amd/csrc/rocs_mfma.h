// MFMA tile building blocks shared by the GEMM and the fused MLP kernels.
//
// LDS operand tiles hold rows of one K slab of bf16 in 16-byte chunks
// (CPR = chunks per row: 8 for a 64-wide slab, 16 for a 128-wide slab).
// Chunk c of row r is stored at chunk position c ^ swz(r): fragment reads
// (32 rows of one chunk column) are conflict-free for both 8-lane (128 B)
// and 16-lane (256 B) LDS service widths.
//
// K order of every bf16 MFMA product in this library: K is consumed in
// 64-wide groups in ascending order; inside a group, k16 step s (0..3) has
// lane half hk supply K elements 32*hk + 8*s .. +7.  All kernels follow it,
// so each output element sums the same 16 k-values per MFMA in the same
// step order whichever kernel computes it (bit-identical results).
#pragma once

#include "rocs_device.h"

namespace rocs {

template <int CPR>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CPR == 16)
    return r & 15;
  else if constexpr (CPR == 8)
    return (r & 7) ^ ((r >> 3) & 1);
  else
    return ((r >> 1) ^ (r >> 3)) & 3;  // 4 chunks per row
}
template <int CPR>
__device__ __forceinline__ int slot(int r, int chunk) {
  return r * CPR + (chunk ^ swz<CPR>(r));
}

// LDS chunk of k16 step ks (counted from the slab start) for lane half hk.
__device__ __forceinline__ int kchunk(int ks, int hk) { return (ks >> 2) * 8 + hk * 4 + (ks & 3); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One wave-instruction of global -> LDS DMA: lane i's 16 bytes land at
// dst + 16*i (dst wave-uniform).
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)dst, 16, 0, 0);
}
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

template <int FM, int FN>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[FM][FN]) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
}

// KS k16 steps over LDS operand tiles: A operand rows ar0 + 32j (j < FN) in a
// tile with CPRA chunks per row, B operand rows br0 + 32i (i < FM) with CPRB
// chunks per row; kc0 is the chunk offset of the slab's first k16 group in
// the B tile (for B tiles that hold more K than one slab).  Fragments of step
// ks+1 are read while the MFMAs of step ks issue.
template <int FM, int FN, int KS, int CPRA, int CPRB>
__device__ __forceinline__ void mfma_steps(const uint4* sa, int ar0, const uint4* sb, int br0, int kc0, int hk,
                                           f32x16 (&acc)[FM][FN]) {
  bf16x8 af[2][FN], bfr[2][FM];
  auto frag = [&](int ks, int buf) {
    const int ch = kchunk(ks, hk);
#pragma unroll
    for (int j = 0; j < FN; ++j) af[buf][j] = __builtin_bit_cast(bf16x8, sa[slot<CPRA>(ar0 + j * 32, ch)]);
#pragma unroll
    for (int i = 0; i < FM; ++i) bfr[buf][i] = __builtin_bit_cast(bf16x8, sb[slot<CPRB>(br0 + i * 32, kc0 + ch)]);
  };
  frag(0, 0);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (ks + 1 < KS) frag(ks + 1, (ks + 1) & 1);
    // Keep the next step's LDS reads ahead of this step's MFMAs: left alone,
    // the scheduler sinks each read next to its first use, which exposes the
    // LDS latency at every step.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][j], bfr[ks & 1][i], acc[i][j], 0, 0, 0);
  }
}

// Fragment registers of one wave, double-buffered by k16 step parity.
template <int FM, int FN>
struct Frags {
  bf16x8 a[2][FN], b[2][FM];
};

template <int FM, int FN, int CPRA, int CPRB>
__device__ __forceinline__ void load_frags(Frags<FM, FN>& f, int buf, const uint4* sa, int ar0, const uint4* sb,
                                           int br0, int ch) {
#pragma unroll
  for (int j = 0; j < FN; ++j) f.a[buf][j] = __builtin_bit_cast(bf16x8, sa[slot<CPRA>(ar0 + j * 32, ch)]);
#pragma unroll
  for (int i = 0; i < FM; ++i) f.b[buf][i] = __builtin_bit_cast(bf16x8, sb[slot<CPRB>(br0 + i * 32, ch)]);
}

template <int FM, int FN>
__device__ __forceinline__ void mfma_frags(const Frags<FM, FN>& f, int buf, f32x16 (&acc)[FM][FN], int from = 0) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      if (i * FN + j >= from)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[buf][j], f.b[buf][i], acc[i][j], 0, 0, 0);
}

// One 64-wide K slab (four k16 steps, library K order) with the last step
// carried over: its fragments stay in buffer 1 and are multiplied by the
// next call (carry = true) right after that call has requested its slab's
// first fragments, so those MFMAs cover the LDS latency at the slab start
// (behind the slab barrier).  The caller multiplies the final carried step
// after the last slab (mfma_frags(f, 1, acc)).
//
// In a loop that also issues LDS DMA, the compiler waits for fragment reads
// with lgkmcnt(0) (it takes the counter to be out of order), so a wait
// covers every read issued so far.  Each step therefore issues its first
// MFMA (whose wait then covers only that step's own fragments) before it
// requests the next step's fragments, which the remaining MFMAs cover.
// The accumulation order is unchanged.
template <int FM, int FN, int CPRA, int CPRB>
__device__ __forceinline__ void mfma_slab_carry(Frags<FM, FN>& f, bool carry, const uint4* sa, int ar0,
                                                const uint4* sb, int br0, int hk, f32x16 (&acc)[FM][FN]) {
  load_frags<FM, FN, CPRA, CPRB>(f, 0, sa, ar0, sb, br0, kchunk(0, hk));
  __builtin_amdgcn_sched_barrier(0);
  if (carry) mfma_frags(f, 1, acc);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < 3; ++ks) {
    acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[ks & 1][0], f.b[ks & 1][0], acc[0][0], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_frags<FM, FN, CPRA, CPRB>(f, (ks + 1) & 1, sa, ar0, sb, br0, kchunk(ks + 1, hk));
    __builtin_amdgcn_sched_barrier(0);
    mfma_frags(f, ks & 1, acc, 1);
    __builtin_amdgcn_sched_barrier(0);
  }
}

}  // namespace rocs
