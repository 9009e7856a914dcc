// Shared pieces of the block-scaled FP8 GEMM engines (gfx950): the argument
// block, the LDS-DMA primitives, explicit vmcnt waits and the swizzled LDS
// fragment reads.  See gemm.hip for the engine these serve.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace moe355 {

enum Mode : int { kDense = 0, kG1U1 = 1, kDown = 2 };

struct GemmArgs {
  const uint8_t* a;        // dense: [M, K]; g1u1: a8 [T, K]; down: h8 [max_sorted, K]
  const float* a_scale;    // element (row, kb) at a_scale[row * ssm + kb * sskb]
  int64_t ssm, sskb;
  const uint8_t* b;        // dense: [N, K]; g1u1: w1 [E, 2I, K]; down: w2 [E, N, K]
  const float* b_scale;    // dense: [N/128, K/128]; g1u1: [E, 2I/128, K/128]; down: [E, N/128, K/128]
  const int32_t* sorted_ids;
  const int32_t* sorted_eids;
  const int32_t* num_valid;
  const float* sorted_w;
  int M;                   // dense rows
  int N;                   // output columns: dense N, g1u1 I, down H
  int K;
  int T, topk;
  uint16_t* c;             // dense out
  int64_t ldc;
  uint8_t* h8;             // g1u1 out [max_sorted, N]
  float* h_scale;          // g1u1 out [max_sorted, N/128]
  float* y;                // down staging [T*topk, N] fp32
  const float* smooth;     // g1u1: optional per-expert channel factors for h [E, N] (fc2 smoothing)
  int splits, kbs;         // dense split-K: K blocks [ks*kbs, ks*kbs+kbs) per split ks
  int out_f16;             // dense: c holds fp16 (1) or bf16 (0) bits
  float* part;             // dense split-K partial sums [splits, M, N] fp32
};

namespace {

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// LDS-DMA: every lane moves 16 (or 4) bytes from base + its 32-bit offset to
// LDS[m0 + 16*lane] (or 4*lane); base is wave-uniform (SGPRs), so advancing a
// stream costs scalar adds only.  Issued from asm so that the compiler does
// not drain the DMA queue before each LDS read; completion is tracked
// explicitly with vm_wait.  No output registers.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(m0)
               : "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "s"(m0)
               : "memory");
}

__device__ __forceinline__ const uint8_t* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// wait until at most a*PER of this wave's DMAs are in flight, a in [0, 2]
template <int PER>
__device__ __forceinline__ void vm_wait_stages(int a) {
  if (a >= 2) {
    vm_wait<2 * PER>();
  } else if (a == 1) {
    vm_wait<PER>();
  } else {
    vm_wait<0>();
  }
}

__device__ __forceinline__ void lgkm_wait0() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0), vmcnt and expcnt untouched
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int swz(int r, int ch) { return r * 128 + ((ch ^ (r & 7)) << 4); }

// MFMA operand for the 16 rows starting at r0: lane l holds row r0 + l%16 with
// K chunks l/16 (low half) and 4 + l/16 (high half; its slot differs in bit 2).
__device__ __forceinline__ v8i lds_frag(const uint8_t* tile, int r0, int lane) {
  const int off = swz(r0 + (lane & 15), lane >> 4);
  const u32x4 lo = *reinterpret_cast<const u32x4*>(tile + off);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(tile + (off ^ 64));
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

}  // namespace

// The grouped GEMMs (g1u1, down) on 256 x 256 tiles with the weight rows as the
// MFMA's row operand (gemm_big.hip): launches the grid for `mblocks` sorted blocks
// of 256 rows; MOE355_* status.
template <int MODE, bool BSH>
int launch_big(const GemmArgs& g, int64_t mblocks, hipStream_t stream);

}  // namespace moe355
