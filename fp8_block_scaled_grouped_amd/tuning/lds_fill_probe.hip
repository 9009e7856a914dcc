// LDS operand-traffic probe for the grouped GEMM engines.
//
//   lds_fill_probe            (prints one JSON line per case)
//
// One 8-wave workgroup per CU (each asks for 160 KB of LDS) streams a window of global
// memory into S LDS stages with the engines' loop (LDS-DMA of 1 KB per wave and op,
// per-wave wait, barrier, refill of the freed stage) and no MFMA.  Optional per-step
// extras model the operand side: RK KB of 16-byte LDS reads per workgroup from the
// landed stage (the MFMA fragment reads), and GK KB of 16-byte global loads into
// registers (two waves read each byte), consumed one step later.  The DMA source stays
// inside the workgroup's window (offsets masked to it) and every LDS address stays below
// 160 KB (checked on the host before each launch).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

namespace {

typedef unsigned gu4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kLdsMax = 160 * 1024;

__device__ __forceinline__ const uint8_t* uniform_base(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(m0)
               : "memory");
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int S, int QW, int RK, int GK>
__global__ __launch_bounds__(512) void probe(const uint8_t* src, uint32_t win, int nwin, int iters, float* sink) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr uint32_t SB = 8u * QW * 1024u;  // stage bytes
  constexpr int NG = GK / 8;                // 1 KB global loads per wave and step
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
  const uint8_t* base = uniform_base(src + (size_t)(blockIdx.x % nwin) * win);
  const uint32_t mask = win - 1;
  auto issue = [&](int st, int it) {
#pragma unroll
    for (int j = 0; j < QW; ++j) {
      const int q = w + 8 * j;
      const uint32_t off = ((uint32_t)it * SB + (uint32_t)q * 1024u + (uint32_t)lane * 16u) & mask;
      dma16(base, off, lds0 + (uint32_t)st * SB + (uint32_t)q * 1024u);
    }
  };
  gu4 px[NG > 0 ? NG : 1], nx[NG > 0 ? NG : 1];
  auto gload = [&](int it, gu4(&dst)[NG > 0 ? NG : 1]) {
#pragma unroll
    for (int r = 0; r < NG; ++r) {
      const uint32_t off =
          ((uint32_t)it * (GK * 512u) + (uint32_t)((w & 3) * NG + r) * 1024u + (uint32_t)lane * 16u + (win >> 1)) & mask;
      dst[r] = *(const __attribute__((address_space(1))) gu4*)((const __attribute__((address_space(1))) uint8_t*)(
                                                                    uintptr_t)base + off);
    }
  };
  uint32_t x = 0;
  if constexpr (NG > 0) gload(0, px);
#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s, s);
  for (int it = 0; it < iters; ++it) {
    if constexpr (NG > 0) gload(it + 1, nx);
    vm_wait<(S - 2) * QW>();
    __syncthreads();
    issue((it + S - 1) % S, it + S - 1);
    if constexpr (RK > 0) {
      const uint8_t* st = lds + (it % S) * SB;
#pragma unroll
      for (int r = 0; r < RK / 8; ++r) {
        const uint32_t o = ((uint32_t)(w * (RK / 8) + r) * 1024u + (uint32_t)lane * 16u) % SB;
        const gu4 v = *reinterpret_cast<const gu4*>(st + o);
        x += v.x ^ v.w;
      }
    }
    if constexpr (NG > 0) {
#pragma unroll
      for (int r = 0; r < NG; ++r) {
        x += px[r].x ^ px[r].y ^ px[r].z ^ px[r].w;
        px[r] = nx[r];
      }
    }
  }
  vm_wait<0>();
  __syncthreads();
  if (tid == 0) sink[blockIdx.x] = reinterpret_cast<const float*>(lds)[1] + (float)x;
}

template <int S, int QW, int RK, int GK>
void run(const uint8_t* src, uint32_t win, int nwin, int wgs, int iters, float* sink, const char* name) {
  constexpr uint32_t SB = 8u * QW * 1024u;
  static_assert(S * SB <= kLdsMax, "stages fit the LDS");
  auto k = probe<S, QW, RK, GK>;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax) !=
      hipSuccess) {
    fprintf(stderr, "%s: cannot request %u bytes of LDS\n", name, kLdsMax);
    exit(1);
  }
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) exit(1);
  hipLaunchKernelGGL(k, dim3(wgs), dim3(512), kLdsMax, 0, src, win, nwin, 50, sink);
  (void)hipEventRecord(e0);
  hipLaunchKernelGGL(k, dim3(wgs), dim3(512), kLdsMax, 0, src, win, nwin, iters, sink);
  (void)hipEventRecord(e1);
  if (hipEventSynchronize(e1) != hipSuccess) {
    fprintf(stderr, "%s: launch failed\n", name);
    exit(1);
  }
  float ms = 0.0f;
  (void)hipEventElapsedTime(&ms, e0, e1);
  const double steps = (double)iters;
  printf("{\"case\": \"%s\", \"stage_kb\": %u, \"stages\": %d, \"lds_reads_kb_per_step\": %d, "
         "\"global_loads_kb_per_step\": %d, \"source_bytes\": %llu, \"ms\": %.4f, \"us_per_step\": %.4f, "
         "\"dma_tb_s\": %.2f}\n",
         name, SB / 1024, S, RK, GK, (unsigned long long)win * nwin, ms, ms * 1e3 / steps,
         (double)wgs * steps * SB / ms / 1e9);
  fflush(stdout);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
}

}  // namespace

int main() {
  const size_t total = 256u << 20;
  uint8_t* src = nullptr;
  float* sink = nullptr;
  if (hipMalloc(&src, total) != hipSuccess || hipMalloc(&sink, 4096 * sizeof(float)) != hipSuccess) return 1;
  if (hipMemset(src, 1, total) != hipSuccess) return 1;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0) != hipSuccess || cus <= 0 || cus > 4096)
    return 1;
  const int it = 4000;
  const uint32_t win = 1u << 20;  // 1 MB per workgroup: 2 windows stay in every L2, 256 stream past it
  // the 128 x 256 engine's step: 48 KB of DMA, 128 KB of fragment reads
  run<3, 6, 0, 0>(src, win, 2, cus, it, sink, "dma 48 KB (L2)");
  run<3, 6, 64, 0>(src, win, 2, cus, it, sink, "dma 48 KB + reads 64 KB (L2)");
  run<3, 6, 128, 0>(src, win, 2, cus, it, sink, "dma 48 KB + reads 128 KB (L2): 128x256 tile");
  run<3, 6, 192, 0>(src, win, 2, cus, it, sink, "dma 48 KB + reads 192 KB (L2)");
  run<3, 6, 0, 0>(src, win, 256, cus, it, sink, "dma 48 KB (256 MB stream)");
  run<3, 6, 128, 0>(src, win, 256, cus, it, sink, "dma 48 KB + reads 128 KB (256 MB stream)");
  // weights straight into registers instead: 16 KB of DMA, 64 KB of reads, 64 KB of loads
  run<3, 2, 64, 0>(src, win, 2, cus, it, sink, "dma 16 KB + reads 64 KB (L2)");
  run<3, 2, 0, 64>(src, win, 2, cus, it, sink, "dma 16 KB + loads 64 KB (L2)");
  run<3, 2, 64, 64>(src, win, 2, cus, it, sink, "dma 16 KB + reads 64 KB + loads 64 KB (L2)");
  // stage size and depth
  run<2, 6, 0, 0>(src, win, 2, cus, it, sink, "dma 48 KB, 2 stages (L2)");
  run<4, 4, 0, 0>(src, win, 2, cus, it, sink, "dma 32 KB, 4 stages (L2)");
  run<2, 8, 0, 0>(src, win, 2, cus, it, sink, "dma 64 KB, 2 stages (L2)");
  (void)hipFree(src);
  (void)hipFree(sink);
  return 0;
}
