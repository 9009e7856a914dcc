// K-step probe for the grouped GEMM engine's 128 x 256 tile.
//
//   kstep_probe            (prints one JSON line per case)
//
// One 8-wave workgroup per CU (each asks for 160 KB of LDS) runs the engine's K step with
// nothing else: three 48 KB LDS stages filled by LDS-DMA from a window of global memory,
// each wave reading its 4 + 4 fragments (64 activation and 64 weight rows of 128 bytes),
// 16 MFMA 16x16x128 (fp8) and the fp32 block-scale fold acc += tile * scale.  Cases:
//   behind  - the step waits for its stage, passes the barrier, then reads its fragments
//   ahead   - the fragments of the next K block are read during the step's MFMAs (each
//             register reloaded after its last use), as the engine does on 64-row and larger
//             tiles; variants without the per-step barrier or without the DMA show their share
// Every DMA source offset stays inside the workgroup's window (masked), every LDS address
// below 3 x 48 KB, and the accumulators are stored at the end so that no work is dead.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned gu4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kLdsMax = 160 * 1024;
constexpr int S = 3, QW = 6;                 // stages; 1 KB DMAs per wave and stage
constexpr uint32_t SB = 8u * QW * 1024u;     // 48 KB: 128 activation + 256 weight rows

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
__device__ __forceinline__ v8i frag(const uint8_t* p) {
  const gu4 lo = *reinterpret_cast<const gu4*>(p), hi = *reinterpret_cast<const gu4*>(p + 64);
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// AHEAD: fragments one block ahead; BAR / DMA: per-step barrier and stage refills on or off
template <int AHEAD, int BAR, int DMA>
__global__ __launch_bounds__(512) void kstep(const uint8_t* src, uint32_t win, int nwin, int iters, float* sink) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 2, wn = w & 3;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
  const uint8_t* base = uniform_base(src + (size_t)(blockIdx.x % nwin) * win);
  const uint32_t mask = win - 1;
  auto issue = [&](int st, int blk, int j) {
    const int q = w + 8 * j;
    const uint32_t off = ((uint32_t)blk * SB + (uint32_t)q * 1024u + (uint32_t)lane * 16u) & mask;
    dma16(base, off, lds0 + (uint32_t)st * SB + (uint32_t)q * 1024u);
  };
  // fragment t of this wave in stage st: activation rows 64 wm + 16 t (first 16 KB),
  // weight rows 64 wn + 16 t (the 32 KB after); lane: row l % 16, chunks l / 16 and l / 16 + 4
  auto pa = [&](int st, int t) { return lds + st * SB + (64 * wm + 16 * t + (lane & 15)) * 128 + (lane >> 4) * 16; };
  auto pb = [&](int st, int t) {
    return lds + st * SB + 16384 + (64 * wn + 16 * t + (lane & 15)) * 128 + (lane >> 4) * 16;
  };
  v4f acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  v8i a[4], b[4];
  float sc[4];
  const int npro = AHEAD ? S : S - 1;
#pragma unroll
  for (int s = 0; s < S; ++s)
    if (s < npro)
      for (int j = 0; j < QW; ++j) issue(s, s, j);
  if constexpr (AHEAD) {
    vm_wait<(S - 1) * QW>();
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      a[t] = frag(pa(0, t));
      b[t] = frag(pb(0, t));
      sc[t] = 1.0f + 1e-7f * (float)(a[t][0] & 255);
    }
  }
  for (int it = 0; it < iters; ++it) {
    const int st = it % S;
    if constexpr (DMA) vm_wait<(S - 2) * QW>();
    if constexpr (AHEAD) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if constexpr (BAR) __syncthreads();
    const int rst = AHEAD ? st : (it + S - 1) % S;  // stage refilled this step
    const int rblk = AHEAD ? it + S : it + S - 1;
    const int nst = (it + 1) % S;
    if constexpr (!AHEAD) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a[t] = frag(pa(st, t));
        b[t] = frag(pb(st, t));
        sc[t] = 1.0f + 1e-7f * (float)(a[t][0] & 255);
      }
    }
    v4f tq[3];
#pragma unroll
    for (int q = 0; q < 18; ++q) {
      if (q < 16)
        tq[q % 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[q % 4], b[q / 4], v4f{0.f, 0.f, 0.f, 0.f}, 0,
                                                                     0, 0, 0, 0, 0);
      if (DMA && 2 * q < 2 * QW && q % 2 == 0) {
        issue(rst, rblk, q / 2);
        issue(rst, rblk, q / 2 + QW / 2);
      }
      if (q >= 2) acc[q - 2] += tq[(q - 2) % 3] * sc[(q - 2) % 4];
      if constexpr (AHEAD) {
        if (q < 16 && q % 4 == 3) b[q / 4] = frag(pb(nst, q / 4));  // last use of b[q / 4]
        if (q >= 12 && q < 16) a[q % 4] = frag(pa(nst, q % 4));      // last use of a[q % 4]
        if (q >= 14) sc[(q - 2) % 4] = 1.0f + 1e-7f * (float)(a[(q - 2) % 4][0] & 255);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  vm_wait<0>();
  __syncthreads();
  float r = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  sink[blockIdx.x * 512 + tid] = r;
}

template <int AHEAD, int BAR, int DMA>
void run(const uint8_t* src, uint32_t win, int nwin, int wgs, int iters, float* sink, const char* name) {
  static_assert(S * SB <= kLdsMax, "stages fit the LDS");
  auto k = kstep<AHEAD, BAR, DMA>;
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
  const double flops = 2.0 * 128 * 256 * 128 * (double)iters * wgs;
  printf("{\"case\": \"%s\", \"source_bytes\": %llu, \"ms\": %.4f, \"us_per_step\": %.4f, \"tflop_s\": %.1f}\n", name,
         (unsigned long long)win * nwin, ms, ms * 1e3 / iters, flops / ms / 1e9);
  fflush(stdout);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
}

}  // namespace

int main() {
  const size_t total = 256u << 20;
  uint8_t* src = nullptr;
  float* sink = nullptr;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0) != hipSuccess || cus <= 0 || cus > 4096)
    return 1;
  if (hipMalloc(&src, total) != hipSuccess || hipMalloc(&sink, (size_t)cus * 512 * sizeof(float)) != hipSuccess)
    return 1;
  if (hipMemset(src, 0x11, total) != hipSuccess) return 1;
  const int it = 4000;
  const uint32_t win = 1u << 20;
  for (int rep = 0; rep < 2; ++rep) {
    run<0, 1, 1>(src, win, 2, cus, it, sink, "reads behind the barrier (L2)");
    run<1, 1, 1>(src, win, 2, cus, it, sink, "fragments one block ahead (L2)");
    run<1, 0, 1>(src, win, 2, cus, it, sink, "one block ahead, no barrier (L2)");
    run<1, 1, 0>(src, win, 2, cus, it, sink, "one block ahead, no DMA");
    run<0, 1, 1>(src, win, 256, cus, it, sink, "reads behind the barrier (256 MB stream)");
    run<1, 1, 1>(src, win, 256, cus, it, sink, "fragments one block ahead (256 MB stream)");
  }
  (void)hipFree(src);
  (void)hipFree(sink);
  return 0;
}
