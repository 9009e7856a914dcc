// Dynamic 1x128 FP8 quantisation ("Accelerate DeepSeek-R1 Inference: Integrate
// AITER into SGLang", section "General Linear Layer": one scale per 1x128 of an
// activation row; section "Blockscale FP8 MoE Computation": the bf16 hidden
// states are quantised per 128 before the grouped GEMM).
//
// 16 lanes own one 128-wide group (8 bf16 = 16 bytes each); amax by xor
// shuffles inside the 16; IEEE fp32 divisions for the scale and each element,
// nearest-even saturating e4m3 encode in integer ops.  When K is not a
// multiple of 128 the last group of a row holds the K % 128 remaining values
// (K % 8 == 0, so a lane's 8 values are all inside or all outside K).
#include "device_common.h"
#include "host_common.h"

namespace moe355 {
namespace {

constexpr int kThreads = 256;
constexpr int kGroupsPerBlock = kThreads / 16;

__global__ __launch_bounds__(kThreads) void quant_1x128_kernel(const uint16_t* __restrict__ x, int64_t ld_x, int M,
                                                               int K, int KB, uint8_t* __restrict__ q, int64_t ld_q,
                                                               float* __restrict__ scale, int64_t ssm, int64_t sskb) {
  const int64_t g = (int64_t)blockIdx.x * kGroupsPerBlock + threadIdx.x / 16;
  const int sub = threadIdx.x % 16;
  if (g >= (int64_t)M * KB) return;  // whole 16-lane groups leave together
  const int64_t m = g / KB;
  const int kb = (int)(g - m * KB);
  const bool live = kb * 128 + sub * 8 < K;  // lanes past K count as zeros in the amax
  const uint4 v = live ? *reinterpret_cast<const uint4*>(x + m * ld_x + kb * 128 + sub * 8) : make_uint4(0, 0, 0, 0);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(w[i] & 0xffffu);
    f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
  const float s = (amax == 0.0f) ? 1.0f : amax / kE4M3Max;
  const uint32_t lo = f32x4_to_e4m3(f[0] / s, f[1] / s, f[2] / s, f[3] / s);
  const uint32_t hi = f32x4_to_e4m3(f[4] / s, f[5] / s, f[6] / s, f[7] / s);
  if (live) *reinterpret_cast<uint2*>(q + m * ld_q + kb * 128 + sub * 8) = make_uint2(lo, hi);
  if (sub == 0) scale[m * ssm + kb * sskb] = s;
}

}  // namespace
}  // namespace moe355

using namespace moe355;

extern "C" int fp8_quant_1x128(const uint16_t* x, int64_t ld_x, int M, int K, uint8_t* q, int64_t ld_q, float* scale,
                               int64_t sstride_m, int64_t sstride_kb, hipStream_t stream) {
  MOE355_CHECK(M >= 0 && K >= 0 && ld_x >= K && ld_q >= K, MOE355_EINVAL);
  MOE355_CHECK(K % 8 == 0, MOE355_EUNSUPPORTED);
  if (M == 0 || K == 0) return MOE355_OK;
  MOE355_CHECK(x && q && scale && sstride_m >= 0 && sstride_kb >= 0, MOE355_EINVAL);
  MOE355_CHECK(aligned16(x) && aligned16(q) && (ld_x * 2) % 16 == 0 && ld_q % 8 == 0, MOE355_EMISALIGNED);
  MOE355_CHECK((reinterpret_cast<uintptr_t>(scale) & 3u) == 0, MOE355_EMISALIGNED);
  const int KB = (int)ceil_div64(K, 128);
  const int64_t groups = (int64_t)M * KB;
  const int64_t blocks = ceil_div64(groups, kGroupsPerBlock);
  MOE355_CHECK(blocks < (1ll << 31), MOE355_EUNSUPPORTED);
  hipLaunchKernelGGL(quant_1x128_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, x, ld_x, M, K, KB, q, ld_q,
                     scale, sstride_m, sstride_kb);
  return launch_status();
}
