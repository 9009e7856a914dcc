// Exhaustive check of the e4m3 encoder the kernels use.
//
//   e4m3_cvt_check         (prints one JSON line)
//
// f32x4_to_e4m3 (the hardware fp32 -> fp8 conversion after a clamp to +-460) against
// f32_to_e4m3 (the integer-op encoder that spells out nearest-even rounding, saturation at
// +-448, kept sign and e4m3 subnormals) on every finite fp32 bit pattern u.  Each call
// converts u, -u and two other patterns (u with bit 22 or bit 0 flipped), so every byte
// position of the packed result is compared.  Counts mismatches and records the first few.
#include <hip/hip_runtime.h>

#include <cstdio>

#include "../csrc/device_common.h"

using namespace moe355;

__global__ void check(unsigned long long* count, unsigned* first) {
  const uint64_t n = 1ull << 32;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x) {
    const uint32_t u = (uint32_t)i;
    if ((u & 0x7f800000u) == 0x7f800000u) continue;  // Inf and NaN: not encoder inputs
    const uint32_t v[4] = {u, u ^ 0x80000000u, u ^ 0x00400000u, u ^ 0x00000001u};
    float y[4];
    for (int k = 0; k < 4; ++k) y[k] = __uint_as_float(v[k]);
    const uint32_t hw = f32x4_to_e4m3(y[0], y[1], y[2], y[3]);
    for (int k = 0; k < 4; ++k) {
      const uint32_t ref = f32_to_e4m3(y[k]);
      const uint32_t got = (hw >> (8 * k)) & 0xffu;
      if (got != ref) {
        const unsigned long long c = atomicAdd(count, 1ull);
        if (c < 8) {
          first[3 * c] = v[k];
          first[3 * c + 1] = ref;
          first[3 * c + 2] = got;
        }
      }
    }
  }
}

int main() {
  unsigned long long* count = nullptr;
  unsigned* first = nullptr;
  if (hipMalloc(&count, sizeof(unsigned long long)) != hipSuccess || hipMalloc(&first, 24 * sizeof(unsigned)) != hipSuccess ||
      hipMemset(count, 0, sizeof(unsigned long long)) != hipSuccess || hipMemset(first, 0, 24 * sizeof(unsigned)) != hipSuccess) {
    std::printf("{\"error\": \"allocation\"}\n");
    return 1;
  }
  hipLaunchKernelGGL(check, dim3(8192), dim3(256), 0, 0, count, first);
  unsigned long long c = 0;
  unsigned f[24] = {0};
  if (hipDeviceSynchronize() != hipSuccess || hipMemcpy(&c, count, sizeof c, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(f, first, sizeof f, hipMemcpyDeviceToHost) != hipSuccess) {
    std::printf("{\"error\": \"launch\"}\n");
    return 1;
  }
  std::printf("{\"check\": \"f32x4_to_e4m3 vs f32_to_e4m3\", \"finite_patterns\": 4278190080, \"mismatches\": %llu, "
              "\"first\": [",
              c);
  for (unsigned long long k = 0; k < c && k < 8; ++k)
    std::printf("%s[\"%08x\", %u, %u]", k ? ", " : "", f[3 * k], f[3 * k + 1], f[3 * k + 2]);
  std::printf("]}\n");
  return c == 0 ? 0 : 2;
}
