// The small-M dense GEMM (dense_small.hip): one workgroup per 16 output columns,
// K split over its waves and the partial tiles summed in LDS in a fixed order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe355 {

struct DenseSmallArgs {
  const uint8_t* a;       // e4m3 [M, K]
  const float* a_scale;   // element (m, kb) at a_scale[m * ssm + kb * sskb]
  int64_t ssm, sskb;
  const uint8_t* b;       // e4m3 [N, K]
  const float* b_scale;   // [ceil(N/128), ceil(K/128)]
  int M, N, K;            // M <= 64, K % 16 == 0, N % 8 == 0
  uint16_t* c;            // [M, N] bf16 or fp16 bits, row stride ldc
  int64_t ldc;
  int out_f16;
};

// Launches the kernel for M <= 64 (16-row tiles of A: 1, 2 or 4); bsh: b holds the
// 128 x 128-tile pre-shuffled layout (N, K multiples of 128); MOE355_* status.
int launch_dense_small(const DenseSmallArgs& g, bool bsh, hipStream_t stream);

}  // namespace moe355
