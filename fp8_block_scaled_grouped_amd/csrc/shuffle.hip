// Pre-shuffled weight layout ("Accelerate DeepSeek-R1 Inference: Integrate AITER
// into SGLang", section "General Linear Layer": the linear path consumes weights
// permuted once, at load time, into an order that suits the matrix cores).
//
// The permutation here is this library's own, matched to its GEMM engine: a
// weight W [rows, K] (rows and K multiples of 128) becomes 128-row x 128-byte
// tiles.  Tile (t, kb) -- rows [128t, 128t+128), bytes [128kb, 128kb+128) of
// each row -- sits at byte (t * K/128 + kb) * 16384, so the K blocks of a row
// tile follow one another; inside a tile, row rr takes 128 bytes at rr * 128
// and its 16-byte chunk c is stored in slot c ^ (rr & 7), the slot the GEMM
// keeps it in LDS.  A GEMM DMA of 8 rows is then one contiguous 1 KB block.
// Expert tensors [E, R, K] are shuffled as one [E*R, K] matrix (R % 128 == 0
// keeps experts apart).
#include "device_common.h"
#include "host_common.h"

namespace moe355 {
namespace {

constexpr int kThreads = 256;

// one thread per 16-byte chunk of the source, in source order (coalesced reads)
__global__ __launch_bounds__(kThreads) void shuffle_128x128_kernel(const uint8_t* __restrict__ w, int64_t chunks,
                                                                   int K, uint8_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= chunks) return;
  const int cpr = K / 16;  // chunks per row
  const int64_t r = i / cpr;
  const int ci = (int)(i - r * cpr);
  const int kb = ci / 8, c = ci % 8;
  const int64_t t = r / 128;
  const int rr = (int)(r % 128);
  const int64_t dst = ((t * (K / 128) + kb) * 128 + rr) * 128 + ((c ^ (rr & 7)) << 4);
  *reinterpret_cast<u32x4*>(out + dst) = *reinterpret_cast<const u32x4*>(w + i * 16);
}

}  // namespace
}  // namespace moe355

using namespace moe355;

extern "C" int shuffle_weight_128x128(const uint8_t* w, int64_t rows, int K, uint8_t* out, hipStream_t stream) {
  MOE355_CHECK(rows >= 0 && K >= 0, MOE355_EINVAL);
  MOE355_CHECK(rows % 128 == 0 && K % 128 == 0, MOE355_EUNSUPPORTED);
  if (rows == 0 || K == 0) return MOE355_OK;
  MOE355_CHECK(w && out, MOE355_EINVAL);
  const int64_t bytes = rows * K;
  const uintptr_t a = reinterpret_cast<uintptr_t>(w), b = reinterpret_cast<uintptr_t>(out);
  MOE355_CHECK(a + bytes <= b || b + bytes <= a, MOE355_EINVAL);  // out must not overlap w
  MOE355_CHECK(aligned16(w) && aligned16(out), MOE355_EMISALIGNED);
  const int64_t chunks = bytes / 16;
  const int64_t blocks = ceil_div64(chunks, kThreads);
  MOE355_CHECK(blocks < (1ll << 31), MOE355_EUNSUPPORTED);
  hipLaunchKernelGGL(shuffle_128x128_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, w, chunks, K, out);
  return launch_status();
}
