// Dense FP8 block-scale GEMM for small M ("General Linear Layer": Y = (XQ, 1x128
// scales) times (WQ, 128x128 scales)^T, WQ stored [N, K]), the decode-sized case
// where the weights are streamed once and nothing is reused.
//
// One workgroup per 16 output columns (16 rows of B); its 8 waves split the K blocks
// into contiguous runs, each wave accumulating a 16 x (16 MT) fp32 tile with the
// block-scale fold acc += tile * (a_scale(row) * b_scale); the 8 partial tiles are
// then summed in LDS in wave order (fixed, so the result is deterministic) and
// rounded once.  One launch, no workspace.  Operands go straight from memory into
// the MFMA registers (B rows as the MFMA's row operand, A rows as its column operand):
// there is no reuse to stage through LDS.  Every lane keeps the operands of kDepth K
// blocks in flight.
#include "dense_small.h"

#include "device_common.h"
#include "host_common.h"

namespace moe355 {
namespace {

constexpr int kNW = 8;      // waves

// 32 bytes of one K block for the MFMA: lane l (row l % 16 of the 16-row fragment)
// takes chunks l / 16 and l / 16 + 4 of the 128-byte block; chunks at or past K
// read as zeros (K % 16 == 0, so a chunk is all in or all out).
__device__ __forceinline__ v8i load_frag(const uint8_t* row, int64_t k0, int K, int lane) {
  const int c0 = lane >> 4;
  const int64_t k_lo = k0 + 16 * c0, k_hi = k0 + 16 * (c0 + 4);
  u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
  if (k_lo < K) lo = *reinterpret_cast<const u32x4*>(row + k_lo);
  if (k_hi < K) hi = *reinterpret_cast<const u32x4*>(row + k_hi);
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// The same for B pre-shuffled into 128 x 128-byte tiles (tile (n / 128, kb) at
// ((n / 128) * KB + kb) * 16 KB, row n % 128 at 128 bytes each, chunk c in slot
// c ^ (n & 7)); N and K are multiples of 128 there.
__device__ __forceinline__ v8i load_frag_bsh(const uint8_t* b, int n, int kb, int KB, int lane) {
  const uint8_t* row = b + ((int64_t)(n >> 7) * KB + kb) * (128 * 128) + (n & 127) * 128;
  const int c0 = lane >> 4;
  const u32x4 lo = *reinterpret_cast<const u32x4*>(row + ((c0 ^ (n & 7)) << 4));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(row + (((c0 + 4) ^ (n & 7)) << 4));
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int MT, bool BSH>
__global__ __launch_bounds__(kNW * 64) void dense_small_kernel(DenseSmallArgs g) {
  constexpr int kDepth = MT >= 4 ? 2 : 4;  // K blocks of operands in flight per wave
  __shared__ v4f part[kNW][MT][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * 16;
  const int KB = (g.K + 127) / 128;
  const int per = (KB + kNW - 1) / kNW;
  const int kb0 = min(KB, w * per), kb1 = min(KB, kb0 + per);

  // B row of this lane (rows past N repeat row N - 1: in bounds, results not stored)
  const int bn = min(n0 + (lane & 15), g.N - 1);
  const uint8_t* brow = g.b + (int64_t)bn * g.K;
  const float* sbrow = g.b_scale + (int64_t)(n0 / 128) * KB;  // the 16 rows share a scale row
  const uint8_t* arow[MT];
  int64_t srow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = min(16 * t + (lane & 15), g.M - 1);
    arow[t] = g.a + (int64_t)m * g.K;
    srow[t] = (int64_t)m * g.ssm;
  }

  v4f acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  // kDepth K blocks of operands and A scales in flight
  v8i bq[kDepth], aq[kDepth][MT];
  float sq[kDepth][MT];
  auto fetch = [&](int d, int k) {
    bq[d] = BSH ? load_frag_bsh(g.b, bn, k, KB, lane) : load_frag(brow, (int64_t)k * 128, g.K, lane);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      aq[d][t] = load_frag(arow[t], (int64_t)k * 128, g.K, lane);
      sq[d][t] = g.a_scale[srow[t] + (int64_t)k * g.sskb];
    }
  };
#pragma unroll
  for (int d = 0; d < kDepth; ++d)
    if (kb0 + d < kb1) fetch(d, kb0 + d);
  for (int kb = kb0; kb < kb1; kb += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int k = kb + d;
      if (k < kb1) {
        const v8i b = bq[d];
        v8i a[MT];
        float sa[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          a[t] = aq[d][t];
          sa[t] = sq[d][t];
        }
        if (k + kDepth < kb1) fetch(d, k + kDepth);
        const float sb = sbrow[k];
#pragma unroll
        for (int t = 0; t < MT; ++t)  // output (B row 4 (l / 16) + i, A row l % 16): one A scale per lane
          acc[t] += mfma16x16x128_fp8(b, a[t], v4f{0.f, 0.f, 0.f, 0.f}) * (sa[t] * sb);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) part[w][t][lane] = acc[t];
  __syncthreads();
  if (tid < MT * 64) {
    const int t = tid >> 6;
    v4f s = part[0][t][lane];
#pragma unroll
    for (int ww = 1; ww < kNW; ++ww) s += part[ww][t][lane];
    const int m = 16 * t + (lane & 15), n = n0 + 4 * (lane >> 4);
    if (m < g.M && n < g.N) {  // N % 8 == 0: the 4 columns are all in or all out
      const bool f16 = g.out_f16 != 0;
      const uint2 r{f32_to_out16(s[0], f16) | (f32_to_out16(s[1], f16) << 16),
                    f32_to_out16(s[2], f16) | (f32_to_out16(s[3], f16) << 16)};
      *reinterpret_cast<uint2*>(g.c + (int64_t)m * g.ldc + n) = r;
    }
  }
}

}  // namespace

template <bool BSH>
int launch_small(const DenseSmallArgs& g, hipStream_t stream) {
  const int mt = (g.M + 15) / 16;
  const int64_t grid = (g.N + 15) / 16;
  if (g.M == 0 || g.N == 0) return MOE355_OK;
  MOE355_CHECK(grid < (1ll << 31), MOE355_EUNSUPPORTED);
  switch (mt) {
    case 1: hipLaunchKernelGGL((dense_small_kernel<1, BSH>), dim3((unsigned)grid), dim3(kNW * 64), 0, stream, g); break;
    case 2: hipLaunchKernelGGL((dense_small_kernel<2, BSH>), dim3((unsigned)grid), dim3(kNW * 64), 0, stream, g); break;
    case 3:
    case 4: hipLaunchKernelGGL((dense_small_kernel<4, BSH>), dim3((unsigned)grid), dim3(kNW * 64), 0, stream, g); break;
    default: return MOE355_EUNSUPPORTED;
  }
  return launch_status();
}

int launch_dense_small(const DenseSmallArgs& g, bool bsh, hipStream_t stream) {
  return bsh ? launch_small<true>(g, stream) : launch_small<false>(g, stream);
}

}  // namespace moe355
