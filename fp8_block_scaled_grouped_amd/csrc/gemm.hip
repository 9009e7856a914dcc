// Block-scaled FP8 GEMM engine on gfx950 FP8 MFMA.
//
// One workgroup (4 waves) computes a BM x 128 output tile; the K loop walks
// 128-wide scale blocks.  Per block each wave runs 16x16x128 FP8 MFMAs into a
// fresh fp32 tile and folds it into its accumulators as acc += tile *
// (a_scale(row) * b_scale), so both scales are applied once per 128 of K in
// fp32 ("Accelerate DeepSeek-R1 Inference: Integrate AITER into SGLang",
// section "General Linear Layer": 1x128 activation scales, 128x128 weight
// scales).  A and B tiles are staged through LDS, double buffered, with
// 16-byte global loads and an XOR swizzle of the 16-byte chunks of each row.
//
// Modes:
//   dense  C[M, N] = A[M, K] * B[N, K]^T, bf16 out ("General Linear Layer").
//   g1u1   grouped GEMM over the sorted pairs ("Complete MoE Implementation" /
//          "Blockscale FP8 MoE Computation"): A rows gathered through
//          sorted_ids, B = gate and up rows of the block's expert, epilogue
//          h = SiLU(gate) * up and 1x128 e4m3 requantisation of h.
//   down   grouped GEMM of h with the expert's down weights; each row is scaled
//          by its routing weight and staged per flat pair; a second kernel sums
//          each token's pairs in ascending order into bf16.
#include "device_common.h"
#include "host_common.h"

namespace moe355 {
namespace {

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
};

template <int BM, int MODE>
struct Tile {
  static constexpr int kParts = MODE == kG1U1 ? 2 : 1;  // g1u1: gate and up
  static constexpr int kBRows = 128 * kParts;
  static constexpr int kWM = BM >= 64 ? 2 : 1;            // waves along M
  static constexpr int kWN = 4 / kWM;                      // waves along N
  static constexpr int kWTM = BM / kWM;                    // rows per wave
  static constexpr int kWTN = 128 / kWN;                   // output columns per wave
  static constexpr int kTM = kWTM / 16;
  static constexpr int kTN = kWTN / 16;
  static constexpr int kAChunks = BM * 8;
  static constexpr int kAPerThread = (kAChunks + 255) / 256;
  static constexpr int kBPerThread = kBRows * 8 / 256;
};

__device__ __forceinline__ int swz(int r, int ch) { return r * 128 + ((ch ^ (r & 7)) << 4); }

// MFMA operand of row r: K slots [32g, 32g+32) are chunks 2g and 2g+1.
__device__ __forceinline__ v8i lds_frag(const uint8_t* tile, int r, int g) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(tile + swz(r, 2 * g));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(tile + swz(r, 2 * g + 1));
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Global -> registers for one K step: 16-byte chunks of the A and B tiles.
template <int NA, int NB>
__device__ __forceinline__ void gload_tile(u32x4 (&ra)[NA], u32x4 (&rb)[NB], const uint8_t* const (&a_src)[NA],
                                           const uint8_t* const (&b_src)[NB], bool a_live, int64_t koff) {
#pragma unroll
  for (int i = 0; i < NA; ++i)
    if (i + 1 < NA || a_live) ra[i] = *reinterpret_cast<const u32x4*>(a_src[i] + koff);
#pragma unroll
  for (int i = 0; i < NB; ++i) rb[i] = *reinterpret_cast<const u32x4*>(b_src[i] + koff);
}

// Registers -> LDS (swizzled offsets precomputed per thread).
template <int NA, int NB>
__device__ __forceinline__ void lstore_tile(uint8_t* a_tile, uint8_t* b_tile, const u32x4 (&ra)[NA],
                                            const u32x4 (&rb)[NB], const int (&a_off)[NA], const int (&b_off)[NB],
                                            bool a_live) {
#pragma unroll
  for (int i = 0; i < NA; ++i)
    if (i + 1 < NA || a_live) *reinterpret_cast<u32x4*>(a_tile + a_off[i]) = ra[i];
#pragma unroll
  for (int i = 0; i < NB; ++i) *reinterpret_cast<u32x4*>(b_tile + b_off[i]) = rb[i];
}

template <int BM, int MODE>
__global__ __launch_bounds__(256) void bs_gemm_kernel(GemmArgs g) {
  using C = Tile<BM, MODE>;
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][BM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t b_lds[2][C::kBRows * 128];
  __shared__ __attribute__((aligned(16))) float sa_lds[2][BM];
  __shared__ int rowinfo[BM];
  __shared__ float red[C::kWN][BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::kWN, wn = wave % C::kWN;
  const int NT = g.N / 128;
  const int nt = (int)(blockIdx.x % NT);
  const int mb = (int)(blockIdx.x / NT);
  const int64_t row0 = (int64_t)mb * BM;
  const int KB = g.K / 128;
  const int npairs = g.T * g.topk;

  int expert = 0, nvalid = 0;
  if constexpr (MODE != kDense) {
    nvalid = g.num_valid[0];
    if (row0 >= nvalid) return;  // uniform: this block holds no sorted rows
    expert = g.sorted_eids[mb];
    if (tid < BM) rowinfo[tid] = g.sorted_ids[row0 + tid];
    __syncthreads();
  }

  // ---- per-thread global sources (advance by 128 bytes per K step)
  const uint8_t* a_src[C::kAPerThread];
  int a_off[C::kAPerThread];
#pragma unroll
  for (int i = 0; i < C::kAPerThread; ++i) {
    const int ci = tid + 256 * i;
    const int r = (ci >> 3) < BM ? (ci >> 3) : BM - 1;
    const int ch = ci & 7;
    int64_t arow;
    if constexpr (MODE == kDense) {
      arow = row0 + r < g.M ? row0 + r : g.M - 1;
    } else if constexpr (MODE == kG1U1) {
      const int pid = rowinfo[r];
      arow = pid < npairs ? pid / g.topk : 0;
    } else {
      arow = row0 + r;
    }
    a_src[i] = g.a + arow * g.K + ch * 16;
    a_off[i] = swz(r, ch);
  }
  const float* sa_src = g.a_scale;
  if (tid < BM) {
    int64_t arow;
    if constexpr (MODE == kDense) {
      arow = row0 + tid < g.M ? row0 + tid : g.M - 1;
    } else if constexpr (MODE == kG1U1) {
      const int pid = rowinfo[tid];
      arow = pid < npairs ? pid / g.topk : 0;
    } else {
      arow = row0 + tid;
    }
    sa_src = g.a_scale + arow * g.ssm;
  }
  const uint8_t* b_src[C::kBPerThread];
  int b_off[C::kBPerThread];
  const int64_t KBYTES = g.K;
#pragma unroll
  for (int i = 0; i < C::kBPerThread; ++i) {
    const int ci = tid + 256 * i;
    const int r = ci >> 3, ch = ci & 7;
    int64_t brow;
    if constexpr (MODE == kDense) {
      brow = (int64_t)nt * 128 + r;
    } else if constexpr (MODE == kG1U1) {
      brow = (int64_t)expert * 2 * g.N + (r < 128 ? nt * 128 + r : g.N + nt * 128 + (r - 128));
    } else {
      brow = (int64_t)expert * g.N + nt * 128 + r;
    }
    b_src[i] = g.b + brow * KBYTES + ch * 16;
    b_off[i] = swz(r, ch);
  }
  const float* sb_src[C::kParts];
  if constexpr (MODE == kDense) {
    sb_src[0] = g.b_scale + (int64_t)nt * KB;
  } else if constexpr (MODE == kG1U1) {
    const int64_t nb2 = 2 * (g.N / 128);
    sb_src[0] = g.b_scale + ((int64_t)expert * nb2 + nt) * KB;
    sb_src[C::kParts - 1] = g.b_scale + ((int64_t)expert * nb2 + g.N / 128 + nt) * KB;
  } else {
    sb_src[0] = g.b_scale + ((int64_t)expert * NT + nt) * KB;
  }

  v4f acc[C::kParts][C::kTM][C::kTN];
#pragma unroll
  for (int p = 0; p < C::kParts; ++p)
#pragma unroll
    for (int tm = 0; tm < C::kTM; ++tm)
#pragma unroll
      for (int tn = 0; tn < C::kTN; ++tn) acc[p][tm][tn] = v4f{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[C::kAPerThread];
  u32x4 rb[C::kBPerThread];
  float rsa = 0.0f;
  const bool a_live = C::kAChunks >= 256 || tid < C::kAChunks;  // only BM = 16 leaves threads idle

  gload_tile<C::kAPerThread, C::kBPerThread>(ra, rb, a_src, b_src, a_live, 0);
  if (tid < BM) rsa = sa_src[0];
  lstore_tile<C::kAPerThread, C::kBPerThread>(a_lds[0], b_lds[0], ra, rb, a_off, b_off, a_live);
  if (tid < BM) sa_lds[0][tid] = rsa;
  __syncthreads();
  const int lr = lane & 15, lg = lane >> 4;
  for (int kb = 0; kb < KB; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < KB) {
      gload_tile<C::kAPerThread, C::kBPerThread>(ra, rb, a_src, b_src, a_live, (int64_t)(kb + 1) * 128);
      if (tid < BM) rsa = sa_src[(int64_t)(kb + 1) * g.sskb];
    }
    float sb[C::kParts];
#pragma unroll
    for (int p = 0; p < C::kParts; ++p) sb[p] = sb_src[p][kb];
    v8i av[C::kTM];
    v4f sa4[C::kTM];
#pragma unroll
    for (int tm = 0; tm < C::kTM; ++tm) {
      av[tm] = lds_frag(a_lds[buf], wm * C::kWTM + tm * 16 + lr, lg);
      sa4[tm] = *reinterpret_cast<const v4f*>(&sa_lds[buf][wm * C::kWTM + tm * 16 + 4 * lg]);
    }
#pragma unroll
    for (int p = 0; p < C::kParts; ++p) {
      v8i bv[C::kTN];
#pragma unroll
      for (int tn = 0; tn < C::kTN; ++tn) bv[tn] = lds_frag(b_lds[buf], p * 128 + wn * C::kWTN + tn * 16 + lr, lg);
#pragma unroll
      for (int tm = 0; tm < C::kTM; ++tm) {
        const v4f s4 = sa4[tm] * sb[p];
#pragma unroll
        for (int tn = 0; tn < C::kTN; ++tn) {
          const v4f t = mfma16x16x128_fp8(av[tm], bv[tn], v4f{0.f, 0.f, 0.f, 0.f});
          acc[p][tm][tn] += t * s4;
        }
      }
    }
    if (kb + 1 < KB) {
      lstore_tile<C::kAPerThread, C::kBPerThread>(a_lds[buf ^ 1], b_lds[buf ^ 1], ra, rb, a_off, b_off, a_live);
      if (tid < BM) sa_lds[buf ^ 1][tid] = rsa;
    }
    __syncthreads();
  }

  // ---- epilogues
  if constexpr (MODE == kDense) {
#pragma unroll
    for (int tm = 0; tm < C::kTM; ++tm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = row0 + wm * C::kWTM + tm * 16 + 4 * lg + i;
        if (m < g.M) {
#pragma unroll
          for (int tn = 0; tn < C::kTN; ++tn) {
            const int n = nt * 128 + wn * C::kWTN + tn * 16 + lr;
            g.c[m * g.ldc + n] = (uint16_t)f32_to_bf16(acc[0][tm][tn][i]);
          }
        }
      }
  } else if constexpr (MODE == kDown) {
#pragma unroll
    for (int tm = 0; tm < C::kTM; ++tm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = wm * C::kWTM + tm * 16 + 4 * lg + i;
        const int pid = rowinfo[rl];
        if (row0 + rl < nvalid && pid < npairs) {
          const float wgt = g.sorted_w[row0 + rl];
          float* dst = g.y + (int64_t)pid * g.N + nt * 128 + wn * C::kWTN + lr;
#pragma unroll
          for (int tn = 0; tn < C::kTN; ++tn) dst[tn * 16] = acc[0][tm][tn][i] * wgt;
        }
      }
  } else {
    // h = SiLU(gate) * up, then 1x128 requantisation of each row's 128 columns
    float rmax[C::kTM][4];
#pragma unroll
    for (int tm = 0; tm < C::kTM; ++tm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mx = 0.0f;
#pragma unroll
        for (int tn = 0; tn < C::kTN; ++tn) {
          const float gt = acc[0][tm][tn][i];
          const float up = acc[C::kParts - 1][tm][tn][i];
          const float h = gt / (1.0f + expf(-gt)) * up;
          acc[0][tm][tn][i] = h;
          mx = fmaxf(mx, fabsf(h));
        }
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
        rmax[tm][i] = mx;
      }
    if (lr == 0) {
#pragma unroll
      for (int tm = 0; tm < C::kTM; ++tm)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wn][wm * C::kWTM + tm * 16 + 4 * lg + i] = rmax[tm][i];
    }
    __syncthreads();
    uint8_t* obuf = a_lds[0];
    const int IB = g.N / 128;
#pragma unroll
    for (int tm = 0; tm < C::kTM; ++tm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = wm * C::kWTM + tm * 16 + 4 * lg + i;
        float amax = red[0][rl];
#pragma unroll
        for (int w2 = 1; w2 < C::kWN; ++w2) amax = fmaxf(amax, red[w2][rl]);
        const float s = (amax == 0.0f) ? 1.0f : amax / kE4M3Max;
#pragma unroll
        for (int tn = 0; tn < C::kTN; ++tn)
          obuf[rl * 128 + wn * C::kWTN + tn * 16 + lr] = (uint8_t)f32_to_e4m3(acc[0][tm][tn][i] / s);
        if (wn == 0 && lr == 0 && rowinfo[rl] < npairs) g.h_scale[(row0 + rl) * IB + nt] = s;
      }
    __syncthreads();
    for (int ci = tid; ci < BM * 8; ci += 256) {
      const int rl = ci >> 3, ch = ci & 7;
      if (rowinfo[rl] < npairs)
        *reinterpret_cast<u32x4*>(g.h8 + (row0 + rl) * g.N + nt * 128 + ch * 16) =
            *reinterpret_cast<const u32x4*>(obuf + rl * 128 + ch * 16);
    }
  }
}

// out[t, n] = bf16(sum_j y[t*k + j, n]), j ascending, fp32.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, int T, int k, int H,
                                                      uint16_t* __restrict__ out, int64_t ld_out) {
  const int H8 = H / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = idx / H8;
  const int c8 = (int)(idx - t * H8);
  if (t >= T) return;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const float4* p = reinterpret_cast<const float4*>(y + ((t * k + j) * (int64_t)H + c8 * 8));
    const float4 a = p[0], b = p[1];
    s[0] += a.x;
    s[1] += a.y;
    s[2] += a.z;
    s[3] += a.w;
    s[4] += b.x;
    s[5] += b.y;
    s[6] += b.z;
    s[7] += b.w;
  }
  const u32x4 o{f32_to_bf16(s[0]) | (f32_to_bf16(s[1]) << 16), f32_to_bf16(s[2]) | (f32_to_bf16(s[3]) << 16),
                f32_to_bf16(s[4]) | (f32_to_bf16(s[5]) << 16), f32_to_bf16(s[6]) | (f32_to_bf16(s[7]) << 16)};
  *reinterpret_cast<u32x4*>(out + t * ld_out + c8 * 8) = o;
}

template <int MODE>
int launch_gemm(const GemmArgs& g, int bm, int64_t mblocks, hipStream_t stream) {
  const int64_t grid = mblocks * (g.N / 128);
  if (grid == 0) return MOE355_OK;
  MOE355_CHECK(grid < (1ll << 31), MOE355_EUNSUPPORTED);
  const dim3 gd((unsigned)grid), bd(256);
  switch (bm) {
    case 16: hipLaunchKernelGGL((bs_gemm_kernel<16, MODE>), gd, bd, 0, stream, g); break;
    case 32: hipLaunchKernelGGL((bs_gemm_kernel<32, MODE>), gd, bd, 0, stream, g); break;
    case 64: hipLaunchKernelGGL((bs_gemm_kernel<64, MODE>), gd, bd, 0, stream, g); break;
    case 128: hipLaunchKernelGGL((bs_gemm_kernel<128, MODE>), gd, bd, 0, stream, g); break;
    default: return MOE355_EUNSUPPORTED;
  }
  return launch_status();
}

int check_sorted_capacity(int T, int topk, int E, int block_m, int64_t max_sorted) {
  int64_t need = 0;
  const int st = moe_sort_sizes(T, topk, E, block_m, &need, nullptr, nullptr);
  if (st != MOE355_OK) return st;
  return max_sorted >= need && max_sorted % block_m == 0 ? MOE355_OK : MOE355_EINVAL;
}

}  // namespace
}  // namespace moe355

using namespace moe355;

extern "C" int gemm_fp8_blockscale(const uint8_t* a8, const float* a_scale, int64_t sstride_m, int64_t sstride_kb,
                                   const uint8_t* b8, const float* b_scale, int M, int N, int K, uint16_t* c,
                                   int64_t ldc, hipStream_t stream) {
  MOE355_CHECK(M >= 0 && N >= 0 && K >= 0 && ldc >= N, MOE355_EINVAL);
  MOE355_CHECK(K % 128 == 0 && N % 128 == 0, MOE355_EUNSUPPORTED);
  if (M == 0 || N == 0) return MOE355_OK;
  MOE355_CHECK(K > 0 && a8 && a_scale && b8 && b_scale && c && sstride_m >= 0 && sstride_kb >= 0, MOE355_EINVAL);
  MOE355_CHECK(aligned16(a8) && aligned16(b8) && (reinterpret_cast<uintptr_t>(c) & 1u) == 0, MOE355_EMISALIGNED);
  GemmArgs g{};
  g.a = a8;
  g.a_scale = a_scale;
  g.ssm = sstride_m;
  g.sskb = sstride_kb;
  g.b = b8;
  g.b_scale = b_scale;
  g.M = M;
  g.N = N;
  g.K = K;
  g.c = c;
  g.ldc = ldc;
  const int bm = M <= 16 ? 16 : M <= 32 ? 32 : M <= 64 ? 64 : 128;
  return launch_gemm<kDense>(g, bm, ceil_div64(M, bm), stream);
}

extern "C" int moe_fp8_blockscale_g1u1(const uint8_t* a8, const float* a_scale, int64_t sstride_m, int64_t sstride_kb,
                                       const uint8_t* w1, const float* w1_scale, const int32_t* sorted_ids,
                                       const int32_t* sorted_expert_ids, const int32_t* num_valid, int T, int H,
                                       int I, int E, int topk, int block_m, int64_t max_sorted, uint8_t* h8,
                                       float* h_scale, hipStream_t stream) {
  MOE355_CHECK(T >= 0 && H > 0 && I > 0 && E > 0 && topk > 0, MOE355_EINVAL);
  MOE355_CHECK(H % 128 == 0 && I % 128 == 0 && valid_block_m(block_m), MOE355_EUNSUPPORTED);
  const int cap = check_sorted_capacity(T, topk, E, block_m, max_sorted);
  if (cap != MOE355_OK) return cap;
  if (T == 0) return MOE355_OK;
  MOE355_CHECK(a8 && a_scale && w1 && w1_scale && sorted_ids && sorted_expert_ids && num_valid && h8 && h_scale,
               MOE355_EINVAL);
  MOE355_CHECK(sstride_m >= 0 && sstride_kb >= 0, MOE355_EINVAL);
  MOE355_CHECK(aligned16(a8) && aligned16(w1) && aligned16(h8), MOE355_EMISALIGNED);
  GemmArgs g{};
  g.a = a8;
  g.a_scale = a_scale;
  g.ssm = sstride_m;
  g.sskb = sstride_kb;
  g.b = w1;
  g.b_scale = w1_scale;
  g.sorted_ids = sorted_ids;
  g.sorted_eids = sorted_expert_ids;
  g.num_valid = num_valid;
  g.N = I;
  g.K = H;
  g.T = T;
  g.topk = topk;
  g.h8 = h8;
  g.h_scale = h_scale;
  return launch_gemm<kG1U1>(g, block_m, max_sorted / block_m, stream);
}

extern "C" int moe_down_combine_workspace(int T, int H, int topk, size_t* bytes) {
  MOE355_CHECK(T >= 0 && H > 0 && topk > 0 && bytes, MOE355_EINVAL);
  *bytes = (size_t)T * topk * H * sizeof(float) + 256;
  return MOE355_OK;
}

extern "C" int moe_down_combine(const uint8_t* h8, const float* h_scale, const uint8_t* w2, const float* w2_scale,
                                const int32_t* sorted_ids, const float* sorted_weights,
                                const int32_t* sorted_expert_ids, const int32_t* num_valid, int T, int H, int I,
                                int E, int topk, int block_m, int64_t max_sorted, uint16_t* out, int64_t ld_out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  MOE355_CHECK(T >= 0 && H > 0 && I > 0 && E > 0 && topk > 0 && ld_out >= H, MOE355_EINVAL);
  MOE355_CHECK(H % 128 == 0 && I % 128 == 0 && valid_block_m(block_m), MOE355_EUNSUPPORTED);
  const int cap = check_sorted_capacity(T, topk, E, block_m, max_sorted);
  if (cap != MOE355_OK) return cap;
  if (T == 0) return MOE355_OK;
  MOE355_CHECK(h8 && h_scale && w2 && w2_scale && sorted_ids && sorted_weights && sorted_expert_ids && num_valid &&
                   out && workspace,
               MOE355_EINVAL);
  size_t need = 0;
  moe_down_combine_workspace(T, H, topk, &need);
  MOE355_CHECK(workspace_bytes >= need, MOE355_EINVAL);
  MOE355_CHECK(aligned16(h8) && aligned16(w2) && aligned16(out) && aligned16(workspace) && ld_out % 8 == 0,
               MOE355_EMISALIGNED);
  GemmArgs g{};
  g.a = h8;
  g.a_scale = h_scale;
  g.ssm = I / 128;
  g.sskb = 1;
  g.b = w2;
  g.b_scale = w2_scale;
  g.sorted_ids = sorted_ids;
  g.sorted_eids = sorted_expert_ids;
  g.num_valid = num_valid;
  g.sorted_w = sorted_weights;
  g.N = H;
  g.K = I;
  g.T = T;
  g.topk = topk;
  g.y = static_cast<float*>(workspace);
  int st = launch_gemm<kDown>(g, block_m, max_sorted / block_m, stream);
  if (st != MOE355_OK) return st;
  const int64_t threads = (int64_t)T * (H / 8);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)ceil_div64(threads, 256)), dim3(256), 0, stream, g.y, T, topk, H,
                     out, ld_out);
  return launch_status();
}
