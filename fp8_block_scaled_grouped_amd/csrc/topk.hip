// Biased grouped top-k routing ("Accelerate DeepSeek-R1 Inference: Integrate
// AITER into SGLang", section "Complete MoE Implementation" / "Top-K routing").
//
// One wave64 per token.  The group ranking and the expert selection are rounds
// of a wave-wide arg-best under the key (value desc, index asc), so ties always
// go to the lower index.  Scores stay in registers when a group covers a
// power-of-two number of lanes (DeepSeek-V3: 256 experts, 8 groups -> 8 lanes
// of 4 experts); other group shapes take an LDS path.
#include <limits.h>

#include "device_common.h"
#include "host_common.h"

namespace moe355 {
namespace {

constexpr int kTokPerBlock = 4;
constexpr int kMaxE = 1024;

__device__ __forceinline__ bool key_better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// Wave-wide arg-best; every lane ends with the winner.
__device__ __forceinline__ void wave_argbest(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o, kWave);
    const int oi = __shfl_xor(i, o, kWave);
    if (key_better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}

// Fast path: lane L holds the P = E/64 (rounded up) contiguous experts
// L*P .. L*P+P-1 in registers; a group of E/n_group experts spans LPG = gsz/P
// consecutive lanes (a power of two), so the group top-2 is a butterfly merge.
// logit e of row x: fp32, or bf16 bits widened exactly
__device__ __forceinline__ float load_logit(const void* x, int e, bool bf16) {
  return bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(x)[e]) : reinterpret_cast<const float*>(x)[e];
}

template <int P>
__global__ __launch_bounds__(256) void grouped_topk_reg_kernel(
    const void* __restrict__ logits, int logits_bf16, int64_t ld_logits, const float* __restrict__ bias, int T, int E,
    int n_group, int topk_group, int topk, int renorm, float factor, float* __restrict__ topk_weights,
    int32_t* __restrict__ topk_ids, int64_t ld_topk, int lpg) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * kTokPerBlock + threadIdx.x / kWave;
  if (t >= T) return;  // whole wave
  const int e0 = lane * P;
  float s[P], b[P];
  const void* x = reinterpret_cast<const uint8_t*>(logits) + (int64_t)t * ld_logits * (logits_bf16 ? 2 : 4);
#pragma unroll
  for (int q = 0; q < P; ++q) {
    const int e = e0 + q;
    if (e < E) {
      const double d = 1.0 / (1.0 + exp(-(double)load_logit(x, e, logits_bf16 != 0)));
      s[q] = (float)d;
      b[q] = s[q] + bias[e];
    } else {
      s[q] = 0.0f;
      b[q] = -INFINITY;
    }
  }
  // group score = top1 + top2 of the biased scores (values only, so ties do not matter)
  float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll
  for (int q = 0; q < P; ++q) {
    if (b[q] > m1) {
      m2 = m1;
      m1 = b[q];
    } else if (b[q] > m2) {
      m2 = b[q];
    }
  }
  for (int o = 1; o < lpg; o <<= 1) {
    const float o1 = __shfl_xor(m1, o, kWave), o2 = __shfl_xor(m2, o, kWave);
    const float hi = fmaxf(m1, o1), lo = fmaxf(fminf(m1, o1), fmaxf(m2, o2));
    m1 = hi;
    m2 = lo;
  }
  const int grp = lane / lpg;
  const bool leader = (lane % lpg) == 0 && e0 < E;
  const float gs = m1 + m2;
  uint64_t gsel = 0;
  for (int r = 0; r < topk_group; ++r) {
    const bool avail = leader && !((gsel >> grp) & 1ull);
    float v = avail ? gs : -INFINITY;
    int i = avail ? grp : INT_MAX;
    wave_argbest(v, i);
    gsel |= 1ull << i;
  }
  const bool cand_lane = e0 < E && ((gsel >> grp) & 1ull);
  uint32_t taken = 0;
  int my_id = 0;
  for (int j = 0; j < topk; ++j) {
    float v = -INFINITY;
    int i = INT_MAX;
    if (cand_lane) {
#pragma unroll
      for (int q = 0; q < P; ++q)
        if (!((taken >> q) & 1u) && e0 + q < E && b[q] > v) {  // ascending e: strict > keeps the lower id
          v = b[q];
          i = e0 + q;
        }
    }
    wave_argbest(v, i);
    if (i / P == lane) taken |= 1u << (i - e0);
    if (lane == j) my_id = i;
  }
  // weights from the unbiased score of each chosen expert
  float wsel = 0.0f;
  const int owner = my_id / P;
  // fetch s[id] from the owning lane: every lane reads slot q of its owner, q = 0..P-1
#pragma unroll
  for (int q = 0; q < P; ++q) {
    const float sq = __shfl(s[q], owner, kWave);
    if (my_id - owner * P == q) wsel = sq;
  }
  float wv = (lane < topk) ? wsel : 0.0f;
  if (renorm) {
    float S = __shfl(wv, 0, kWave);
    for (int j = 1; j < topk; ++j) S = S + __shfl(wv, j, kWave);
    wv = wv / S;
  }
  wv = wv * factor;
  if (lane < topk) {
    topk_ids[(int64_t)t * ld_topk + lane] = my_id;
    topk_weights[(int64_t)t * ld_topk + lane] = wv;
  }
}

// General path (any group shape): scores in LDS, group top-2 by a scan per group.
__global__ __launch_bounds__(256) void grouped_topk_kernel(
    const void* __restrict__ logits, int logits_bf16, int64_t ld_logits, const float* __restrict__ bias, int T, int E,
    int n_group, int topk_group, int topk, int renorm, float factor, float* __restrict__ topk_weights,
    int32_t* __restrict__ topk_ids, int64_t ld_topk) {
  __shared__ float s_sh[kTokPerBlock][kMaxE];
  __shared__ float b_sh[kTokPerBlock][kMaxE];
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * kTokPerBlock + w;
  const bool live = t < T;
  const int gsz = E / n_group;

  // scores: fl32 of the binary64 logistic, then the biased score in fp32
  if (live) {
    const void* x = reinterpret_cast<const uint8_t*>(logits) + (int64_t)t * ld_logits * (logits_bf16 ? 2 : 4);
    for (int e = lane; e < E; e += kWave) {
      const double d = 1.0 / (1.0 + exp(-(double)load_logit(x, e, logits_bf16 != 0)));
      const float s = (float)d;
      s_sh[w][e] = s;
      b_sh[w][e] = s + bias[e];
    }
  }
  __syncthreads();
  if (!live) return;

  // group score = top1 + top2 of the biased scores; lane g owns group g
  float gs = -INFINITY;
  if (lane < n_group) {
    float m1 = -INFINITY, m2 = -INFINITY;
    const float* bg = &b_sh[w][lane * gsz];
    for (int q = 0; q < gsz; ++q) {
      const float v = bg[q];
      if (v > m1) {
        m2 = m1;
        m1 = v;
      } else if (v > m2) {
        m2 = v;
      }
    }
    gs = m1 + m2;
  }
  uint64_t gsel = 0;
  for (int r = 0; r < topk_group; ++r) {
    float v = (lane < n_group && !((gsel >> lane) & 1ull)) ? gs : -INFINITY;
    int i = (lane < n_group && !((gsel >> lane) & 1ull)) ? lane : INT_MAX;
    wave_argbest(v, i);
    gsel |= 1ull << i;
  }

  // experts e = lane + 64*q; candidates are the experts of the kept groups
  const int nq = (E + kWave - 1) / kWave;
  uint32_t cand = 0;
  for (int q = 0; q < nq; ++q) {
    const int e = lane + kWave * q;
    if (e < E && ((gsel >> (e / gsz)) & 1ull)) cand |= 1u << q;
  }
  int my_id = 0;
  for (int j = 0; j < topk; ++j) {
    float v = -INFINITY;
    int i = INT_MAX;
    for (int q = 0; q < nq; ++q) {
      if ((cand >> q) & 1u) {
        const int e = lane + kWave * q;
        const float bv = b_sh[w][e];
        if (key_better(bv, e, v, i)) {
          v = bv;
          i = e;
        }
      }
    }
    wave_argbest(v, i);
    if ((i % kWave) == lane) cand &= ~(1u << (i / kWave));
    if (lane == j) my_id = i;
  }

  // weights from the unbiased score; optional renorm (fp32, left to right); factor
  float wv = (lane < topk) ? s_sh[w][my_id] : 0.0f;
  if (renorm) {
    float S = __shfl(wv, 0, kWave);
    for (int j = 1; j < topk; ++j) S = S + __shfl(wv, j, kWave);
    wv = wv / S;
  }
  wv = wv * factor;
  if (lane < topk) {
    topk_ids[(int64_t)t * ld_topk + lane] = my_id;
    topk_weights[(int64_t)t * ld_topk + lane] = wv;
  }
}

}  // namespace
}  // namespace moe355

using namespace moe355;

extern "C" int grouped_topk(const void* logits, int logits_bf16, int64_t ld_logits, const float* bias, int T, int E,
                            int n_group, int topk_group, int topk, int renorm, float routed_scaling_factor,
                            float* topk_weights, int32_t* topk_ids, int64_t ld_topk, hipStream_t stream) {
  MOE355_CHECK(T >= 0 && E > 0 && n_group > 0 && topk_group > 0 && topk > 0, MOE355_EINVAL);
  MOE355_CHECK(logits_bf16 == 0 || logits_bf16 == 1, MOE355_EINVAL);
  MOE355_CHECK(ld_logits >= E && ld_topk >= topk, MOE355_EINVAL);
  MOE355_CHECK(E <= kMaxE && n_group <= 64 && E % n_group == 0 && E / n_group >= 2, MOE355_EUNSUPPORTED);
  MOE355_CHECK(topk_group <= n_group && topk <= 32 && topk <= topk_group * (E / n_group), MOE355_EUNSUPPORTED);
  if (T == 0) return MOE355_OK;
  MOE355_CHECK(logits && bias && topk_weights && topk_ids, MOE355_EINVAL);
  const int blocks = (T + kTokPerBlock - 1) / kTokPerBlock;
  const int P = (E + kWave - 1) / kWave;
  const int gsz = E / n_group;
  const int lpg = gsz % P == 0 ? gsz / P : 0;
  if (lpg > 0 && (lpg & (lpg - 1)) == 0 && lpg <= kWave && P <= 16) {
#define MOE355_TOPK_REG(PP)                                                                                         \
  case PP:                                                                                                          \
    hipLaunchKernelGGL(grouped_topk_reg_kernel<PP>, dim3(blocks), dim3(kTokPerBlock * kWave), 0, stream, logits,    \
                       logits_bf16, ld_logits, bias, T, E, n_group, topk_group, topk, renorm, routed_scaling_factor,           \
                       topk_weights, topk_ids, ld_topk, lpg);                                                    \
    return launch_status();
    switch (P) {
      MOE355_TOPK_REG(1)
      MOE355_TOPK_REG(2)
      MOE355_TOPK_REG(4)
      MOE355_TOPK_REG(8)
      MOE355_TOPK_REG(16)
      default: break;
    }
#undef MOE355_TOPK_REG
  }
  hipLaunchKernelGGL(grouped_topk_kernel, dim3(blocks), dim3(kTokPerBlock * kWave), 0, stream, logits, logits_bf16,
                     ld_logits, bias, T, E, n_group, topk_group, topk, renorm, routed_scaling_factor, topk_weights, topk_ids,
                     ld_topk);
  return launch_status();
}
