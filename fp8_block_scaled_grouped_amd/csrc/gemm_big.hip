// The grouped GEMMs of the MoE layer on 256 x 256 tiles (block_m 256), with the
// weight rows as the MFMA's row operand ("Accelerate DeepSeek-R1 Inference:
// Integrate AITER into SGLang", section "Blockscale FP8 MoE Computation": one
// activation scale per 1x128, one weight scale per 128x128).
//
// A workgroup computes 256 activation rows (sorted token-expert pairs of one
// expert) against 256 weight rows.  Wave w owns 32 weight rows --
// rows [32w, 32w+32) of the tile, or for g1u1 the 16 gate rows of output columns
// [16w, 16w+16) and the 16 up rows of the same columns -- and runs them against
// all 256 activation rows, so the tile holds 256 x 256 fp32 results in 128
// registers per lane.  The MFMA computes (weight rows) x (activation rows): a
// lane then holds 4 weight rows of one activation row, so the block-scale fold
// acc += tile * (a_scale(row) * w_scale) takes one scale product per lane and
// 16-row tile, shared by the tile's two MFMAs.
//
// Data movement (LDS-DMA, as in gemm.hip):
//   activations  two LDS stages of 32 KB (+ their scales), shared by the 8 waves,
//                published by a barrier; stage kb+1 is fetched during step kb.
//   weights      each wave's 32 rows go to its own LDS slots (4 KB per K block,
//                two slots); a wave reads its fragments into registers at the
//                start of a step, so slot kb%2 takes the rows of step kb+2:
//                the weight stream, which mostly misses L2, runs two steps ahead.
// Each wave waits for its own DMAs with s_waitcnt vmcnt (activation DMAs of a
// step are issued before its weight DMAs, so one count covers both).
#include <type_traits>

#include "device_common.h"
#include "gemm_engine.h"
#include "host_common.h"

namespace moe355 {
namespace {

constexpr int kBT = 256;                          // activation rows per tile
constexpr int kBW = 256;                          // weight rows per tile
constexpr int kNW = 8;                            // waves
constexpr int kThr = kNW * 64;
constexpr int kXT = kBT / 16;                     // 16-row activation tiles
constexpr int kXBytes = kBT * 128;                // one K block of the activation rows
constexpr int kSOff = kXBytes;                    // activation scales of a stage (wave w: 256 B at w*256)
constexpr int kXStage = kXBytes + kNW * 256;
constexpr int kWOff = 2 * kXStage;                // weight slots: [slot][wave] 4 KB each
constexpr int kWSlot = 32 * 128;
constexpr int kPipe = kWOff + 2 * kNW * kWSlot;
constexpr int kXDma = kBT / 8 / kNW;              // activation DMAs per wave and step (8 rows each)
constexpr int kXOps = kXDma + 1;                  // + the scale DMA
constexpr int kWDma = 32 / 8;                     // weight DMAs per wave and step
constexpr int kLdsBytes = kPipe;
constexpr int kHRS = 144;                         // g1u1 epilogue: row stride of the staged codes (bytes)
static_assert(kBT * kHRS <= kLdsBytes, "g1u1 code staging fits");
static_assert(kXOps + kWDma < 64, "vmcnt range");

template <int MODE, bool BSH>
__global__ __launch_bounds__(kThr) void big_gemm_kernel(GemmArgs g) {
  static_assert(MODE == kG1U1 || MODE == kDown, "grouped GEMMs only");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  __shared__ int rowinfo[kBT];    // sorted pair index of each activation row (grouped modes)
  __shared__ float rowval[kBT];   // down: routing weight of each row; g1u1: scale of its h
  __shared__ float red[kNW][kBT];  // g1u1: per-wave maxima of |h| per row

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int KB = g.K / 128;
  const int npairs = g.T * g.topk;
  const int NT = MODE == kG1U1 ? g.N / 128 : g.N / kBW;
  const int nvalid = g.num_valid[0];
  const int64_t total = nvalid > 0 ? (int64_t)(nvalid / kBT) * NT : 0;
  const int64_t tile = blockIdx.x;
  if (tile >= total) return;  // uniform: blocks past num_valid hold no rows
  const int nt = (int)(tile % NT);
  const int mb = (int)(tile / NT);
  const int64_t row0 = (int64_t)mb * kBT;
  const int expert = g.sorted_eids[mb];

  // weight-scale rows of this wave (g1u1: gate block, up block; else one block for both tiles)
  const float* sbp_g;
  const float* sbp_u;
  if constexpr (MODE == kG1U1) {
    const int64_t nbi = g.N / 128;
    sbp_g = g.b_scale + ((int64_t)expert * 2 * nbi + nt) * KB;
    sbp_u = g.b_scale + ((int64_t)expert * 2 * nbi + nbi + nt) * KB;
  } else {
    sbp_g = sbp_u = g.b_scale + ((int64_t)expert * (g.N / 128) + (nt * kBW + 32 * w) / 128) * KB;
  }
  // lane L holds the scales of K blocks L and L + 64 (at most 128 blocks); read per step with readlane
  const float sg0 = lane < KB ? sbp_g[lane] : 0.0f;
  const float sg1 = lane + 64 < KB ? sbp_g[lane + 64] : 0.0f;
  const float su0 = MODE == kG1U1 && lane < KB ? sbp_u[lane] : sg0;
  const float su1 = MODE == kG1U1 && lane + 64 < KB ? sbp_u[lane + 64] : sg1;

  if (tid < kBT) {
    rowinfo[tid] = g.sorted_ids[row0 + tid];
    if constexpr (MODE == kDown) rowval[tid] = g.sorted_w[row0 + tid];
  }
  __syncthreads();
  // valid rows form a prefix of the block (padding sits at the end of an expert's segment)
  const int nrows = __syncthreads_count(tid < kBT && rowinfo[tid < kBT ? tid : 0] < npairs);
  // activation row tiles holding a valid row, rounded up to an even count
  const int xt_live = __builtin_amdgcn_readfirstlane(min(kXT, ((nrows + 31) / 32) * 2));

  // activation row r of the tile -> row of the A operand
  auto x_row = [&](int r) -> int64_t {
    if constexpr (MODE == kG1U1) {
      const int pid = rowinfo[r];
      return pid < npairs ? pid / g.topk : 0;
    } else {
      return row0 + r;
    }
  };
  // this wave's weight row r (0..31) -> row inside the B base of the workgroup
  auto w_row = [&](int r) -> int {
    if constexpr (MODE == kG1U1) {
      return r < 16 ? nt * 128 + 16 * w + r : g.N + nt * 128 + 16 * w + (r - 16);
    } else {
      return nt * kBW + 32 * w + r;
    }
  };
  const uint8_t* a_base = uniform_ptr(g.a);
  const uint8_t* b_base;
  if constexpr (MODE == kG1U1) {
    b_base = uniform_ptr(g.b + (int64_t)expert * 2 * g.N * g.K);
  } else {
    b_base = uniform_ptr(g.b + (int64_t)expert * g.N * g.K);
  }
  const uint8_t* s_base = uniform_ptr(g.a_scale);

  // per-lane DMA offsets (fixed for the whole K loop).  A 1 KB block q of 8 rows:
  // lane L moves the 16-byte chunk of row 8q + L/8 that belongs in LDS slot L%8
  // (chunk c of row r sits in slot c ^ (r & 7)).
  uint32_t voffx[kXDma], voffw[kWDma];
#pragma unroll
  for (int j = 0; j < kXDma; ++j) {
    const int q = w + j * kNW;
    const int r = q * 8 + (lane >> 3);
    const int ch = (lane & 7) ^ (r & 7);
    // a block of 8 rows past the valid ones reads 16 bytes of the first row into every slot
    voffx[j] = q * 8 < nrows ? (uint32_t)(x_row(r) * g.K + ch * 16) : 0u;
  }
#pragma unroll
  for (int j = 0; j < kWDma; ++j) {
    const int r = j * 8 + (lane >> 3);
    if constexpr (BSH) {
      // pre-shuffled 128 x 128-byte tiles: the 8 rows are one contiguous 1 KB block
      const int br0 = w_row(j * 8);
      voffw[j] = (uint32_t)((int64_t)(br0 >> 7) * KB * (128 * 128) + (br0 & 127) * 128) + lane * 16;
    } else {
      voffw[j] = (uint32_t)((int64_t)w_row(r) * g.K + ((lane & 7) ^ (r & 7)) * 16);
    }
  }
  // scale DMA: waves w and w + 4 both move the scales of rows [64 (w % 4), 64 (w % 4) + 64);
  // consumers read the first 1 KB
  const uint32_t soff = (uint32_t)(x_row((w & 3) * 64 + lane) * g.ssm * 4);
  constexpr int64_t kWStep = BSH ? 128 * 128 : 128;  // bytes between K blocks of a weight row

  vm_wait<0>();  // every ordinary load lands before the first DMA is queued
  const uint32_t lds0 = lds_addr(lds);
  auto issue_x = [&](int stage, int kb, int j) {
    const uint32_t base = lds0 + stage * kXStage;
    if (j < kXDma) {
      dma16(a_base + (int64_t)kb * 128, voffx[j], base + (w + j * kNW) * 1024);
    } else {
      dma4(s_base + (int64_t)kb * g.sskb * 4, soff, base + kSOff + w * 256);
    }
  };
  auto issue_w = [&](int slot, int kb, int j) {
    dma16(b_base + (int64_t)kb * kWStep, voffw[j], lds0 + kWOff + (slot * kNW + w) * kWSlot + j * 1024);
  };

  v4f acc[2][kXT];
#pragma unroll
  for (int t = 0; t < kXT; ++t) acc[0][t] = acc[1][t] = v4f{0.f, 0.f, 0.f, 0.f};

  // prologue: activations of step 0, weights of steps 0 and 1
#pragma unroll
  for (int j = 0; j < kXOps; ++j) issue_x(0, 0, j);
#pragma unroll
  for (int j = 0; j < kWDma; ++j) issue_w(0, 0, j);
  if (KB > 1) {
#pragma unroll
    for (int j = 0; j < kWDma; ++j) issue_w(1, 1, j);
  }

  // one K step on stage / slot PAR = kb % 2 with TMV live activation tiles.  RF 1: a
  // steady-state step (steps kb + 1 and kb + 2 exist: both refills, no branches);
  // RF 0: the refills are checked
  auto step = [&](const int kb, auto tmv_c, auto par_c, auto rf_c) {
    constexpr int TMV = decltype(tmv_c)::value;
    constexpr int PAR = decltype(par_c)::value;
    constexpr int RF = decltype(rf_c)::value;
    // outstanding after this step's data: the weight DMAs of step kb + 1, if issued
    if (RF == 1 || kb + 1 < KB) {
      vm_wait<kWDma>();
    } else {
      vm_wait<0>();
    }
    barrier_only();
    const bool rx = RF == 1 || kb + 1 < KB, rw = RF == 1 || kb + 2 < KB;
    const uint8_t* st = lds + PAR * kXStage;
    const uint8_t* wsl = lds + kWOff + (PAR * kNW + w) * kWSlot;
    const v8i wv0 = lds_frag(wsl, 0, lane);
    const v8i wv1 = lds_frag(wsl, 16, lane);
    const float sbg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(kb < 64 ? sg0 : sg1), kb & 63));
    const float sbu = MODE == kG1U1
                          ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(kb < 64 ? su0 : su1), kb & 63))
                          : sbg;
    if constexpr (TMV == 0) {
      if (rx) {
#pragma unroll
        for (int j = 0; j < kXOps; ++j) issue_x(PAR ^ 1, kb + 1, j);
      }
      lgkm_wait0();  // the weight fragments are in registers before their slot is refilled
      if (rw) {
#pragma unroll
        for (int j = 0; j < kWDma; ++j) issue_w(PAR, kb + 2, j);
      }
    } else {
      v8i xv[TMV];
      float sa[TMV];
      auto load_x = [&](int t) {
        xv[t] = lds_frag(st, t * 16, lane);
        sa[t] = *reinterpret_cast<const float*>(st + kSOff + (t * 16 + lr) * 4);
      };
      load_x(0);
      // MFMA q covers activation tile q / 2 with weight tile q % 2; the fold of q - 2
      // follows MFMA q.  The refill DMAs are spread between the MFMAs, activation
      // DMAs first (op j after MFMA 1 + j * kGap): the weight DMAs of slot PAR come
      // after the first MFMAs, which have waited for the fragments read from that slot.
      constexpr int NQ = 2 * TMV;
      constexpr int kOps = kXOps + kWDma;
      constexpr int kGap = NQ / kOps > 0 ? NQ / kOps : 1;
      v4f tq[3];
#pragma unroll
      for (int q = 0; q < NQ + 2; ++q) {
        const int t = q >> 1, wt = q & 1;
        if (q < NQ && wt == 0 && t + 1 < TMV) load_x(t + 1);
        if (q < NQ) tq[q % 3] = mfma16x16x128_fp8(wt ? wv1 : wv0, xv[t], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int j = 0; j < kOps; ++j) {
          const int at = 1 + j * kGap < NQ + 1 ? 1 + j * kGap : NQ + 1;
          if (at == q) {
            if (j < kXOps) {
              if (rx) issue_x(PAR ^ 1, kb + 1, j);
            } else if (rw) {
              issue_w(PAR, kb + 2, j - kXOps);
            }
          }
        }
        if (q >= 2) {
          const int p = q - 2, pt = p >> 1, pw = p & 1;
          acc[pw][pt] += tq[p % 3] * (sa[pt] * (pw ? sbu : sbg));
        }
      }
    }
  };
  auto kloop = [&](auto tmv_c) {
    using One = std::integral_constant<int, 1>;
    using Zero = std::integral_constant<int, 0>;
    int kb = 0;
    for (; kb + 3 < KB; kb += 2) {  // pairs of steps that refill both streams
      step(kb, tmv_c, Zero{}, One{});
      step(kb + 1, tmv_c, One{}, One{});
    }
    for (; kb < KB; kb += 2) {  // the last (at most three) steps
      step(kb, tmv_c, Zero{}, Zero{});
      if (kb + 1 < KB) step(kb + 1, tmv_c, One{}, Zero{});
    }
  };
  switch (xt_live) {
    case 0: kloop(std::integral_constant<int, 0>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 4: kloop(std::integral_constant<int, 4>{}); break;
    case 6: kloop(std::integral_constant<int, 6>{}); break;
    case 8: kloop(std::integral_constant<int, 8>{}); break;
    case 10: kloop(std::integral_constant<int, 10>{}); break;
    case 12: kloop(std::integral_constant<int, 12>{}); break;
    case 14: kloop(std::integral_constant<int, 14>{}); break;
    default: kloop(std::integral_constant<int, 16>{}); break;
  }
  vm_wait<0>();
  __syncthreads();

  // ---- epilogues (LDS is free again).  acc[wt][t][i]: weight row 32w + 16wt + 4lg + i
  // of the tile (g1u1: wt 0 gate, wt 1 up of column 16w + 4lg + i), activation row 16t + lr.
  if constexpr (MODE == kDown) {
    // routing-weighted fp32 rows per flat pair: each lane stores 4 consecutive columns
#pragma unroll
    for (int t = 0; t < kXT; ++t) {
      const int r = t * 16 + lr;
      const int pid = rowinfo[r];
      if (row0 + r < nvalid && pid < npairs) {
        const float wgt = rowval[r];
        float* yr = g.y + (int64_t)pid * g.N + nt * kBW + 32 * w + 4 * lg;
#pragma unroll
        for (int wt = 0; wt < 2; ++wt) *reinterpret_cast<v4f*>(yr + 16 * wt) = acc[wt][t] * wgt;
      }
    }
  } else {
    // h = SiLU(gate) * up (times the smoothing factors of its columns), in registers;
    // the row's |h| maximum over the tile's 128 columns (4 values per lane, 4 lanes per
    // wave, 8 waves), its 1x128 scale, and the e4m3 codes staged in LDS for row stores
    const float* sm = g.smooth ? g.smooth + (int64_t)expert * g.N + nt * 128 + 16 * w + 4 * lg : nullptr;
    const v4f f = sm ? *reinterpret_cast<const v4f*>(sm) : v4f{1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int t = 0; t < kXT; ++t) {
      float mx = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gt = acc[0][t][i], up = acc[1][t][i];
        float h = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
        if (sm) h = h * f[i];
        acc[0][t][i] = h;
        mx = fmaxf(mx, fabsf(h));
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      if (lg == 0) red[w][t * 16 + lr] = mx;
    }
    __syncthreads();
    if (tid < kBT) {
      float amax = red[0][tid];
#pragma unroll
      for (int ww = 1; ww < kNW; ++ww) amax = fmaxf(amax, red[ww][tid]);
      rowval[tid] = (amax == 0.0f) ? 1.0f : amax / kE4M3Max;
    }
    __syncthreads();
    uint8_t* hq = lds;
#pragma unroll
    for (int t = 0; t < kXT; ++t) {
      const int r = t * 16 + lr;
      const float sc = rowval[r];
      const v4f h = acc[0][t];
      *reinterpret_cast<uint32_t*>(hq + r * kHRS + 16 * w + 4 * lg) =
          f32_to_e4m3(h[0] / sc) | (f32_to_e4m3(h[1] / sc) << 8) | (f32_to_e4m3(h[2] / sc) << 16) |
          (f32_to_e4m3(h[3] / sc) << 24);
    }
    __syncthreads();
    for (int ci = tid; ci < kBT * 8; ci += kThr) {
      const int r = ci >> 3, ch = ci & 7;
      if (rowinfo[r] < npairs)
        *reinterpret_cast<u32x4*>(g.h8 + (row0 + r) * g.N + nt * 128 + ch * 16) =
            *reinterpret_cast<const u32x4*>(hq + r * kHRS + ch * 16);
    }
    if (tid < kBT && rowinfo[tid] < npairs) g.h_scale[(row0 + tid) * (g.N / 128) + nt] = rowval[tid];
  }
}

}  // namespace

template <int MODE, bool BSH>
int launch_big(const GemmArgs& g, int64_t mblocks, hipStream_t stream) {
  if (g.K % 128 != 0 || g.K / 128 > 128) return MOE355_EUNSUPPORTED;
  if (MODE == kG1U1 && g.N % 128 != 0) return MOE355_EUNSUPPORTED;
  if (MODE == kDown && g.N % kBW != 0) return MOE355_EUNSUPPORTED;
  const int64_t nt = MODE == kG1U1 ? g.N / 128 : g.N / kBW;
  const int64_t grid = mblocks * nt;
  if (grid == 0) return MOE355_OK;
  MOE355_CHECK(grid < (1ll << 31), MOE355_EUNSUPPORTED);
  hipLaunchKernelGGL((big_gemm_kernel<MODE, BSH>), dim3((unsigned)grid), dim3(kThr), 0, stream, g);
  return launch_status();
}

template int launch_big<kG1U1, false>(const GemmArgs&, int64_t, hipStream_t);
template int launch_big<kG1U1, true>(const GemmArgs&, int64_t, hipStream_t);
template int launch_big<kDown, false>(const GemmArgs&, int64_t, hipStream_t);
template int launch_big<kDown, true>(const GemmArgs&, int64_t, hipStream_t);

}  // namespace moe355
