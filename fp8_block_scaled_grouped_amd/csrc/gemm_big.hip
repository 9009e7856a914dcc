// The grouped GEMMs of the MoE layer on 256 x 256 tiles (block_m 256), with the
// weight rows as the MFMA's row operand ("Accelerate DeepSeek-R1 Inference:
// Integrate AITER into SGLang", section "Blockscale FP8 MoE Computation": one
// activation scale per 1x128, one weight scale per 128x128).
//
// A workgroup computes 256 activation rows (sorted token-expert pairs of one
// expert) against 256 weight rows: down, 256 output columns; g1u1, the 128 gate
// rows of 128 output columns and the matching 128 up rows.  Per 128-wide K step it
// moves 64 KB into LDS for 16.8 MFLOP, 1.5x less data per flop than a 128 x 256
// tile, which matters because the rate at which a CU fills its LDS, not the matrix
// cores, bounds these GEMMs.
//
// Wave w owns weight rows [128 wb, 128 wb + 128) (wb = w / 4: down, half of the
// columns; g1u1, gate or up) against activation rows [64 wa, 64 wa + 64)
// (wa = w % 4): 8 x 4 MFMA tiles, 128 fp32 accumulators per lane.  Its 128 weight
// rows fall in one 128 x 128 scale block, so the block-scale fold
// acc += tile * (a_scale(row) * w_scale) takes one product per activation tile
// and step.  A step reads the wave's 4 activation fragments once and streams its
// 8 weight fragments one ahead, 4 MFMAs per weight fragment.
//
// Data movement: two LDS stages of [activations 32 KB | weights 32 KB |
// activation scales 1 KB], filled by LDS-DMA (each wave issues 4 + 4 + 1
// instructions per step, spread between its MFMAs); stage kb + 1 is fetched
// during step kb.  A step starts with the wave's own DMA wait and one barrier,
// which both publishes stage kb and frees stage kb + 1 (everyone finished step
// kb - 1).  Blocks of 8 activation rows that hold only padding are not fetched,
// and waves whose 64 rows are all padding skip their MFMAs.
#include <type_traits>

#include "device_common.h"
#include "gemm_engine.h"
#include "host_common.h"

namespace moe355 {
namespace {

constexpr int kBT = 256;                  // activation rows per tile
constexpr int kBW = 256;                  // weight rows per tile
constexpr int kNW = 8;                    // waves
constexpr int kThr = kNW * 64;
constexpr int kXBytes = kBT * 128;        // one K block of the activation rows
constexpr int kWOff = kXBytes;            // weight rows of a stage
constexpr int kSOff = kXBytes + kBW * 128;  // activation scales of a stage
constexpr int kStage = kSOff + kBT * 4;
constexpr int kLdsBytes = 2 * kStage;
constexpr int kXDma = kBT / 8 / kNW;      // activation DMAs per wave and step (8 rows each)
constexpr int kWDma = kBW / 8 / kNW;      // weight DMAs per wave and step
constexpr int kOps = kXDma + kWDma + 1;   // + one activation-scale DMA
constexpr int kWT = 8;                    // weight tiles (16 rows) per wave
constexpr int kAT = 4;                    // activation tiles (16 rows) per wave
constexpr int kHRS = 144;                 // g1u1 epilogue: row stride of the staged codes (bytes)
static_assert(kBT * kHRS <= kLdsBytes, "g1u1 code staging fits");
static_assert(4 * kWT * kAT * 64 * 16 <= kLdsBytes, "g1u1 up-tile exchange fits");
static_assert(kOps < 64, "vmcnt range");

template <int MODE, bool BSH>
__global__ __launch_bounds__(kThr) void big_gemm_kernel(GemmArgs g) {
  static_assert(MODE == kG1U1 || MODE == kDown, "grouped GEMMs only");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  __shared__ int rowinfo[kBT];   // sorted pair index of each activation row
  __shared__ float rowval[kBT];  // down: routing weight of each row; g1u1: scale of its h

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wa = w & 3, wb = w >> 2;
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

  // scale row of this wave's 128 weight rows; lane L holds K blocks L and L + 64
  const float* sbp;
  if constexpr (MODE == kG1U1) {
    const int64_t nbi = g.N / 128;
    sbp = g.b_scale + ((int64_t)expert * 2 * nbi + wb * nbi + nt) * KB;
  } else {
    sbp = g.b_scale + ((int64_t)expert * (g.N / 128) + 2 * nt + wb) * KB;
  }
  const float sb0 = lane < KB ? sbp[lane] : 0.0f;
  const float sb1 = lane + 64 < KB ? sbp[lane + 64] : 0.0f;

  if (tid < kBT) {
    rowinfo[tid] = g.sorted_ids[row0 + tid];
    if constexpr (MODE == kDown) rowval[tid] = g.sorted_w[row0 + tid];
  }
  __syncthreads();
  // valid rows form a prefix of the block (padding sits at the end of an expert's segment)
  const int nrows =
      __builtin_amdgcn_readfirstlane(__syncthreads_count(tid < kBT && rowinfo[tid < kBT ? tid : 0] < npairs));
  // this wave's activation tiles that hold a valid row
  const int atl = __builtin_amdgcn_readfirstlane(min(kAT, max(0, (nrows - 64 * wa + 15) / 16)));

  // activation row r of the tile -> row of the A operand
  auto x_row = [&](int r) -> int64_t {
    if constexpr (MODE == kG1U1) {
      const int pid = rowinfo[r];
      return pid < npairs ? pid / g.topk : 0;
    } else {
      return row0 + r;
    }
  };
  // weight row r (0..255) of the tile -> row inside the expert's weights
  auto w_row = [&](int r) -> int {
    if constexpr (MODE == kG1U1) {
      return r < 128 ? nt * 128 + r : g.N + nt * 128 + (r - 128);
    } else {
      return nt * kBW + r;
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

  // per-lane DMA offsets (fixed for the whole K loop).  DMA j of wave w moves the
  // 1 KB block q = w + 8 j (rows 8q .. 8q + 7): lane L the 16-byte chunk of row
  // 8q + L/8 that belongs in LDS slot L%8 (chunk c of row r sits in slot c ^ (r & 7)).
  // activation DMA j of wave (wa, wb) moves rows 64 wa + 16 j + 8 wb .. +8 (half of the
  // wave's activation tile j; wave (wa, 1 - wb) moves the other half): only the live
  // tiles of the quarter are fetched, so the DMA count per step is the compile-time ATL
  uint32_t voffx[kXDma];
#pragma unroll
  for (int j = 0; j < kXDma; ++j) {
    const int r = 64 * wa + 16 * j + 8 * wb + (lane >> 3);
    const int ch = (lane & 7) ^ (r & 7);
    voffx[j] = (uint32_t)(x_row(r) * g.K + ch * 16);
  }
  // weight DMA j moves rows 8 w + 64 j .. +8 of the tile: one per-lane offset for j = 0
  // and a wave-uniform byte offset per j (rows 64 j further on; g1u1: j >= 2 are up rows)
  uint32_t voffw;
  if constexpr (BSH) {
    // pre-shuffled 128 x 128-byte tiles: the 8 rows are one contiguous 1 KB block
    const int br0 = w_row(8 * w);
    voffw = (uint32_t)((int64_t)(br0 >> 7) * KB * (128 * 128) + (br0 & 127) * 128) + lane * 16;
  } else {
    const int r = 8 * w + (lane >> 3);
    voffw = (uint32_t)((int64_t)w_row(r) * g.K + ((lane & 7) ^ (r & 7)) * 16);
  }
  auto w_jofs = [&](int j) -> int64_t {
    const int r0 = 8 * w + 64 * j;
    if constexpr (BSH) {
      const int br0 = w_row(r0), b0 = w_row(8 * w);
      return ((int64_t)(br0 >> 7) - (b0 >> 7)) * KB * (128 * 128) + ((br0 & 127) - (b0 & 127)) * 128;
    } else {
      return ((int64_t)w_row(r0) - w_row(8 * w)) * g.K;
    }
  };
  // activation-scale DMA: waves w and w + 4 both move the scales of rows [64 (w % 4), +64)
  const uint32_t soff = (uint32_t)(x_row(wa * 64 + lane) * g.ssm * 4);
  constexpr int64_t kWStep = BSH ? 128 * 128 : 128;  // bytes between K blocks of a weight row

  vm_wait<0>();  // every ordinary load lands before the first DMA is queued
  const uint32_t lds0 = lds_addr(lds);
  int64_t wofs[kWDma];  // wave-uniform byte offsets of the weight DMAs
#pragma unroll
  for (int j = 0; j < kWDma; ++j) wofs[j] = w_jofs(j);
  // DMA op j of step kb into stage `stage` with ATL live activation tiles: ops
  // [0, ATL) activations, [ATL, ATL + 4) weights, then (ATL > 0) the activation scales
  auto issue_op = [&](int stage, int kb, auto atl_c, int j) {
    constexpr int ATL = decltype(atl_c)::value;
    const uint32_t base = lds0 + stage * kStage;
    if (j < ATL) {
      dma16(a_base + (int64_t)kb * 128, voffx[j], base + (8 * wa + 2 * j + wb) * 1024);
    } else if (j < ATL + kWDma) {
      const int jw = j - ATL;
      dma16(uniform_ptr(b_base + (int64_t)kb * kWStep + wofs[jw]), voffw, base + kWOff + (w + jw * kNW) * 1024);
    } else {
      dma4(s_base + (int64_t)kb * g.sskb * 4, soff, base + kSOff + wa * 256);
    }
  };
  auto n_ops = [](auto atl_c) { return decltype(atl_c)::value + kWDma + (decltype(atl_c)::value > 0 ? 1 : 0); };
  auto issue = [&](int stage, int kb, auto atl_c) {
#pragma unroll
    for (int j = 0; j < n_ops(atl_c); ++j) issue_op(stage, kb, atl_c, j);
  };

  v4f acc[kWT][kAT];
#pragma unroll
  for (int i = 0; i < kWT; ++i)
#pragma unroll
    for (int t = 0; t < kAT; ++t) acc[i][t] = v4f{0.f, 0.f, 0.f, 0.f};

  // one K step on stage PAR = kb % 2 with ATL live activation tiles; RF: the step
  // fetches stage kb + 1 (a compile-time flag, so that the MFMA sequence has no branch)
  auto step = [&](const int kb, auto atl_c, auto par_c, auto rf_c) {
    constexpr int ATL = decltype(atl_c)::value;
    constexpr int PAR = decltype(par_c)::value;
    constexpr bool RF = decltype(rf_c)::value != 0;
    vm_wait<0>();
    barrier_only();
    if constexpr (ATL == 0) {
      if constexpr (RF) issue(PAR ^ 1, kb + 1, atl_c);
    } else {
      const uint8_t* st = lds + PAR * kStage;
      const float sb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(kb < 64 ? sb0 : sb1), kb & 63));
      v8i xf[ATL];
      float s[ATL];
#pragma unroll
      for (int t = 0; t < ATL; ++t) {
        xf[t] = lds_frag(st, 64 * wa + 16 * t, lane);
        s[t] = *reinterpret_cast<const float*>(st + kSOff + (64 * wa + 16 * t + lr) * 4) * sb;
      }
      v8i wf[2];
      wf[0] = lds_frag(st + kWOff, 128 * wb, lane);
      // MFMA q covers weight tile q / ATL with activation tile q % ATL; the fold of
      // q - 2 follows MFMA q.  The next stage's DMAs are spread between the MFMAs (a
      // DMA instruction waits until the CU's memory pipeline takes it: issued in one
      // burst they would hold back this wave's MFMAs)
      constexpr int NQ = kWT * ATL;
      constexpr int NOPS = ATL + kWDma + 1;
      constexpr int kGap = 1;
      v4f tq[3];
#pragma unroll
      for (int q = 0; q < NQ + 2; ++q) {
        const int wt = q / ATL, t = q % ATL;
        if (q < NQ && t == 0 && wt + 1 < kWT) wf[(wt + 1) & 1] = lds_frag(st + kWOff, 128 * wb + 16 * (wt + 1), lane);
        if (q < NQ) tq[q % 3] = mfma16x16x128_fp8(wf[wt & 1], xf[t], v4f{0.f, 0.f, 0.f, 0.f});
        if constexpr (RF) {
#pragma unroll
          for (int j = 0; j < NOPS; ++j)
            if (q == (1 + j * kGap < NQ + 1 ? 1 + j * kGap : NQ + 1)) issue_op(PAR ^ 1, kb + 1, atl_c, j);
        }
        if (q >= 2) {
          const int p = q - 2;
          acc[p / ATL][p % ATL] += tq[p % 3] * s[p % ATL];
        }
        // keep the program order (MFMA q, the fold of q - 2): left to itself the
        // scheduler runs MFMAs ahead of their folds and runs out of registers
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto kloop = [&](auto atl_c) {
    using One = std::integral_constant<int, 1>;
    using Zero = std::integral_constant<int, 0>;
    issue(0, 0, atl_c);
    int kb = 0;
    for (; kb + 2 < KB; kb += 2) {  // both steps fetch the next stage
      step(kb, atl_c, Zero{}, One{});
      step(kb + 1, atl_c, One{}, One{});
    }
    if (kb + 1 < KB) {  // the last two steps
      step(kb, atl_c, Zero{}, One{});
      step(kb + 1, atl_c, One{}, Zero{});
    } else {  // the last step
      step(kb, atl_c, Zero{}, Zero{});
    }
  };
  switch (atl) {
    case 0: kloop(std::integral_constant<int, 0>{}); break;
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    default: kloop(std::integral_constant<int, 4>{}); break;
  }
  vm_wait<0>();
  __syncthreads();

  // ---- epilogues (LDS is free again).  acc[wt][t][i]: weight row 128 wb + 16 wt + 4 lg + i
  // of the tile (g1u1: gate (wb 0) or up (wb 1) of column 16 wt + 4 lg + i), activation
  // row 64 wa + 16 t + lr.
  if constexpr (MODE == kDown) {
    // routing-weighted fp32 rows per flat pair: each lane stores 4 consecutive columns
    // (non-temporal: the combine reads them once)
#pragma unroll
    for (int t = 0; t < kAT; ++t) {
      const int r = 64 * wa + 16 * t + lr;
      const int pid = rowinfo[r];
      if (pid < npairs) {
        const float wgt = rowval[r];
        float* yr = g.y + (int64_t)pid * g.N + nt * kBW + 128 * wb + 4 * lg;
#pragma unroll
        for (int wt = 0; wt < kWT; ++wt) __builtin_nontemporal_store(acc[wt][t] * wgt, reinterpret_cast<v4f*>(yr + 16 * wt));
      }
    }
  } else {
    // the up waves hand their tiles to the gate waves of the same rows (same lane layout);
    // a gate wave then holds all 128 columns of its 64 rows: h = SiLU(gate) * up (times
    // the smoothing factors of its columns), the row's |h| maximum (in registers and over
    // the 4 lane groups), its 1x128 scale, and the e4m3 codes staged in LDS for row stores
    v4f* ex = reinterpret_cast<v4f*>(lds);
    if (wb == 1) {
#pragma unroll
      for (int wt = 0; wt < kWT; ++wt)
#pragma unroll
        for (int t = 0; t < kAT; ++t) ex[((wa * kWT + wt) * kAT + t) * 64 + lane] = acc[wt][t];
    }
    __syncthreads();
    float sc[kAT];
    if (wb == 0) {
      const float* sm = g.smooth ? g.smooth + (int64_t)expert * g.N + nt * 128 + 4 * lg : nullptr;
#pragma unroll
      for (int t = 0; t < kAT; ++t) {
        float mx = 0.0f;
#pragma unroll
        for (int wt = 0; wt < kWT; ++wt) {
          const v4f up = ex[((wa * kWT + wt) * kAT + t) * 64 + lane];
          const v4f f = sm ? *reinterpret_cast<const v4f*>(sm + 16 * wt) : v4f{1.f, 1.f, 1.f, 1.f};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gt = acc[wt][t][i];
            float h = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up[i];
            if (sm) h = h * f[i];
            acc[wt][t][i] = h;
            mx = fmaxf(mx, fabsf(h));
          }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        sc[t] = (mx == 0.0f) ? 1.0f : mx / kE4M3Max;
      }
    }
    __syncthreads();  // the exchanged tiles are consumed
    uint8_t* hq = lds;
    if (wb == 0) {
#pragma unroll
      for (int t = 0; t < kAT; ++t) {
        const int r = 64 * wa + 16 * t + lr;
        if (lg == 0) rowval[r] = sc[t];
#pragma unroll
        for (int wt = 0; wt < kWT; ++wt) {
          const v4f h = acc[wt][t];
          *reinterpret_cast<uint32_t*>(hq + r * kHRS + 16 * wt + 4 * lg) =
              f32x4_to_e4m3(h[0] / sc[t], h[1] / sc[t], h[2] / sc[t], h[3] / sc[t]);
        }
      }
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
