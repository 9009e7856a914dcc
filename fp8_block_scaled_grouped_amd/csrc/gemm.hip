// Block-scaled FP8 GEMM engine on gfx950 FP8 MFMA.
//
// Each workgroup computes a BM x BNB tile of A[rows, K] * B[BNB rows, K]^T
// ("Accelerate DeepSeek-R1 Inference: Integrate AITER into SGLang", section
// "General Linear Layer": one activation scale per 1x128, one weight scale
// per 128x128).  The K loop walks 128-wide scale blocks.  Per block each wave
// runs 16x16x128 FP8 MFMAs into fresh fp32 tiles and folds every tile into
// its accumulators as acc += tile * (a_scale(row) * b_scale) two MFMAs after
// issuing it, so the fold overlaps the matrix pipe.
//
// Data movement: A and B tiles (and the per-row A scales) go HBM -> LDS by
// LDS-DMA (global_load_lds), S stages deep, with no VGPR staging.  Rows are
// 128 bytes in LDS, 16-byte chunk c of row r in slot c ^ (r & 7); one DMA
// instruction moves 8 whole rows (full 128-byte lines).  MFMA lane group g
// (lanes 16g..16g+15) takes K chunks g and g+4 of a 128-wide K block -- any K
// permutation shared by A and B leaves the product unchanged -- which makes
// the fragment reads free of LDS bank conflicts.  Each wave waits for its own
// DMAs with s_waitcnt vmcnt and a bare s_barrier publishes the stage.
//
// Modes:
//   dense  C[M, N] = A[M, K] B[N, K]^T, bf16 or fp16 out ("General Linear
//          Layer"); small M splits K over workgroups into fp32 partials that
//          a reduce kernel adds in a fixed order.
//   g1u1   grouped GEMM over the sorted token-expert pairs ("Complete MoE
//          Implementation" / "Blockscale FP8 MoE Computation"): A rows
//          gathered through sorted_ids, B = 128 gate rows and the matching 128
//          up rows of the block's expert; epilogue h = SiLU(gate) * up
//          (optionally times per-channel smoothing factors) and a 1x128 e4m3
//          requantisation of h.
//   down   grouped GEMM of h with the expert's down weights; each row is
//          scaled by its routing weight and stored per flat pair; a second
//          kernel sums each token's pairs in ascending order into bf16.
#include <algorithm>
#include <type_traits>

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
  const float* smooth;     // g1u1: optional per-expert channel factors for h [E, N] (fc2 smoothing)
  int splits, kbs;         // dense split-K: K blocks [ks*kbs, ks*kbs+kbs) per split ks
  int out_f16;             // dense: c holds fp16 (1) or bf16 (0) bits
  float* part;             // dense split-K partial sums [splits, M, N] fp32
};

// Tile configuration.  BNB = B rows staged per workgroup (g1u1: 128 gate + 128 up).
template <int MODE, int BM_, int BNB_, int NW_, int WM_, int S_>
struct Cfg {
  static constexpr int BM = BM_, BNB = BNB_, NW = NW_, WM = WM_, S = S_;
  static constexpr int kThreads = NW * 64;
  static constexpr int kWN = NW / WM;
  static constexpr int kParts = MODE == kG1U1 ? 2 : 1;
  static constexpr int kOutN = BNB / kParts;          // output columns per workgroup
  static constexpr int kWTM = BM / WM;                // rows per wave
  static constexpr int kWTNB = BNB / kWN;             // B rows per wave (inside one part)
  static constexpr int kTM = kWTM / 16;
  static constexpr int kTN = kWTNB / 16;
  static constexpr int kAQ0 = BM / 8;                 // 1 KB DMA rows-of-8 for A
  static constexpr int kBQ = BNB / 8;
  static constexpr int kAQ = (kAQ0 + kBQ + NW - 1) / NW * NW - kBQ;  // padded: every wave issues the same count
  static constexpr int kQW = (kAQ + kBQ) / NW;        // 16-byte DMAs per lane per stage
  static constexpr int kLoadsPerStage = kQW + 1;      // + the wave's A-scale DMA
  static constexpr int kAOff = 0;
  static constexpr int kBOff = kAQ * 1024;
  static constexpr int kSOff = kBOff + kBQ * 1024;
  static constexpr int kStage = kSOff + NW * 256;     // 64 fp32 A scales per wave
  static constexpr int kLds = S * kStage;
  // g1u1 epilogue: threads per output row (each takes 128 / kQPR columns)
  static constexpr int kQPR = kThreads / BM >= 8 ? 8 : kThreads / BM;
  static_assert(MODE != kG1U1 || (kQPR >= 1 && 128 % kQPR == 0 && 128 / kQPR % 16 == 0), "g1u1 epilogue split");
  static constexpr int kRed = kQPR > kWN ? kQPR : kWN;
  static_assert(kWTM % 16 == 0 && kWTNB % 16 == 0, "wave tile must be whole MFMA tiles");
  static_assert(kWTNB <= 128 && 128 % kWTNB == 0, "a wave's columns lie in one 128-column scale block");
  static_assert(kWTM <= 64, "one A-scale DMA per wave covers 64 rows");
  static_assert(MODE != kG1U1 || BNB == 256, "g1u1 stages 128 gate and 128 up rows");
  static_assert(kWN % kParts == 0, "gate and up waves split evenly");
  static_assert(S >= 2 && S <= 4 && 2 * kLoadsPerStage < 64, "pipeline depth");
};


__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// LDS-DMA: every lane moves 16 (or 4) bytes from base + its 32-bit offset to
// LDS[m0 + 16*lane] (or 4*lane); base is wave-uniform (SGPRs), so advancing a
// stream costs scalar adds only.  Issued from asm so that the compiler does
// not drain the DMA queue before each LDS read; completion is tracked
// explicitly with vm_wait.  No output registers.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(m0)
               : "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "s"(m0)
               : "memory");
}

__device__ __forceinline__ const uint8_t* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// wait until at most a*PER of this wave's DMAs are in flight, a in [0, 2]
template <int PER>
__device__ __forceinline__ void vm_wait_stages(int a) {
  if (a >= 2) {
    vm_wait<2 * PER>();
  } else if (a == 1) {
    vm_wait<PER>();
  } else {
    vm_wait<0>();
  }
}

__device__ __forceinline__ void lgkm_wait0() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0), vmcnt and expcnt untouched
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int swz(int r, int ch) { return r * 128 + ((ch ^ (r & 7)) << 4); }

// MFMA operand for the 16 rows starting at r0: lane l holds row r0 + l%16 with
// K chunks l/16 (low half) and 4 + l/16 (high half; its slot differs in bit 2).
__device__ __forceinline__ v8i lds_frag(const uint8_t* tile, int r0, int lane) {
  const int off = swz(r0 + (lane & 15), lane >> 4);
  const u32x4 lo = *reinterpret_cast<const u32x4*>(tile + off);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(tile + (off ^ 64));
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// PK (dense only): K is not a multiple of 128, so the last K block holds
// K % 128 bytes of each row.  The DMA pipeline walks the full blocks; the
// workgroup that owns the last block then loads it through registers into
// stage 0 with its chunks past K written as zeros (they add nothing to the
// block sum) and runs one more K step on it.
//
// BSH: B is stored pre-shuffled (shuffle_weight_128x128): 128-row x 128-byte tiles,
// the K blocks of a row tile one after another, each row's 16-byte chunks already in
// their LDS slots, so every B DMA moves one contiguous 1 KB block.
template <class C, int MODE, bool PK = false, bool BSH = false>
__global__ __launch_bounds__(C::kThreads) void bs_gemm_kernel(GemmArgs g) {
  static_assert(!PK || MODE == kDense, "partial K blocks: dense mode only");
  static_assert(!(PK && BSH), "pre-shuffled B has whole 128x128 tiles");
  constexpr int64_t kBStep = BSH ? 128 * 128 : 128;  // bytes between K blocks of a B row
  // pre-shuffled B blocks are 1 KB copies from the first row of 8; their offset goes
  // in the wave-uniform address for the 128-row tiles (short of VGPRs) and in the
  // per-lane offset for the smaller ones (short of SGPRs)
  constexpr bool kBUni = BSH && C::BM == 128;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::kLds];
  __shared__ int rowinfo[C::BM];
  __shared__ float red[C::kRed][C::BM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in SGPRs
  const int wm = w / C::kWN, wn = w % C::kWN;
  // dense N may end inside a tile: the last tile's B rows past N repeat row N-1
  // and its columns past N are not stored
  const int NT = MODE == kDense ? (g.N + C::kOutN - 1) / C::kOutN : g.N / C::kOutN;
  const int KBtot = (g.K + 127) / 128;  // K blocks of the whole problem (row stride of the B scales)
  const int npairs = g.T * g.topk;

  // Tiles are (M block, N tile) pairs, N tile fastest, one per workgroup: the N
  // tiles of an M block share its A rows and run side by side; consecutive M
  // blocks of one expert share weights.  Workgroup b runs on XCD b % 8 (one L2
  // each), in order of b; orders that put all readers of a tile on one XCD
  // (contiguous ranges, persistent rounds, paired M blocks) measured slower.
  // Dense split-K: tile index = split * (M blocks * N tiles) + M block * N tiles + N tile.
  int64_t total;
  int nvalid = 0;
  if constexpr (MODE == kDense) {
    total = (int64_t)((g.M + C::BM - 1) / C::BM) * NT;
  } else {
    nvalid = g.num_valid[0];
    total = nvalid > 0 ? (int64_t)(nvalid / C::BM) * NT : 0;
  }
  int64_t tile = blockIdx.x;
  int ks = 0;
  if constexpr (MODE == kDense) {
    ks = (int)(tile / total);
    tile -= (int64_t)ks * total;
    if (ks >= g.splits) return;
  }
  if (tile >= total) return;  // uniform: blocks past num_valid hold no rows
  const int kbase = ks * g.kbs;                        // first K block of this split
  const int KB = min(g.kbs, KBtot - kbase);            // K blocks this workgroup walks
  // blocks the DMA pipeline walks: with PK the last, partial block of K (if this
  // workgroup owns it) is staged separately after the pipeline
  const int KBp = PK && kbase + KB == KBtot ? KB - 1 : KB;
  const int nt = (int)(tile % NT);
  const int mb = (int)(tile / NT);
  const int64_t row0 = (int64_t)mb * C::BM;

  // valid rows of this block form a prefix (padding sits at the end of an expert's segment)
  int expert = 0, nrows;
  if constexpr (MODE != kDense) expert = g.sorted_eids[mb];

  // per-wave B scale column block
  const int part = wn / (C::kWN / C::kParts);
  const int colofs = (wn % (C::kWN / C::kParts)) * C::kWTNB;  // first output column of this wave in its part
  const float* sbp;
  if constexpr (MODE == kDense) {
    const int nb = min((nt * C::BNB + wn * C::kWTNB) / 128, (g.N + 127) / 128 - 1);  // waves past N: any valid row
    sbp = g.b_scale + (int64_t)nb * KBtot + kbase;
  } else if constexpr (MODE == kG1U1) {
    const int64_t nb2 = 2 * (g.N / 128);
    sbp = g.b_scale + ((int64_t)expert * nb2 + (part == 0 ? nt : g.N / 128 + nt)) * KBtot;
  } else {
    sbp = g.b_scale + ((int64_t)expert * (g.N / 128) + (nt * C::BNB + wn * C::kWTNB) / 128) * KBtot;
  }

  // this wave's B scales for every K block, fetched before the DMA pipeline starts:
  // lane L holds blocks L and L + 64 (a workgroup walks at most 128); read per step with readlane
  const float sbv0 = lane < KB ? sbp[lane] : 0.0f;
  const float sbv1 = lane + 64 < KB ? sbp[lane + 64] : 0.0f;

  if constexpr (MODE != kDense) {
    for (int i = tid; i < C::BM; i += C::kThreads) rowinfo[i] = g.sorted_ids[row0 + i];
    __syncthreads();
    nrows = __syncthreads_count(tid < C::BM && rowinfo[tid < C::BM ? tid : 0] < npairs);
  } else {
    nrows = (int)min((int64_t)C::BM, g.M - row0);
  }
  // MFMA row tiles of this wave holding at least one valid row
  const int tm_live = __builtin_amdgcn_readfirstlane(min(C::kTM, max(0, (nrows - wm * C::kWTM + 15) / 16)));

  // A-tile row r -> row of the A operand (relative to g.a)
  auto a_row = [&](int r) -> int64_t {
    if constexpr (MODE == kDense) {
      return row0 + r < g.M ? row0 + r : g.M - 1;
    } else if constexpr (MODE == kG1U1) {
      const int pid = rowinfo[r];
      return pid < npairs ? pid / g.topk : 0;
    } else {
      return row0 + r;
    }
  };
  // B-tile row r -> row inside the B base of this workgroup
  auto b_row = [&](int r) -> int {
    if constexpr (MODE == kG1U1) {
      return r < 128 ? nt * 128 + r : g.N + nt * 128 + (r - 128);
    } else if constexpr (MODE == kDense) {
      return min(nt * C::BNB + r, g.N - 1);
    } else {
      return nt * C::BNB + r;
    }
  };
  const uint8_t* a_base = uniform_ptr(g.a);
  const uint8_t* b_base;
  if constexpr (MODE == kDense) {
    b_base = uniform_ptr(g.b);
  } else if constexpr (MODE == kG1U1) {
    b_base = uniform_ptr(g.b + (int64_t)expert * 2 * g.N * g.K);
  } else {
    b_base = uniform_ptr(g.b + (int64_t)expert * g.N * g.K);
  }

  // ---- per-lane DMA offsets (fixed) and wave-uniform LDS offsets.
  // 1 KB block q of a region holds rows 8q .. 8q+7; lane L of its DMA moves the
  // chunk of row 8q + L/8 that belongs in slot L%8
  // (A blocks come first and B blocks follow, so block q sits at q * 1 KB of a stage)
  // (kAQ is a multiple of NW, so DMA j of every wave moves A rows iff j < kJA)
  static_assert(C::kAOff == 0 && C::kBOff == C::kAQ * 1024, "stage layout");
  static_assert(C::kAQ % C::NW == 0, "A/B split of the DMAs is the same in every wave");
  constexpr int kJA = C::kAQ / C::NW;
  uint32_t voff[C::kQW];
#pragma unroll
  for (int j = 0; j < C::kQW; ++j) {
    const int q = w + j * C::NW;
    const bool is_a = BSH ? j < kJA : q < C::kAQ;
    const int qq = is_a ? q : q - C::kAQ;
    const int r = qq * 8 + (lane >> 3);
    const int ch = (lane & 7) ^ (r & 7);
    if (is_a) {
      voff[j] = (uint32_t)(a_row(r < C::BM ? r : 0) * g.K + ch * 16);
    } else if constexpr (kBUni) {
      voff[j] = 0;  // unused: addressed from the wave-uniform base
    } else if constexpr (BSH) {
      const int br0 = b_row(qq * 8);
      voff[j] = (uint32_t)((int64_t)(br0 >> 7) * KBtot * (128 * 128) + (br0 & 127) * 128) + lane * 16;
    } else {
      voff[j] = (uint32_t)((int64_t)b_row(r) * g.K + ch * 16);
    }
  }
  const uint32_t lane16 = (uint32_t)lane * 16;
  const int my_row = wm * C::kWTM + (lane < C::kWTM ? lane : 0);
  const uint32_t soff = (uint32_t)(a_row(my_row) * g.ssm * 4);
  const uint8_t* s_base = uniform_ptr(g.a_scale);
  const int sofs = C::kSOff + w * 256;

  vm_wait<0>();  // every ordinary load lands before the first DMA is queued

  const uint32_t lds0 = lds_addr(lds);
  // DMA j of this wave for K block kb into LDS stage `stage`: j < kQW moves A/B
  // rows, j == kQW the wave's A scales
  // (every operand but voff / soff is wave-uniform: addresses and m0 stay in SGPRs)
  auto issue_one = [&](int stage, int kb, int j) {
    const uint32_t base = lds0 + stage * C::kStage;
    const int64_t kg = kbase + kb;  // K block in the whole problem
    if (j < C::kQW) {
      const int q = w + j * C::NW;
      if constexpr (kBUni) {
        if (j < kJA) {
          dma16(a_base + kg * 128, voff[j], base + q * 1024);
        } else {
          // 8 consecutive rows of one 128-row tile with every stored chunk already in its
          // LDS slot: one contiguous 1 KB copy from the block's first row
          const int br0 = b_row((q - C::kAQ) * 8);
          const int64_t bofs = (int64_t)(br0 >> 7) * KBtot * (128 * 128) + (br0 & 127) * 128;
          dma16(b_base + kg * kBStep + bofs, lane16, base + q * 1024);
        }
      } else if constexpr (BSH) {
        dma16(j < kJA ? a_base + kg * 128 : b_base + kg * kBStep, voff[j], base + q * 1024);
      } else {
        dma16((q < C::kAQ ? a_base : b_base) + kg * 128, voff[j], base + q * 1024);
      }
    } else {
      dma4(s_base + kg * g.sskb * 4, soff, base + sofs);
    }
  };
  auto issue = [&](int stage, int kb) {
#pragma unroll
    for (int j = 0; j <= C::kQW; ++j) issue_one(stage, kb, j);
  };

  v4f acc[C::kTM][C::kTN];
#pragma unroll
  for (int tm = 0; tm < C::kTM; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::kTN; ++tn) acc[tm][tn] = v4f{0.f, 0.f, 0.f, 0.f};

  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int s = 0; s < C::S - 1; ++s)
    if (s < KBp) issue(s, s);

  // one K step on LDS stage `stage`; only the first TMV row tiles of the wave are computed
  // RF 1: the step refills its stage (steady state, no branches); RF 0: checked
  auto step = [&](const int kb, const int stage, auto tmv_c, auto rf_c) {
    constexpr int TMV = decltype(tmv_c)::value;
    constexpr int RF = decltype(rf_c)::value;
    if constexpr (RF == 1) {
      vm_wait<(C::S - 2) * C::kLoadsPerStage>();
    } else {
      vm_wait_stages<C::kLoadsPerStage>(min(C::S - 2, KBp - 1 - kb));
    }
    barrier_only();
    const bool refill = RF == 1 || kb + C::S - 1 < KBp;
    const int nstage = (stage + C::S - 1) % C::S, nkb = kb + C::S - 1;
    if constexpr (TMV == 0) {
      if (refill) issue(nstage, nkb);
    } else {
      const uint8_t* st = lds + stage * C::kStage;
      const float sb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(kb < 64 ? sbv0 : sbv1), kb & 63));
      v8i av[TMV];
      v4f s4[TMV];
#pragma unroll
      for (int tm = 0; tm < TMV; ++tm) {
        av[tm] = lds_frag(st + C::kAOff, wm * C::kWTM + tm * 16, lane);
        s4[tm] = *reinterpret_cast<const v4f*>(st + sofs + (tm * 16 + 4 * lg) * 4) * sb;
      }
      v8i bv[C::kTN];
#pragma unroll
      for (int tn = 0; tn < C::kTN; ++tn) bv[tn] = lds_frag(st + C::kBOff, wn * C::kWTNB + tn * 16, lane);
      // rolling window: tile q is issued, tile q-2 is folded.  The refill DMAs of
      // the stage freed by the barrier are spread between the MFMAs (DMA j after
      // MFMA j * kGap), so a wave never stalls on a burst of DMA issues.
      constexpr int NQ = TMV * C::kTN;
      constexpr int kGap = NQ / (C::kQW + 1) > 0 ? NQ / (C::kQW + 1) : 1;
      v4f tq[3];
#pragma unroll
      for (int q = 0; q < NQ + 2; ++q) {
        if (q < NQ) tq[q % 3] = mfma16x16x128_fp8(av[q % TMV], bv[q / TMV], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int j = 0; j <= C::kQW; ++j)
          if (refill && (j * kGap < NQ + 1 ? j * kGap : NQ + 1) == q) issue_one(nstage, nkb, j);
        if (q >= 2) {
          const int p = q - 2;
          acc[p % TMV][p / TMV] += tq[p % 3] * s4[p % TMV];
        }
      }
    }
  };
  // unrolled by the stage count: every LDS address is base + immediate
  auto kloop = [&](auto tmv_c) {
    int kb0 = 0;
    // rounds whose every step refills (kb + S - 1 < KBp for the round's last step)
    for (; kb0 + 2 * C::S - 1 <= KBp; kb0 += C::S) {
#pragma unroll
      for (int u = 0; u < C::S; ++u) step(kb0 + u, u, tmv_c, std::integral_constant<int, 1>{});
    }
    for (; kb0 < KBp; kb0 += C::S) {
#pragma unroll
      for (int u = 0; u < C::S; ++u)
        if (kb0 + u < KBp) step(kb0 + u, u, tmv_c, std::integral_constant<int, 0>{});
    }
    if constexpr (PK) {
      if (KBp < KB) {
        // the last, partial K block goes through registers into stage 0, chunks
        // past K as zeros (they then add nothing to the block sum)
        __syncthreads();  // every wave is done with the pipeline's stages
        const int64_t kg = KBtot - 1;
        const int kt = g.K - (int)kg * 128;  // bytes of each row inside K
        // this lane's chunk inside its row (rows of a 1 KB DMA block start at multiples of 8)
        const int chb = ((lane & 7) ^ ((lane >> 3) & 7)) * 16;
#pragma unroll
        for (int j = 0; j < C::kQW; ++j) {
          const int q = w + j * C::NW;
          u32x4 v{0u, 0u, 0u, 0u};
          if (chb < kt) v = *reinterpret_cast<const u32x4*>((q < C::kAQ ? a_base : b_base) + kg * 128 + voff[j]);
          *reinterpret_cast<u32x4*>(lds + q * 1024 + lane * 16) = v;
        }
        *reinterpret_cast<float*>(lds + sofs + lane * 4) =
            *reinterpret_cast<const float*>(s_base + kg * g.sskb * 4 + soff);
        lgkm_wait0();
        step(KBp, 0, tmv_c, std::integral_constant<int, 0>{});
      }
    }
  };
  static_assert(C::kTM <= 4, "row tiles per wave");
  static_assert(C::BM * (C::BNB + 4) * 4 <= C::kLds, "padded fp32 output tile fits the pipeline LDS");
  switch (tm_live) {
    case 0: kloop(std::integral_constant<int, 0>{}); break;
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    case 2: if constexpr (C::kTM >= 2) kloop(std::integral_constant<int, 2>{}); break;
    case 3: if constexpr (C::kTM >= 3) kloop(std::integral_constant<int, 3>{}); break;
    default: if constexpr (C::kTM >= 4) kloop(std::integral_constant<int, 4>{}); break;
  }
  vm_wait<0>();
  __syncthreads();

  // ---- epilogues (LDS is free again)
  if (MODE == kDense && g.splits > 1) {
    // split-K partial: fp32 tile [BM][BNB] in LDS (rows padded by 16 bytes so that
    // rows 4 apart do not share banks), then 16-byte stores into part[ks]
    constexpr int RS = C::BNB + 4;
    float* ob = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int tm = 0; tm < C::kTM; ++tm)
#pragma unroll
      for (int tn = 0; tn < C::kTN; ++tn)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ob[(wm * C::kWTM + tm * 16 + 4 * lg + i) * RS + wn * C::kWTNB + tn * 16 + lr] = acc[tm][tn][i];
    __syncthreads();
    constexpr int CPR = C::BNB * 4 / 16;
    float* dst = g.part + (int64_t)ks * g.M * g.N;
    for (int ci = tid; ci < C::BM * CPR; ci += C::kThreads) {
      const int r = ci / CPR, ch = ci % CPR;
      const int64_t m = row0 + r;
      if (m < g.M && nt * C::BNB + ch * 4 < g.N)  // N % 8 == 0: a chunk is all in or all out
        *reinterpret_cast<u32x4*>(dst + m * g.N + (int64_t)nt * C::BNB + ch * 4) =
            *reinterpret_cast<const u32x4*>(ob + r * RS + ch * 4);
    }
  } else if constexpr (MODE == kDense) {
    // bf16 tile [BM][BNB] in LDS (rows padded by 16 bytes), then 16-byte row stores
    constexpr int RS = C::BNB + 8;
    uint16_t* ob = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
    for (int tm = 0; tm < C::kTM; ++tm)
#pragma unroll
      for (int tn = 0; tn < C::kTN; ++tn)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ob[(wm * C::kWTM + tm * 16 + 4 * lg + i) * RS + wn * C::kWTNB + tn * 16 + lr] =
              (uint16_t)f32_to_out16(acc[tm][tn][i], g.out_f16 != 0);
    __syncthreads();
    constexpr int CPR = C::BNB * 2 / 16;  // 16-byte chunks per row
    for (int ci = tid; ci < C::BM * CPR; ci += C::kThreads) {
      const int r = ci / CPR, ch = ci % CPR;
      const int64_t m = row0 + r;
      if (m < g.M && nt * C::BNB + ch * 8 < g.N)
        *reinterpret_cast<u32x4*>(g.c + m * g.ldc + (int64_t)nt * C::BNB + ch * 8) =
            *reinterpret_cast<const u32x4*>(ob + r * RS + ch * 8);
    }
  } else if constexpr (MODE == kDown) {
    // routing-weighted fp32 rows straight from the MFMA layout: for each of its rows
    // a group of 16 lanes writes 64 contiguous bytes per row tile (the neighbouring
    // column tiles complete the 128-byte lines in L2)
#pragma unroll
    for (int tm = 0; tm < C::kTM; ++tm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = wm * C::kWTM + tm * 16 + 4 * lg + i;
        const int pid = rowinfo[rl];
        if (row0 + rl < nvalid && pid < npairs) {
          const float wgt = g.sorted_w[row0 + rl];
          float* yr = g.y + (int64_t)pid * g.N + (int64_t)nt * C::BNB + wn * C::kWTNB + lr;
#pragma unroll
          for (int tn = 0; tn < C::kTN; ++tn) yr[tn * 16] = acc[tm][tn][i] * wgt;
        }
      }
  } else {
    // Both parts stage their fp32 tiles in LDS as rows [gate 128 | up 128] (row
    // stride kFS words: conflict-free stores).  Then each thread takes kCPI
    // consecutive columns of one row: h = SiLU(gate) * up, the row's amax over its
    // 128 columns (partial maxima through red), 1x128 requantisation, and 16-byte
    // stores of the codes straight to h8.
    constexpr int kFS = 2 * 128 + 4;
    constexpr int kQPR = C::kQPR, kCPI = 128 / kQPR;
    static_assert(C::BM * kFS * 4 <= C::kLds, "gate/up tile fits the pipeline LDS");
    float* F = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int tm = 0; tm < C::kTM; ++tm)
#pragma unroll
      for (int tn = 0; tn < C::kTN; ++tn)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          F[(wm * C::kWTM + tm * 16 + 4 * lg + i) * kFS + part * 128 + colofs + tn * 16 + lr] = acc[tm][tn][i];
    __syncthreads();
    const int r = tid % C::BM, qc = tid / C::BM;  // row and column group of this thread
    const bool active = qc < kQPR;
    float h[kCPI];
    if (active) {
      float mx = 0.0f;
      // fc2 smoothing factors of this expert's columns (uniform branch: pointer or none)
      const float* sm = g.smooth ? g.smooth + (int64_t)expert * g.N + nt * 128 + qc * kCPI : nullptr;
#pragma unroll
      for (int v = 0; v < kCPI; v += 4) {
        const v4f gt = *reinterpret_cast<const v4f*>(F + r * kFS + qc * kCPI + v);
        const v4f up = *reinterpret_cast<const v4f*>(F + r * kFS + 128 + qc * kCPI + v);
        const v4f f = sm ? *reinterpret_cast<const v4f*>(sm + v) : v4f{1.f, 1.f, 1.f, 1.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          h[v + i] = gt[i] * __builtin_amdgcn_rcpf(1.0f + __expf(-gt[i])) * up[i];
          if (sm) h[v + i] = h[v + i] * f[i];
          mx = fmaxf(mx, fabsf(h[v + i]));
        }
      }
      red[qc][r] = mx;
    }
    __syncthreads();
    if (active && rowinfo[r] < npairs) {
      float amax = red[0][r];
#pragma unroll
      for (int k2 = 1; k2 < kQPR; ++k2) amax = fmaxf(amax, red[k2][r]);
      const float sc = (amax == 0.0f) ? 1.0f : amax / kE4M3Max;
      uint32_t wds[kCPI / 4];
#pragma unroll
      for (int v = 0; v < kCPI / 4; ++v)
        wds[v] = f32_to_e4m3(h[4 * v] / sc) | (f32_to_e4m3(h[4 * v + 1] / sc) << 8) |
                 (f32_to_e4m3(h[4 * v + 2] / sc) << 16) | (f32_to_e4m3(h[4 * v + 3] / sc) << 24);
      uint8_t* dst = g.h8 + (row0 + r) * g.N + nt * 128 + qc * kCPI;
#pragma unroll
      for (int v = 0; v < kCPI / 16; ++v)
        *reinterpret_cast<u32x4*>(dst + 16 * v) = u32x4{wds[4 * v], wds[4 * v + 1], wds[4 * v + 2], wds[4 * v + 3]};
      if (qc == 0) g.h_scale[(row0 + r) * (g.N / 128) + nt] = sc;
    }
  }
}

// out[t, n] = bf16(sum_j y[t*k + j, n]), j ascending, fp32.  Writes nothing when
// the sort flagged an invalid expert id (num_valid < 0: the pairs were not placed).
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, int T, int k, int H,
                                                      uint16_t* __restrict__ out, int64_t ld_out,
                                                      const int32_t* __restrict__ num_valid) {
  if (num_valid[0] < 0) return;
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

// c[m, n] = bf16 (or fp16) of the fp32 sum of part[split, m, n] over the splits, in a fixed
// order: wave w sums splits w, w+4, w+8, ... in ascending order, then the four
// wave sums are added in wave order.  One workgroup covers 256 columns of one
// row (workgroup b: row b / ceil(N/256), column block b % ceil(N/256)); every lane
// keeps up to 8 loads in flight.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits, int M, int N,
                                                            uint16_t* __restrict__ c, int64_t ldc, int out_f16) {
  __shared__ float sh[4][256];
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int nbn = (N + 255) / 256;
  const int m = (int)(blockIdx.x / nbn);
  const int col = (int)(blockIdx.x % nbn) * 256 + lane * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (col < N) {
    const float* p = part + (int64_t)m * N + col;
    const int64_t sstride = (int64_t)M * N;
    for (int k0 = w; k0 < splits; k0 += 32) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (k0 + 4 * u < splits) v[u] = *reinterpret_cast<const float4*>(p + (k0 + 4 * u) * sstride);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (k0 + 4 * u < splits) {
          acc.x += v[u].x;
          acc.y += v[u].y;
          acc.z += v[u].z;
          acc.w += v[u].w;
        }
    }
  }
  *reinterpret_cast<float4*>(&sh[w][lane * 4]) = acc;
  __syncthreads();
  if (w == 0 && col < N) {
    float o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = ((sh[0][lane * 4 + i] + sh[1][lane * 4 + i]) + sh[2][lane * 4 + i]) + sh[3][lane * 4 + i];
    const bool f16 = out_f16 != 0;
    const uint2 r{f32_to_out16(o[0], f16) | (f32_to_out16(o[1], f16) << 16),
                  f32_to_out16(o[2], f16) | (f32_to_out16(o[3], f16) << 16)};
    *reinterpret_cast<uint2*>(c + (int64_t)m * ldc + col) = r;
  }
}

template <class C, int MODE, bool PK, bool BSH>
int launch_cfg(const GemmArgs& g, int64_t mblocks, hipStream_t stream) {
  if (MODE != kDense && g.N % C::kOutN != 0) return MOE355_EUNSUPPORTED;
  const int64_t grid = mblocks * ceil_div64(g.N, C::kOutN) * (MODE == kDense ? g.splits : 1);
  if (grid == 0) return MOE355_OK;
  MOE355_CHECK(grid < (1ll << 31), MOE355_EUNSUPPORTED);
  hipLaunchKernelGGL((bs_gemm_kernel<C, MODE, PK, BSH>), dim3((unsigned)grid), dim3(C::kThreads), 0, stream, g);
  return launch_status();
}

// Tile choice per M tile: small tiles stream weights (decode, small M), 128-row
// tiles with 8 waves feed the matrix cores (prefill, large M).
template <int MODE, int BNB = 256, bool PK = false, bool BSH = false>
int launch_gemm(const GemmArgs& g, int bm, int64_t mblocks, hipStream_t stream) {
  switch (bm) {
    case 16: return launch_cfg<Cfg<MODE, 16, BNB, 4, 1, 4>, MODE, PK, BSH>(g, mblocks, stream);
    case 32: return launch_cfg<Cfg<MODE, 32, BNB, 4, 1, 4>, MODE, PK, BSH>(g, mblocks, stream);
    case 64: return launch_cfg<Cfg<MODE, 64, BNB, 4, 1, 3>, MODE, PK, BSH>(g, mblocks, stream);
    case 128: return launch_cfg<Cfg<MODE, 128, BNB, 8, 2, 3>, MODE, PK, BSH>(g, mblocks, stream);
    default: return MOE355_EUNSUPPORTED;
  }
}

// Dense tiling: M tile, B rows per workgroup and K splits.  When M <= 64 leaves
// fewer output tiles than compute units, K is split so that the grid comes close
// to one workgroup per compute unit (kSplitTargetWG) without going over: short K
// loops per workgroup lose more to pipeline fill and epilogue than a second
// round of workgroups gains.  The fp32 partials (written once, read once) are
// capped at 1/kSplitBytesDiv of the weight bytes: splits * M * N * 4 <= N * K /
// kSplitBytesDiv.  Each split walks at least two K blocks.  A workgroup holds the
// weight scales of at most kMaxKbs K blocks (two per lane), so K beyond 128 blocks
// is always split, whatever M.
constexpr int64_t kSplitTargetWG = 256;
constexpr int kMaxKbs = 128;
constexpr int64_t kSplitBytesDiv = 4;
constexpr int kNarrowMaxN = 4096;  // M <= 64: 128-column tiles up to this N, 256 above

struct DensePlan {
  int bm, bnb, splits, kbs;
};

DensePlan dense_plan(int M, int N, int K) {
  DensePlan p;
  p.bm = M <= 16 ? 16 : M <= 32 ? 32 : M <= 64 ? 64 : 128;
  p.bnb = (N % 256 != 0 || (M <= 64 && N <= kNarrowMaxN)) ? 128 : 256;
  const int KB = (int)ceil_div64(K, 128);
  const int64_t base = ceil_div64(M, p.bm) * ceil_div64(N, p.bnb);
  int splits = 1;
  if (M <= 64 && 2 * base <= kSplitTargetWG && KB >= 4) {
    const int64_t by_bytes = std::max<int64_t>(1, K / (kSplitBytesDiv * 4 * M));
    splits = (int)std::min<int64_t>({(int64_t)KB / 2, kSplitTargetWG / base, by_bytes});
  }
  splits = std::max(splits, (int)ceil_div64(KB, kMaxKbs));
  p.kbs = (int)ceil_div64(KB, splits);
  p.splits = (int)ceil_div64(KB, p.kbs);
  return p;
}

size_t dense_workspace_bytes(const DensePlan& p, int M, int N) {
  return p.splits > 1 ? (size_t)p.splits * M * N * sizeof(float) + 256 : 0;
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

extern "C" int gemm_fp8_blockscale_workspace(int M, int N, int K, size_t* bytes) {
  MOE355_CHECK(M >= 0 && N >= 0 && K >= 0 && bytes, MOE355_EINVAL);
  MOE355_CHECK(K % 16 == 0 && N % 8 == 0, MOE355_EUNSUPPORTED);
  *bytes = (M == 0 || N == 0 || K == 0) ? 0 : dense_workspace_bytes(dense_plan(M, N, K), M, N);
  return MOE355_OK;
}

extern "C" int moe_down_combine_workspace(int T, int H, int topk, size_t* bytes) {
  MOE355_CHECK(T >= 0 && H > 0 && topk > 0 && bytes, MOE355_EINVAL);
  *bytes = (size_t)T * topk * H * sizeof(float) + 256;
  return MOE355_OK;
}

namespace {

int dense_gemm(const uint8_t* a8, const float* a_scale, int64_t sstride_m, int64_t sstride_kb, const uint8_t* b8,
               const float* b_scale, int M, int N, int K, uint16_t* c, int64_t ldc, int out_fp16, void* workspace,
               size_t workspace_bytes, hipStream_t stream, bool bsh) {
  MOE355_CHECK(M >= 0 && N >= 0 && K >= 0 && ldc >= N && (out_fp16 == 0 || out_fp16 == 1), MOE355_EINVAL);
  MOE355_CHECK(K % 16 == 0 && N % 8 == 0, MOE355_EUNSUPPORTED);
  MOE355_CHECK(!bsh || (K % 128 == 0 && N % 128 == 0), MOE355_EUNSUPPORTED);
  MOE355_CHECK((int64_t)M * K < (1ll << 32) && (int64_t)N * K < (1ll << 32), MOE355_EUNSUPPORTED);
  if (M == 0 || N == 0) return MOE355_OK;
  MOE355_CHECK(K > 0 && a8 && a_scale && b8 && b_scale && c && sstride_m >= 0 && sstride_kb >= 0, MOE355_EINVAL);
  MOE355_CHECK(aligned16(a8) && aligned16(b8) && aligned16(c) && ldc % 8 == 0, MOE355_EMISALIGNED);
  MOE355_CHECK((reinterpret_cast<uintptr_t>(a_scale) & 3u) == 0, MOE355_EMISALIGNED);
  DensePlan plan = dense_plan(M, N, K);
  const size_t need = dense_workspace_bytes(plan, M, N);
  if (need == 0 || workspace == nullptr || workspace_bytes < need) {
    // without (enough) workspace: one workgroup per output tile walks all of K, which
    // holds the weight scales of at most kMaxKbs K blocks
    MOE355_CHECK(ceil_div64(K, 128) <= kMaxKbs, need > 0 && workspace != nullptr ? MOE355_EINVAL : MOE355_EUNSUPPORTED);
    plan.splits = 1;
    plan.kbs = (int)ceil_div64(K, 128);
  } else {
    MOE355_CHECK(aligned16(workspace), MOE355_EMISALIGNED);
  }
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
  g.splits = plan.splits;
  g.kbs = plan.kbs;
  g.out_f16 = out_fp16;
  g.part = static_cast<float*>(workspace);
  const int64_t mblocks = ceil_div64(M, plan.bm);
  int st;
  if (bsh) {
    st = plan.bnb == 128 ? launch_gemm<kDense, 128, false, true>(g, plan.bm, mblocks, stream)
                         : launch_gemm<kDense, 256, false, true>(g, plan.bm, mblocks, stream);
  } else if (K % 128 == 0) {
    st = plan.bnb == 128 ? launch_gemm<kDense, 128>(g, plan.bm, mblocks, stream)
                         : launch_gemm<kDense, 256>(g, plan.bm, mblocks, stream);
  } else {
    st = plan.bnb == 128 ? launch_gemm<kDense, 128, true>(g, plan.bm, mblocks, stream)
                         : launch_gemm<kDense, 256, true>(g, plan.bm, mblocks, stream);
  }
  if (st != MOE355_OK || plan.splits == 1) return st;
  const int64_t rblocks = ceil_div64(N, 256) * M;
  MOE355_CHECK(rblocks < (1ll << 31), MOE355_EUNSUPPORTED);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)rblocks), dim3(256), 0, stream, g.part, plan.splits, M, N, c,
                     ldc, out_fp16);
  return launch_status();
}

int g1u1_gemm(const uint8_t* a8, const float* a_scale, int64_t sstride_m, int64_t sstride_kb, const uint8_t* w1,
              const float* w1_scale, const int32_t* sorted_ids, const int32_t* sorted_expert_ids,
              const int32_t* num_valid, int T, int H, int I, int E, int topk, int block_m, int64_t max_sorted,
              uint8_t* h8, float* h_scale, const float* fc2_smooth_scale, hipStream_t stream, bool bsh) {
  MOE355_CHECK(T >= 0 && H > 0 && I > 0 && E > 0 && topk > 0, MOE355_EINVAL);
  MOE355_CHECK(H % 128 == 0 && I % 128 == 0 && H <= 16384 && valid_block_m(block_m), MOE355_EUNSUPPORTED);
  MOE355_CHECK((int64_t)T * H < (1ll << 32) && (int64_t)2 * I * H < (1ll << 32), MOE355_EUNSUPPORTED);
  const int cap = check_sorted_capacity(T, topk, E, block_m, max_sorted);
  if (cap != MOE355_OK) return cap;
  if (T == 0) return MOE355_OK;
  MOE355_CHECK(a8 && a_scale && w1 && w1_scale && sorted_ids && sorted_expert_ids && num_valid && h8 && h_scale,
               MOE355_EINVAL);
  MOE355_CHECK(sstride_m >= 0 && sstride_kb >= 0, MOE355_EINVAL);
  MOE355_CHECK(aligned16(a8) && aligned16(w1) && aligned16(h8), MOE355_EMISALIGNED);
  MOE355_CHECK((reinterpret_cast<uintptr_t>(a_scale) & 3u) == 0 && aligned16(fc2_smooth_scale),
               MOE355_EMISALIGNED);
  GemmArgs g{};
  g.a = a8;
  g.a_scale = a_scale;
  g.ssm = sstride_m;
  g.sskb = sstride_kb;
  g.smooth = fc2_smooth_scale;
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
  g.splits = 1;
  g.kbs = H / 128;
  return bsh ? launch_gemm<kG1U1, 256, false, true>(g, block_m, max_sorted / block_m, stream)
             : launch_gemm<kG1U1>(g, block_m, max_sorted / block_m, stream);
}

int down_gemm(const uint8_t* h8, const float* h_scale, const uint8_t* w2, const float* w2_scale,
              const int32_t* sorted_ids, const float* sorted_weights, const int32_t* sorted_expert_ids,
              const int32_t* num_valid, int T, int H, int I, int E, int topk, int block_m, int64_t max_sorted,
              uint16_t* out, int64_t ld_out, void* workspace, size_t workspace_bytes, hipStream_t stream, bool bsh) {
  MOE355_CHECK(T >= 0 && H > 0 && I > 0 && E > 0 && topk > 0 && ld_out >= H, MOE355_EINVAL);
  MOE355_CHECK(H % 256 == 0 && I % 128 == 0 && I <= 16384 && valid_block_m(block_m), MOE355_EUNSUPPORTED);
  MOE355_CHECK(max_sorted * I < (1ll << 32) && (int64_t)H * I < (1ll << 32), MOE355_EUNSUPPORTED);
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
  g.splits = 1;
  g.kbs = I / 128;
  int st = bsh ? launch_gemm<kDown, 256, false, true>(g, block_m, max_sorted / block_m, stream)
               : launch_gemm<kDown>(g, block_m, max_sorted / block_m, stream);
  if (st != MOE355_OK) return st;
  const int64_t threads = (int64_t)T * (H / 8);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)ceil_div64(threads, 256)), dim3(256), 0, stream, g.y, T, topk, H,
                     out, ld_out, num_valid);
  return launch_status();
}

}  // namespace

extern "C" int gemm_fp8_blockscale(const uint8_t* a8, const float* a_scale, int64_t sstride_m, int64_t sstride_kb,
                                   const uint8_t* b8, const float* b_scale, int M, int N, int K, uint16_t* c,
                                   int64_t ldc, int out_fp16, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  return dense_gemm(a8, a_scale, sstride_m, sstride_kb, b8, b_scale, M, N, K, c, ldc, out_fp16, workspace,
                    workspace_bytes, stream, false);
}

extern "C" int gemm_fp8_blockscale_wpreshuffle(const uint8_t* a8, const float* a_scale, int64_t sstride_m,
                                               int64_t sstride_kb, const uint8_t* b8, const float* b_scale, int M,
                                               int N, int K, uint16_t* c, int64_t ldc, int out_fp16,
                                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return dense_gemm(a8, a_scale, sstride_m, sstride_kb, b8, b_scale, M, N, K, c, ldc, out_fp16, workspace,
                    workspace_bytes, stream, true);
}

extern "C" int moe_fp8_blockscale_g1u1(const uint8_t* a8, const float* a_scale, int64_t sstride_m, int64_t sstride_kb,
                                       const uint8_t* w1, const float* w1_scale, const int32_t* sorted_ids,
                                       const int32_t* sorted_expert_ids, const int32_t* num_valid, int T, int H,
                                       int I, int E, int topk, int block_m, int64_t max_sorted, uint8_t* h8,
                                       float* h_scale, const float* fc2_smooth_scale, hipStream_t stream) {
  return g1u1_gemm(a8, a_scale, sstride_m, sstride_kb, w1, w1_scale, sorted_ids, sorted_expert_ids, num_valid, T, H,
                   I, E, topk, block_m, max_sorted, h8, h_scale, fc2_smooth_scale, stream, false);
}

extern "C" int moe_fp8_blockscale_g1u1_wpreshuffle(const uint8_t* a8, const float* a_scale, int64_t sstride_m,
                                                   int64_t sstride_kb, const uint8_t* w1, const float* w1_scale,
                                                   const int32_t* sorted_ids, const int32_t* sorted_expert_ids,
                                                   const int32_t* num_valid, int T, int H, int I, int E, int topk,
                                                   int block_m, int64_t max_sorted, uint8_t* h8, float* h_scale,
                                                   const float* fc2_smooth_scale, hipStream_t stream) {
  return g1u1_gemm(a8, a_scale, sstride_m, sstride_kb, w1, w1_scale, sorted_ids, sorted_expert_ids, num_valid, T, H,
                   I, E, topk, block_m, max_sorted, h8, h_scale, fc2_smooth_scale, stream, true);
}

extern "C" int moe_down_combine(const uint8_t* h8, const float* h_scale, const uint8_t* w2, const float* w2_scale,
                                const int32_t* sorted_ids, const float* sorted_weights,
                                const int32_t* sorted_expert_ids, const int32_t* num_valid, int T, int H, int I,
                                int E, int topk, int block_m, int64_t max_sorted, uint16_t* out, int64_t ld_out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return down_gemm(h8, h_scale, w2, w2_scale, sorted_ids, sorted_weights, sorted_expert_ids, num_valid, T, H, I, E,
                   topk, block_m, max_sorted, out, ld_out, workspace, workspace_bytes, stream, false);
}

extern "C" int moe_down_combine_wpreshuffle(const uint8_t* h8, const float* h_scale, const uint8_t* w2,
                                            const float* w2_scale, const int32_t* sorted_ids,
                                            const float* sorted_weights, const int32_t* sorted_expert_ids,
                                            const int32_t* num_valid, int T, int H, int I, int E, int topk,
                                            int block_m, int64_t max_sorted, uint16_t* out, int64_t ld_out,
                                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return down_gemm(h8, h_scale, w2, w2_scale, sorted_ids, sorted_weights, sorted_expert_ids, num_valid, T, H, I, E,
                   topk, block_m, max_sorted, out, ld_out, workspace, workspace_bytes, stream, true);
}
