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
#include <mutex>
#include <type_traits>

#include <hip/hip_cooperative_groups.h>

#include "dense_small.h"
#include "dense_tuned.h"
#include "device_common.h"
#include "gemm_engine.h"
#include "host_common.h"

namespace moe355 {
namespace {

// Tile configuration.  BNB = B rows staged per workgroup (g1u1: 128 gate + 128 up).
template <int MODE, int BM_, int BNB_, int NW_, int WM_, int S_>
struct Cfg {
  static constexpr int BM = BM_, BNB = BNB_, NW = NW_, WM = WM_, S = S_;
  static constexpr int kMode = MODE;
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
  static constexpr int kSD = (kWTM + 63) / 64;        // A-scale DMAs per wave and stage (64 rows each)
  static constexpr int kLoadsPerStage = kQW + kSD;
  static constexpr int kAOff = 0;
  static constexpr int kBOff = kAQ * 1024;
  static constexpr int kSOff = kBOff + kBQ * 1024;
  static constexpr int kStage = kSOff + NW * kSD * 256;  // 64 fp32 A scales per scale DMA
  static constexpr int kLds = S * kStage;
  // scale ring (the prefetching K loop with row-major activation scales): two slots, each
  // 4 K blocks x 64 rows of fp32 scales (1 KB) per wave row, held in the scale regions of
  // stages 0 and 1 (which the ring mode's stage DMAs leave alone)
  static constexpr bool kRingFits = kWTM == 64 && WM * 1024 <= NW * kSD * 256 && S >= 2;
  // more than 4 row tiles per wave: A fragments are read one row tile at a time,
  // just ahead of the 4 MFMAs that use them, instead of all at the start of a step
  static constexpr bool kStreamA = kWTM / 16 > 4;
  // g1u1 epilogue: rows per pass (a pass stages its fp32 gate/up rows in LDS) and
  // threads per output row (each takes 128 / kQPR columns)
  static constexpr int kEpR = BM < 128 ? BM : 128;
  static constexpr int kQPR = kThreads / kEpR >= 8 ? 8 : kThreads / kEpR;
  static_assert(MODE != kG1U1 || (kQPR >= 1 && 128 % kQPR == 0 && 128 / kQPR % 16 == 0), "g1u1 epilogue split");
  static_assert(BM % kEpR == 0 && (kWTM <= kEpR ? kEpR % kWTM == 0 : kWTM % kEpR == 0), "epilogue passes");
  static constexpr int kRed = kQPR;
  static_assert(kWTM % 16 == 0 && kWTNB % 16 == 0, "wave tile must be whole MFMA tiles");
  static_assert(kWTNB <= 128 && 128 % kWTNB == 0, "a wave's columns lie in one 128-column scale block");
  static_assert(kWTM <= 128, "at most two A-scale DMAs per wave");
  static_assert(MODE != kG1U1 || BNB == 256, "g1u1 stages 128 gate and 128 up rows");
  static_assert(kWN % kParts == 0, "gate and up waves split evenly");
  static_assert(S >= 2 && S <= 4 && 2 * kLoadsPerStage < 64, "pipeline depth");
  static_assert(kLds + (MODE == kDown ? 2 : 1) * BM * 4 + kRed * kEpR * 4 <= 160 * 1024, "LDS of one workgroup");
};


// calls f(integral_constant<int, i>) for i = 0 .. N-1 in order
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
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
// LDS of one tile of the engine
template <class C>
struct GemmSmem {
  __attribute__((aligned(16))) uint8_t lds[C::kLds];
  int rowinfo[C::BM];
  float roww[C::kMode == kDown ? C::BM : 1];  // down: routing weights of the tile's rows
  float red[C::kRed][C::kEpR];
#ifdef MOE355_PHASE_TRACE
  uint32_t trace[8][64][3];  // per wave and K step: clock before the wait, after it, after the barrier
#endif
};

#ifdef MOE355_PHASE_TRACE
}  // namespace
}  // namespace moe355
#include "../../include/moe355_trace.h"
namespace moe355 {
namespace {
// Diagnostic build only (libmoe355_trace.so): per-step phase clocks (s_memtime) of the
// gate/up kernel on 128-row tiles, tiles [0, kTraceTiles) of each launch, up to 64 K
// steps, read back with moe355_phase_trace_read.
constexpr int kTraceTiles = 64;
__device__ uint32_t g_phase_trace[kTraceTiles][8][64][3];
#endif

// One output tile (tile index `tile_id` of the launch grid) with the workgroup's LDS.
// Every thread of the workgroup calls it with the same tile; it returns (uniformly)
// for tiles past the problem.
//
// SR (scale ring; the prefetching K loop on 64- and 128-row tiles, row-major activation
// scales with a 16-byte aligned row stride, K blocks a multiple of 4): instead of every
// wave fetching its rows' scales with a 4-byte DMA per K step (the waves of one wave row
// all fetching the same 64 values), the first wave of each wave row fetches 4 K blocks
// of its 64 rows' scales with one 16-byte DMA every fourth step into a two-slot LDS ring.
// Same scale values, so the same results bit for bit; 8 DMA instructions per step fewer
// on the 128-row tile.
template <class C, int MODE, bool PK, bool BSH, bool SR = false>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, const int64_t tile_id, GemmSmem<C>& sm) {
  static_assert(!PK || MODE == kDense, "partial K blocks: dense mode only");
  constexpr bool kPrefetch = !PK && !C::kStreamA && C::BM >= 64;
  constexpr bool kSR = SR && kPrefetch && C::kRingFits;
  static_assert(!SR || kSR, "the scale ring needs the prefetching K loop");
  static_assert(!(PK && BSH), "pre-shuffled B has whole 128x128 tiles");
  constexpr int64_t kBStep = BSH ? 128 * 128 : 128;  // bytes between K blocks of a B row
  // pre-shuffled B blocks are 1 KB copies from the first row of 8; their offset goes
  // in the wave-uniform address for the 128-row tiles (short of VGPRs) and in the
  // per-lane offset for the smaller ones (short of SGPRs)
  constexpr bool kBUni = BSH && C::BM == 128;
  uint8_t* const lds = sm.lds;
  int* const rowinfo = sm.rowinfo;
  float (&red)[C::kRed][C::kEpR] = sm.red;

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
  int64_t tile = tile_id;
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
    for (int i = tid; i < C::BM; i += C::kThreads) {
      rowinfo[i] = g.sorted_ids[row0 + i];
      // down: the weights too, so that the epilogue reads them from LDS
      if constexpr (MODE == kDown) sm.roww[i] = g.sorted_w[row0 + i];
    }
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
  // kAOwn (the prefetching K loop): wave w moves A blocks 2w and 2w + 1, the rows of its own
  // 16-row MFMA tile (tile wn of wave row wm), so a wave whose tile holds only padding skips
  // its A DMAs altogether; otherwise wave w moves A blocks w, w + NW, ...
  constexpr bool kAOwn = kPrefetch && kJA == 2 && C::kWTM == 16 * C::kWN && C::kAQ == C::kAQ0;
  auto dma_block = [&](int j) { return kAOwn && j < kJA ? kJA * w + j : w + j * C::NW; };
  // this wave's A rows hold at least one valid row (uniform)
  const bool a_live = !kAOwn || 16 * w < nrows;
  uint32_t voff[C::kQW];
#pragma unroll
  for (int j = 0; j < C::kQW; ++j) {
    const int q = dma_block(j);
    const bool is_a = BSH ? j < kJA : q < C::kAQ;
    const int qq = is_a ? q : q - C::kAQ;
    const int r = qq * 8 + (lane >> 3);
    const int ch = (lane & 7) ^ (r & 7);
    if (is_a) {
      // a block of 8 rows that holds only padding (or rows past M) reads 16 bytes of the
      // first row into every slot instead: its rows are never used
      voff[j] = qq * 8 < nrows ? (uint32_t)(a_row(r < C::BM ? r : 0) * g.K + ch * 16) : 0u;
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
  // scale DMA d of this wave moves the A scales of its rows [64d, 64d + 64)
  uint32_t soff[C::kSD];
#pragma unroll
  for (int d = 0; d < C::kSD; ++d) {
    const int rr = d * 64 + lane;
    soff[d] = (uint32_t)(a_row(wm * C::kWTM + (rr < C::kWTM ? rr : 0)) * g.ssm * 4);
  }
  const uint8_t* s_base = uniform_ptr(g.a_scale);
  const int sofs = C::kSOff + w * C::kSD * 256;
  // scale ring: K blocks [4 grp, 4 grp + 4) of wave row wm's scales into ring slot grp & 1,
  // lane L moving row wm * 64 + L's 16 bytes.  Group 0 goes out from every wave of the row
  // with the pipeline prologue (the same bytes to the same place); later groups from the row's
  // first wave only, between K steps.  Ring slot s of wave row wm: the scale region of stage s.
  auto ring_ofs = [&](int slot) { return slot * C::kStage + C::kSOff + wm * 1024; };
  const uint32_t soff_r = kSR ? (uint32_t)(a_row(wm * C::kWTM + lane) * g.ssm * 4) : 0u;
  auto issue_scales = [&](int grp) {
    dma16(s_base + (int64_t)(kbase + 4 * grp) * 4, soff_r, lds_addr(lds) + ring_ofs(grp & 1));
  };

  vm_wait<0>();  // every ordinary load lands before the first DMA is queued

  const uint32_t lds0 = lds_addr(lds);
  // DMA j of this wave for K block kb into LDS stage `stage`: j < kQW moves A/B
  // rows, j >= kQW the wave's A scales
  // (every operand but voff / soff is wave-uniform: addresses and m0 stay in SGPRs)
  auto issue_one = [&](int stage, int kb, int j) {
    const uint32_t base = lds0 + stage * C::kStage;
    const int64_t kg = kbase + kb;  // K block in the whole problem
    if (j < C::kQW) {
      const int q = dma_block(j);
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
      const int d = j - C::kQW;
      dma4(s_base + kg * g.sskb * 4, soff[d], base + sofs + d * 256);
    }
  };
  auto issue = [&](int stage, int kb) {
#pragma unroll
    for (int j = 0; j < C::kLoadsPerStage; ++j) issue_one(stage, kb, j);
  };

  v4f acc[C::kTM][C::kTN];
#pragma unroll
  for (int tm = 0; tm < C::kTM; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::kTN; ++tn) acc[tm][tn] = v4f{0.f, 0.f, 0.f, 0.f};

  const int lr = lane & 15, lg = lane >> 4;

  // one K step on LDS stage `stage`; only the first TMV row tiles of the wave are computed
  // RF 1: the step refills its stage (steady state, no branches); RF 0: checked
  auto step = [&](const int kb, const int stage, auto tmv_c, auto rf_c) {
    constexpr int TMV = decltype(tmv_c)::value;
    constexpr int RF = decltype(rf_c)::value;
#ifdef MOE355_PHASE_TRACE
    constexpr bool kTrace = MODE == kG1U1 && C::BM == 128;
    uint32_t* const tr = kTrace ? &sm.trace[w][min(kb, 63)][0] : nullptr;
    if constexpr (kTrace) tr[0] = (uint32_t)__builtin_amdgcn_s_memtime();
#endif
    if constexpr (RF == 1) {
      vm_wait<(C::S - 2) * C::kLoadsPerStage>();
    } else {
      vm_wait_stages<C::kLoadsPerStage>(min(C::S - 2, KBp - 1 - kb));
    }
#ifdef MOE355_PHASE_TRACE
    if constexpr (kTrace) tr[1] = (uint32_t)__builtin_amdgcn_s_memtime();
#endif
    barrier_only();
#ifdef MOE355_PHASE_TRACE
    if constexpr (kTrace) tr[2] = (uint32_t)__builtin_amdgcn_s_memtime();
#endif
    const bool refill = RF == 1 || kb + C::S - 1 < KBp;
    const int nstage = (stage + C::S - 1) % C::S, nkb = kb + C::S - 1;
    if constexpr (TMV == 0) {
      if (refill) issue(nstage, nkb);
    } else {
      const uint8_t* st = lds + stage * C::kStage;
      const float sb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(kb < 64 ? sbv0 : sbv1), kb & 63));
      v8i av[TMV];
      v4f s4[TMV];
      auto load_a = [&](int tm) {
        av[tm] = lds_frag(st + C::kAOff, wm * C::kWTM + tm * 16, lane);
        s4[tm] = *reinterpret_cast<const v4f*>(st + sofs + (tm * 16 + 4 * lg) * 4) * sb;
      };
      if constexpr (!C::kStreamA) {
#pragma unroll
        for (int tm = 0; tm < TMV; ++tm) load_a(tm);
      } else {
        load_a(0);
      }
      v8i bv[C::kTN];
#pragma unroll
      for (int tn = 0; tn < C::kTN; ++tn) bv[tn] = lds_frag(st + C::kBOff, wn * C::kWTNB + tn * 16, lane);
      // rolling window: tile q is issued, tile q-2 is folded.  The refill DMAs of
      // the stage freed by the barrier are spread between the MFMAs (DMA j after
      // MFMA j * kGap), so a wave never stalls on a burst of DMA issues.  Tile
      // order: row tile fastest, or (kStreamA) column tile fastest so that one row
      // tile's fragment serves 4 consecutive MFMAs and the next is read meanwhile.
      constexpr int NQ = TMV * C::kTN;
      constexpr int kGap = NQ / C::kLoadsPerStage > 0 ? NQ / C::kLoadsPerStage : 1;
      auto tile_m = [](int q) { return C::kStreamA ? q / C::kTN : q % TMV; };
      auto tile_n = [](int q) { return C::kStreamA ? q % C::kTN : q / TMV; };
      v4f tq[3];
#pragma unroll
      for (int q = 0; q < NQ + 2; ++q) {
        if constexpr (C::kStreamA) {
          if (q < NQ && tile_n(q) == 0 && tile_m(q) + 1 < TMV) load_a(tile_m(q) + 1);
        }
        if (q < NQ) tq[q % 3] = mfma16x16x128_fp8(av[tile_m(q)], bv[tile_n(q)], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int j = 0; j < C::kLoadsPerStage; ++j)
          if (refill && (j * kGap < NQ + 1 ? j * kGap : NQ + 1) == q) issue_one(nstage, nkb, j);
        if (q >= 2) {
          const int p = q - 2;
          acc[tile_m(p)][tile_n(p)] += tq[p % 3] * s4[tile_m(p)];
        }
      }
    }
  };
  // unrolled by the stage count: every LDS address is base + immediate
  // (its first S - 1 stages are issued before the row-tile dispatch below)
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
#pragma unroll
        for (int d = 0; d < C::kSD; ++d)
          *reinterpret_cast<float*>(lds + sofs + d * 256 + lane * 4) =
              *reinterpret_cast<const float*>(s_base + kg * g.sskb * 4 + soff[d]);
        lgkm_wait0();
        step(KBp, 0, tmv_c, std::integral_constant<int, 0>{});
      }
    }
  };
  // K loop with the fragments of block kb + 1 read during step kb (whole K blocks only).
  // Every fragment register takes the next block's data right after its last use in the
  // step's MFMA sequence (weight fragments early in the step, activation fragments and
  // their scales towards its end), so a step starts on operands already in registers
  // instead of all waves reading LDS at once behind the barrier.  Step kb: wait for this
  // wave's DMAs of block kb + 1, wait for its own LDS reads (they read block kb's stage,
  // which is refilled next), barrier (block kb + 1 is published and no wave reads block kb's
  // stage any more), refill block kb's stage with block kb + S, then block kb's MFMAs with
  // block kb + 1's reads between them.  All S stages are in flight ahead of the registers.
  // LA 0: this wave's A rows are all padding (kAOwn), so its DMAs of a stage are the B
  // blocks (and scales) only, j = J0 .. J0 + L - 1
  auto kloop_pf = [&](auto tmv_c, auto la_c) {
    constexpr int TMV = decltype(tmv_c)::value;
    constexpr int NQ = TMV * C::kTN;
    static_assert(!C::kStreamA, "row tile fastest");
    constexpr int J0 = decltype(la_c)::value ? 0 : kJA;
    static_assert(J0 == 0 || kAOwn, "A DMAs are skipped only where each wave moves its own tile's rows");
    constexpr int L = (kSR ? C::kQW : C::kLoadsPerStage) - J0;  // DMAs of a stage per wave
    static_assert(C::S * L < 64 && L > 0, "vmcnt range of the prefetching K loop");
    auto issue_pf = [&](int stage, int kb) {
#pragma unroll
      for (int j = 0; j < L; ++j) issue_one(stage, kb, J0 + j);
    };
    auto wait_blocks = [&](int a) {  // at most a blocks of this wave's DMAs still outstanding
      if (a >= 3) {
        vm_wait<3 * L>();
      } else if (a == 2) {
        vm_wait<2 * L>();
      } else if (a == 1) {
        vm_wait<L>();
      } else {
        vm_wait<0>();
      }
    };
    // (scale ring: the scales of blocks 0-3 go out ahead of block 0; a wait for block kb
    // then also covers the scales of its group, which were issued before it)
    if constexpr (kSR) issue_scales(0);
#pragma unroll
    for (int s = 0; s < C::S; ++s)
      if (s < KBp) issue_pf(s, s);
    v8i av[TMV > 0 ? TMV : 1], bv[C::kTN];
    v4f s4[TMV > 0 ? TMV : 1];
    auto sb_of = [&](int kb) {
      return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(kb < 64 ? sbv0 : sbv1), kb & 63));
    };
    auto read_a = [&](const uint8_t* st, int tm) { av[tm] = lds_frag(st + C::kAOff, wm * C::kWTM + tm * 16, lane); };
    auto read_s = [&](const uint8_t* st, int tm, float sb, int kbr) {
      if constexpr (kSR) {
        // slot (kbr / 4) & 1, rows of 16 bytes (4 K blocks each)
        const float* rg = reinterpret_cast<const float*>(lds + ring_ofs((kbr >> 2) & 1)) + (tm * 16 + 4 * lg) * 4 +
                          (kbr & 3);
        s4[tm] = v4f{rg[0], rg[4], rg[8], rg[12]} * sb;
      } else {
        s4[tm] = *reinterpret_cast<const v4f*>(st + sofs + (tm * 16 + 4 * lg) * 4) * sb;
      }
    };
    auto read_b = [&](const uint8_t* st, int tn) { bv[tn] = lds_frag(st + C::kBOff, wn * C::kWTNB + tn * 16, lane); };
    wait_blocks(min(C::S - 1, KBp - 1));
    barrier_only();
    if constexpr (TMV > 0) {
      const float sb = sb_of(0);
#pragma unroll
      for (int tm = 0; tm < TMV; ++tm) {
        read_a(lds, tm);
        read_s(lds, tm, sb, 0);
      }
#pragma unroll
      for (int tn = 0; tn < C::kTN; ++tn) read_b(lds, tn);
    }
    // RF 1: the step refills (kb + S < KBp, no branches); RF 0: checked.  NX: block kb + 1 exists
    auto step = [&](const int kb, const int stage, auto rf_c, auto nx_c) {
      constexpr int RF = decltype(rf_c)::value;
      constexpr int NX = decltype(nx_c)::value;
#ifdef MOE355_PHASE_TRACE
      constexpr bool kTrace = MODE == kG1U1 && C::BM == 128;
      uint32_t* tr = nullptr;
      if constexpr (kTrace) tr = &sm.trace[w][min(kb, 63)][0];
      if constexpr (kTrace) tr[0] = (uint32_t)__builtin_amdgcn_s_memtime();
#endif
      if constexpr (NX) {
        if constexpr (RF == 1) {
          vm_wait<(C::S - 2) * L>();
        } else {
          wait_blocks(min(C::S - 2, KBp - 2 - kb));
        }
      }
      lgkm_wait0();
#ifdef MOE355_PHASE_TRACE
      if constexpr (kTrace) tr[1] = (uint32_t)__builtin_amdgcn_s_memtime();
#endif
      barrier_only();
#ifdef MOE355_PHASE_TRACE
      if constexpr (kTrace) tr[2] = (uint32_t)__builtin_amdgcn_s_memtime();
#endif
      const bool refill = RF == 1 || kb + C::S < KBp;
      const int nkb = kb + C::S;
      if constexpr (TMV == 0) {
        if (refill) issue_pf(stage, nkb);
      } else {
        const uint8_t* nst = lds + ((stage + 1) % C::S) * C::kStage;
        const float sbn = NX ? sb_of(kb + 1) : 0.0f;
        // tile q: row tile q % TMV, column tile q / TMV; the refill DMAs of block kb's stage
        // are spread between the MFMAs; the fold of q - 2 follows MFMA q
        constexpr int kGap = NQ / L > 0 ? NQ / L : 1;
        v4f tq[3];
#pragma unroll
        for (int q = 0; q < NQ + 2; ++q) {
          if (q < NQ) tq[q % 3] = mfma16x16x128_fp8(av[q % TMV], bv[q / TMV], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int j = 0; j < L; ++j)
            if (refill && (j * kGap < NQ + 1 ? j * kGap : NQ + 1) == q) issue_one(stage, nkb, J0 + j);
          if (q >= 2) {
            const int pq = q - 2;
            acc[pq % TMV][pq / TMV] += tq[pq % 3] * s4[pq % TMV];
          }
          if constexpr (NX) {
            if (q < NQ && q % TMV == TMV - 1) read_b(nst, q / TMV);        // last use of bv[q / TMV]
            if (q < NQ && q / TMV == C::kTN - 1) read_a(nst, q % TMV);     // last use of av[q % TMV]
            if (q >= 2 && (q - 2) / TMV == C::kTN - 1) read_s(nst, (q - 2) % TMV, sbn, kb + 1);  // its last fold
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    using One = std::integral_constant<int, 1>;
    using Zero = std::integral_constant<int, 0>;
    int kb0 = 0;
    // Scale ring: group ng (K blocks 4 ng .. 4 ng + 3) goes out at the start of a step s
    // (before its wait) with 4 ng - 4 <= s <= 4 ng - 2.  From s >= 4 ng - 4: the slot's
    // previous group (ng - 2) was last read during step 4 ng - 6, and those reads completed
    // before the barrier of step 4 ng - 5.  From s <= 4 ng - 2: the group's first read is
    // during step 4 ng - 1, whose wait leaves only the DMAs of step 4 ng - 2 outstanding.
    // Rounds start every S = 3 steps, so each such window of 3 steps holds one, and the issue
    // sits between steps, outside the MFMA sequences.
    int ng = 1;
    auto ring_issue = [&](int s) {
      if constexpr (kSR) {
        static_assert(!kSR || C::S <= 3, "one round start in every 3-step window");
        if (4 * ng < KBp && s >= 4 * ng - 4) {
          // the first wave of the row fetches the group; the others see it behind the barrier
          // of step 4 ng - 1, which follows its wait for its DMAs of the steps before
          if (wn == 0) issue_scales(ng);
          ++ng;
        }
      }
    };
    // rounds of S steps whose every step refills (kb + S < KBp for the round's last step)
    for (; kb0 + 2 * C::S - 1 < KBp; kb0 += C::S) {
      ring_issue(kb0);
      static_for<C::S>([&](auto uc) { step(kb0 + decltype(uc)::value, decltype(uc)::value, One{}, One{}); });
    }
    for (; kb0 < KBp; ++kb0) {
      ring_issue(kb0);
      if (kb0 + 1 < KBp) {
        step(kb0, kb0 % C::S, Zero{}, One{});
      } else {
        step(kb0, kb0 % C::S, Zero{}, Zero{});
      }
    }
  };
  static_assert(C::kTM <= 8, "row tiles per wave");
  // the prefetching loop for whole K blocks on tiles of 64 rows or more; 16- and 32-row
  // tiles (decode-sized grouped blocks, split-K dense runs of a few K blocks) keep kloop,
  // whose shallower prologue measured no slower there, and so does the partial block of PK
  if constexpr (!kPrefetch) {
#pragma unroll
    for (int s = 0; s < C::S - 1; ++s)
      if (s < KBp) issue(s, s);
  }
  auto kloop_any = [&](auto tmv_c) {
    constexpr int TMV = decltype(tmv_c)::value;
    using One = std::integral_constant<int, 1>;
    using Zero = std::integral_constant<int, 0>;
    if constexpr (kPrefetch) {
      if constexpr (!kAOwn || TMV == C::kTM) {
        kloop_pf(tmv_c, One{});  // (every tile of a full wave row holds valid rows)
      } else if constexpr (TMV == 0) {
        kloop_pf(tmv_c, Zero{});
      } else {
        if (a_live) {
          kloop_pf(tmv_c, One{});
        } else {
          kloop_pf(tmv_c, Zero{});
        }
      }
    } else {
      kloop(tmv_c);
    }
  };
  switch (tm_live) {
    case 0: kloop_any(std::integral_constant<int, 0>{}); break;
    case 1: kloop_any(std::integral_constant<int, 1>{}); break;
    case 2: if constexpr (C::kTM >= 2) kloop_any(std::integral_constant<int, 2>{}); break;
    case 3: if constexpr (C::kTM >= 3) kloop_any(std::integral_constant<int, 3>{}); break;
    case 4: if constexpr (C::kTM >= 4) kloop_any(std::integral_constant<int, 4>{}); break;
    case 5: if constexpr (C::kTM >= 5) kloop_any(std::integral_constant<int, 5>{}); break;
    case 6: if constexpr (C::kTM >= 6) kloop_any(std::integral_constant<int, 6>{}); break;
    case 7: if constexpr (C::kTM >= 7) kloop_any(std::integral_constant<int, 7>{}); break;
    default: if constexpr (C::kTM >= 8) kloop_any(std::integral_constant<int, 8>{}); break;
  }
  vm_wait<0>();
  __syncthreads();
#ifdef MOE355_PHASE_TRACE
  if constexpr (MODE == kG1U1 && C::BM == 128) {
    if (tile_id < kTraceTiles)
#pragma unroll
      for (int i = 0; i < 3; ++i) g_phase_trace[tile_id][w][lane][i] = sm.trace[w][lane][i];
  }
#endif

  // ---- epilogues (LDS is free again)
  if (MODE == kDense && C::BM <= 128 && g.splits > 1) {
    // split-K partial: fp32 tile [BM][BNB] in LDS (rows padded by 16 bytes so that
    // rows 4 apart do not share banks), then 16-byte stores into part[ks]
    // (the host splits K only for M tiles of at most 64 rows)
    constexpr int RS = C::BNB + 4;
    static_assert(C::BM > 128 || C::BM * RS * 4 <= C::kLds, "padded fp32 output tile fits the pipeline LDS");
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
    // bf16 tile [BM][BNB] in LDS (rows padded by 16 bytes), then 16-byte row stores, non-
    // temporal: the output is not read again here and cached stores evict the operands
    // (4096 x 18432 x 7168: 645 -> 598 us)
    constexpr int RS = C::BNB + 8;
    static_assert(C::BM * RS * 2 <= C::kLds, "bf16 output tile fits the pipeline LDS");
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
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(ob + r * RS + ch * 8),
                                    reinterpret_cast<u32x4*>(g.c + m * g.ldc + (int64_t)nt * C::BNB + ch * 8));
    }
  } else if constexpr (MODE == kDown) {
    // routing-weighted fp32 rows straight from the MFMA layout: for each of its rows
    // a group of 16 lanes writes 64 contiguous bytes per row tile (the neighbouring
    // column tiles complete the 128-byte lines in L2).  Non-temporal stores: the staging
    // is read once, by the combine, so it should not push the GEMM's operands out of L2
    // (prefill down + combine -2%, skew -8%)
#pragma unroll
    for (int tm = 0; tm < C::kTM; ++tm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = wm * C::kWTM + tm * 16 + 4 * lg + i;
        const int pid = rowinfo[rl];
        if (row0 + rl < nvalid && pid < npairs) {
          const float wgt = sm.roww[rl];
          float* yr = g.y + (int64_t)pid * g.N + (int64_t)nt * C::BNB + wn * C::kWTNB + lr;
#pragma unroll
          for (int tn = 0; tn < C::kTN; ++tn) __builtin_nontemporal_store(acc[tm][tn][i] * wgt, yr + tn * 16);
        }
      }
  } else {
    // Both parts stage their fp32 tiles in LDS as rows [gate 128 | up 128] (row
    // stride kFS words: conflict-free stores), kEpR rows per pass.  Then each thread
    // takes kCPI consecutive columns of one row: h = SiLU(gate) * up, the row's amax
    // over its 128 columns (partial maxima through red), 1x128 requantisation, and
    // 16-byte stores of the codes straight to h8.
    constexpr int kFS = 2 * 128 + 4;
    constexpr int kEpR = C::kEpR;
    constexpr int kQPR = C::kQPR, kCPI = 128 / kQPR;
    static_assert(kEpR * kFS * 4 <= C::kLds, "gate/up rows of a pass fit the pipeline LDS");
    float* F = reinterpret_cast<float*>(lds);
    const int r = tid % kEpR, qc = tid / kEpR;  // row (within a pass) and column group of this thread
    const bool active = qc < kQPR;
#pragma unroll
    for (int pass = 0; pass < C::BM / kEpR; ++pass) {
      if (pass > 0) __syncthreads();  // the previous pass has read F and red
      const int wrow0 = wm * C::kWTM - pass * kEpR;  // this wave's first row inside the pass
      if (wrow0 >= 0 && wrow0 < kEpR) {
#pragma unroll
        for (int tm = 0; tm < C::kTM; ++tm)
#pragma unroll
          for (int tn = 0; tn < C::kTN; ++tn)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              F[(wrow0 + tm * 16 + 4 * lg + i) * kFS + part * 128 + colofs + tn * 16 + lr] = acc[tm][tn][i];
      }
      __syncthreads();
      const int rt = pass * kEpR + r;  // row inside the tile
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
      if (active && rowinfo[rt] < npairs) {
        float amax = red[0][r];
#pragma unroll
        for (int k2 = 1; k2 < kQPR; ++k2) amax = fmaxf(amax, red[k2][r]);
        const float sc = (amax == 0.0f) ? 1.0f : amax / kE4M3Max;
        uint32_t wds[kCPI / 4];
#pragma unroll
        for (int v = 0; v < kCPI / 4; ++v)
          wds[v] = f32x4_to_e4m3(h[4 * v] / sc, h[4 * v + 1] / sc, h[4 * v + 2] / sc, h[4 * v + 3] / sc);
        uint8_t* dst = g.h8 + (row0 + rt) * g.N + nt * 128 + qc * kCPI;
#pragma unroll
        for (int v = 0; v < kCPI / 16; ++v)
          *reinterpret_cast<u32x4*>(dst + 16 * v) = u32x4{wds[4 * v], wds[4 * v + 1], wds[4 * v + 2], wds[4 * v + 3]};
        if (qc == 0) g.h_scale[(row0 + rt) * (g.N / 128) + nt] = sc;
      }
    }
  }
}

template <class C, int MODE, bool PK = false, bool BSH = false, bool SR = false>
__global__ __launch_bounds__(C::kThreads) void bs_gemm_kernel(GemmArgs g) {
  __shared__ GemmSmem<C> sm;
  gemm_tile<C, MODE, PK, BSH, SR>(g, blockIdx.x, sm);
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

// The expert computation of the layer in one cooperative launch ("Blockscale FP8 MoE
// Computation": the pages run sorted buffers -> moe_buf as a single call): persistent
// workgroups walk the gate/up tiles, the runtime's grid barrier publishes every h8
// row (it is a device-scope release/acquire, so rows written on one XCD are read
// correctly on another), the workgroups walk the down tiles, a second barrier
// publishes the per-pair staging, and they sum each token's pairs as combine_kernel
// does.  Each tile runs exactly the arithmetic of the two-launch path.
struct FusedArgs {
  GemmArgs gu, dn;             // the gate/up and down launches' arguments
  int nt_gu, nt_dn;            // their N tiles per sorted block
  uint16_t* out;
  int64_t ld_out;
};

template <class CG, class CD>
__global__ __launch_bounds__(CG::kThreads) void fused_moe_kernel(FusedArgs f) {
  static_assert(CG::kThreads == CD::kThreads, "both GEMMs run with the same workgroup size");
  union Smem {
    GemmSmem<CG> g;
    GemmSmem<CD> d;
  };
  __shared__ Smem sm;
  cooperative_groups::grid_group grid = cooperative_groups::this_grid();
  // only the blocks below num_valid hold rows
  const int nvalid = f.gu.num_valid[0];
  const int64_t nblk = nvalid > 0 ? nvalid / CG::BM : 0;
  for (int64_t t = blockIdx.x; t < nblk * f.nt_gu; t += gridDim.x) {
    __syncthreads();  // the previous tile is done with the LDS
    gemm_tile<CG, kG1U1, false, false>(f.gu, t, sm.g);
  }
  grid.sync();
  for (int64_t t = blockIdx.x; t < nblk * f.nt_dn; t += gridDim.x) {
    __syncthreads();
    gemm_tile<CD, kDown, false, false>(f.dn, t, sm.d);
  }
  grid.sync();
  if (nvalid < 0) return;  // ids outside [0, E): nothing was placed
  const int T = f.dn.T, k = f.dn.topk, H = f.dn.N, H8 = H / 8;
  const int64_t n8 = (int64_t)T * H8;
  for (int64_t idx = (int64_t)blockIdx.x * CG::kThreads + threadIdx.x; idx < n8;
       idx += (int64_t)gridDim.x * CG::kThreads) {
    const int64_t t = idx / H8;
    const int c8 = (int)(idx - t * H8);
    float s8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const float4* p = reinterpret_cast<const float4*>(f.dn.y + ((t * k + j) * (int64_t)H + c8 * 8));
      const float4 a = p[0], b = p[1];
      s8[0] += a.x;
      s8[1] += a.y;
      s8[2] += a.z;
      s8[3] += a.w;
      s8[4] += b.x;
      s8[5] += b.y;
      s8[6] += b.z;
      s8[7] += b.w;
    }
    const u32x4 o{f32_to_bf16(s8[0]) | (f32_to_bf16(s8[1]) << 16), f32_to_bf16(s8[2]) | (f32_to_bf16(s8[3]) << 16),
                  f32_to_bf16(s8[4]) | (f32_to_bf16(s8[5]) << 16), f32_to_bf16(s8[6]) | (f32_to_bf16(s8[7]) << 16)};
    *reinterpret_cast<u32x4*>(f.out + t * f.ld_out + c8 * 8) = o;
  }
}

// The scale ring (see gemm_tile) applies when the activation scales are row-major with a
// row stride of whole 16-byte groups, 16-byte aligned, and every workgroup's K blocks
// come in whole groups of 4.
bool scale_ring_ok(const GemmArgs& g) {
  const int64_t KB = ceil_div64(g.K, 128);
  return g.sskb == 1 && g.ssm % 4 == 0 && (reinterpret_cast<uintptr_t>(g.a_scale) & 15u) == 0 && g.K % 128 == 0 &&
         KB % 4 == 0 && g.kbs % 4 == 0;
}

template <class C, int MODE, bool PK, bool BSH>
int launch_cfg(const GemmArgs& g, int64_t mblocks, hipStream_t stream) {
  if (MODE != kDense && g.N % C::kOutN != 0) return MOE355_EUNSUPPORTED;
  const int64_t grid = mblocks * ceil_div64(g.N, C::kOutN) * (MODE == kDense ? g.splits : 1);
  if (grid == 0) return MOE355_OK;
  MOE355_CHECK(grid < (1ll << 31), MOE355_EUNSUPPORTED);
  constexpr bool kRingable = !PK && !C::kStreamA && C::BM >= 64 && C::kRingFits;
  if (kRingable && scale_ring_ok(g)) {
    hipLaunchKernelGGL((bs_gemm_kernel<C, MODE, PK, BSH, kRingable>), dim3((unsigned)grid), dim3(C::kThreads), 0,
                       stream, g);
  } else {
    hipLaunchKernelGGL((bs_gemm_kernel<C, MODE, PK, BSH>), dim3((unsigned)grid), dim3(C::kThreads), 0, stream, g);
  }
  return launch_status();
}

// One cooperative launch of the fused kernel with as many workgroups as the GPU holds
// at once (the grid barrier needs every workgroup resident).
template <class CG, class CD>
int launch_fused_cfg(FusedArgs& f, hipStream_t stream) {
  const void* kern = reinterpret_cast<const void*>(&fused_moe_kernel<CG, CD>);
  int dev = -1, ncu = 0, coop = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, CG::kThreads, 0) != hipSuccess) {
    (void)hipGetLastError();
    return MOE355_ELAUNCH;
  }
  MOE355_CHECK(coop != 0, MOE355_EUNSUPPORTED);
  if (per_cu <= 0 || ncu <= 0) return MOE355_ELAUNCH;
  void* args[] = {&f};
  if (hipLaunchCooperativeKernel(kern, dim3((unsigned)(per_cu * ncu)), dim3(CG::kThreads), args, 0, stream) !=
      hipSuccess) {
    (void)hipGetLastError();
    return MOE355_ELAUNCH;
  }
  return MOE355_OK;
}

// the fused kernel runs the tile configurations launch_gemm picks for block_m
int launch_fused(FusedArgs& f, int bm, hipStream_t stream) {
  switch (bm) {
    case 16: return launch_fused_cfg<Cfg<kG1U1, 16, 256, 4, 1, 4>, Cfg<kDown, 16, 256, 4, 1, 4>>(f, stream);
    case 32: return launch_fused_cfg<Cfg<kG1U1, 32, 256, 4, 1, 4>, Cfg<kDown, 32, 256, 4, 1, 4>>(f, stream);
    case 64: return launch_fused_cfg<Cfg<kG1U1, 64, 256, 4, 1, 3>, Cfg<kDown, 64, 256, 4, 1, 3>>(f, stream);
    case 128: return launch_fused_cfg<Cfg<kG1U1, 128, 256, 8, 2, 3>, Cfg<kDown, 128, 256, 8, 2, 3>>(f, stream);
    default: return MOE355_EUNSUPPORTED;
  }
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
    case 256:
      // grouped GEMMs on 256 x 256 tiles (gemm_big.hip)
      if constexpr (PK || BNB != 256 || MODE == kDense) {
        return MOE355_EUNSUPPORTED;
      } else {
        return launch_big<MODE, BSH>(g, mblocks, stream);
      }
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

// splits -> K blocks per split (kbs) and the split count that covers K with it
void set_splits(DensePlan& p, int K, int splits) {
  const int KB = (int)ceil_div64(K, 128);
  p.kbs = (int)ceil_div64(KB, std::max(1, std::min(splits, KB)));
  p.splits = (int)ceil_div64(KB, p.kbs);
}

DensePlan dense_rule_plan(int M, int N, int K);

DensePlan dense_plan(int M, int N, int K) {
  // measured per-shape plans first (dense_tuned.h): the entry of this N and K whose M
  // range holds M
  const DenseTuned* best = nullptr;
  for (const DenseTuned& t : kDenseTuned)
    if (best == nullptr && t.n == N && t.k == K && t.m_min <= M && M <= t.m_max) best = &t;
  if (best != nullptr) {
    DensePlan p;
    p.bm = best->bm;
    p.bnb = best->bnb;
    // 16-column tiles split K inside the workgroup (no run limit); the others walk at
    // most kMaxKbs K blocks per run
    set_splits(p, K, best->bnb == 16 ? 1 : std::max(best->splits, (int)ceil_div64(ceil_div64(K, 128), kMaxKbs)));
    return p;
  }
  return dense_rule_plan(M, N, K);
}

DensePlan dense_rule_plan(int M, int N, int K) {
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

// fused workspace: h8 [max_sorted, I] | h_scale [max_sorted, I/128] | per-pair staging [T*topk, H]
struct FusedWs {
  size_t h8, hs, y, total;
};

int fused_ws_layout(int T, int H, int I, int E, int topk, int block_m, FusedWs* L) {
  MOE355_CHECK(T >= 0 && H > 0 && I > 0 && E > 0 && topk > 0, MOE355_EINVAL);
  MOE355_CHECK(I % 128 == 0, MOE355_EUNSUPPORTED);
  int64_t ms = 0;
  const int st = moe_sort_sizes(T, topk, E, block_m, &ms, nullptr, nullptr);
  if (st != MOE355_OK) return st;
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  L->h8 = 0;
  L->hs = up((size_t)ms * I);
  L->y = L->hs + up((size_t)ms * (I / 128) * sizeof(float));
  L->total = L->y + (size_t)T * topk * H * sizeof(float) + 256;
  return MOE355_OK;
}

}  // namespace

extern "C" int moe_fp8_blockscale_fused_workspace(int T, int H, int I, int E, int topk, int block_m, size_t* bytes) {
  MOE355_CHECK(bytes, MOE355_EINVAL);
  FusedWs L{};
  const int st = fused_ws_layout(T, H, I, E, topk, block_m, &L);
  if (st != MOE355_OK) return st;
  *bytes = L.total;
  return MOE355_OK;
}

namespace {

// forced: a caller-chosen tiling (gemm_fp8_blockscale_tiled), else the tuned / rule-based plan
int dense_gemm(const uint8_t* a8, const float* a_scale, int64_t sstride_m, int64_t sstride_kb, const uint8_t* b8,
               const float* b_scale, int M, int N, int K, uint16_t* c, int64_t ldc, int out_fp16, void* workspace,
               size_t workspace_bytes, hipStream_t stream, bool bsh, const DensePlan* forced = nullptr) {
  MOE355_CHECK(M >= 0 && N >= 0 && K >= 0 && ldc >= N && (out_fp16 == 0 || out_fp16 == 1), MOE355_EINVAL);
  MOE355_CHECK(K % 16 == 0 && N % 8 == 0, MOE355_EUNSUPPORTED);
  MOE355_CHECK(!bsh || (K % 128 == 0 && N % 128 == 0), MOE355_EUNSUPPORTED);
  MOE355_CHECK((int64_t)M * K < (1ll << 32) && (int64_t)N * K < (1ll << 32), MOE355_EUNSUPPORTED);
  if (M == 0 || N == 0) return MOE355_OK;
  MOE355_CHECK(K > 0 && a8 && a_scale && b8 && b_scale && c && sstride_m >= 0 && sstride_kb >= 0, MOE355_EINVAL);
  // the A-scale DMA takes a 32-bit byte offset per row: row * sstride_m * 4
  MOE355_CHECK((int64_t)M * sstride_m * 4 < (1ll << 32), MOE355_EUNSUPPORTED);
  MOE355_CHECK(aligned16(a8) && aligned16(b8) && aligned16(c) && ldc % 8 == 0, MOE355_EMISALIGNED);
  MOE355_CHECK((reinterpret_cast<uintptr_t>(a_scale) & 3u) == 0, MOE355_EMISALIGNED);
  DensePlan plan = forced ? *forced : dense_plan(M, N, K);
  if (plan.bnb == 16) {
    // small M: one workgroup per 16 columns, K split over its waves (dense_small.hip)
    MOE355_CHECK(M <= 64 && plan.splits == 1, MOE355_EUNSUPPORTED);
    DenseSmallArgs s{};
    s.a = a8;
    s.a_scale = a_scale;
    s.ssm = sstride_m;
    s.sskb = sstride_kb;
    s.b = b8;
    s.b_scale = b_scale;
    s.M = M;
    s.N = N;
    s.K = K;
    s.c = c;
    s.ldc = ldc;
    s.out_f16 = out_fp16;
    return launch_dense_small(s, bsh, stream);
  }
  const size_t need = dense_workspace_bytes(plan, M, N);
  if (forced != nullptr) {
    // a caller-chosen plan runs as given: its split of K needs the workspace
    MOE355_CHECK(plan.kbs <= kMaxKbs, MOE355_EUNSUPPORTED);
    MOE355_CHECK(need == 0 || (workspace != nullptr && workspace_bytes >= need), MOE355_EINVAL);
    MOE355_CHECK(need == 0 || aligned16(workspace), MOE355_EMISALIGNED);
  } else if (need == 0 || workspace == nullptr || workspace_bytes < need) {
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

GemmArgs g1u1_args(const uint8_t* a8, const float* a_scale, int64_t sstride_m, int64_t sstride_kb, const uint8_t* w1,
                   const float* w1_scale, const int32_t* sorted_ids, const int32_t* sorted_expert_ids,
                   const int32_t* num_valid, int T, int H, int I, int topk, uint8_t* h8, float* h_scale,
                   const float* fc2_smooth_scale) {
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
  return g;
}

GemmArgs down_args(const uint8_t* h8, const float* h_scale, const uint8_t* w2, const float* w2_scale,
                   const int32_t* sorted_ids, const float* sorted_weights, const int32_t* sorted_expert_ids,
                   const int32_t* num_valid, int T, int H, int I, int topk, float* y) {
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
  g.y = y;
  g.splits = 1;
  g.kbs = I / 128;
  return g;
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
  // the A-scale DMA takes a 32-bit byte offset per token row: t * sstride_m * 4
  MOE355_CHECK((int64_t)T * sstride_m * 4 < (1ll << 32), MOE355_EUNSUPPORTED);
  MOE355_CHECK(aligned16(a8) && aligned16(w1) && aligned16(h8), MOE355_EMISALIGNED);
  MOE355_CHECK((reinterpret_cast<uintptr_t>(a_scale) & 3u) == 0 && aligned16(fc2_smooth_scale),
               MOE355_EMISALIGNED);
  const GemmArgs g = g1u1_args(a8, a_scale, sstride_m, sstride_kb, w1, w1_scale, sorted_ids, sorted_expert_ids,
                               num_valid, T, H, I, topk, h8, h_scale, fc2_smooth_scale);
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
  const GemmArgs g = down_args(h8, h_scale, w2, w2_scale, sorted_ids, sorted_weights, sorted_expert_ids, num_valid, T,
                               H, I, topk, static_cast<float*>(workspace));
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

extern "C" int gemm_fp8_blockscale_tiled(const uint8_t* a8, const float* a_scale, int64_t sstride_m,
                                         int64_t sstride_kb, const uint8_t* b8, const float* b_scale, int M, int N,
                                         int K, uint16_t* c, int64_t ldc, int out_fp16, int tile_m, int tile_n,
                                         int splits, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  MOE355_CHECK(splits >= 1, MOE355_EINVAL);
  MOE355_CHECK((tile_m == 16 || tile_m == 32 || tile_m == 64 || tile_m == 128) &&
                   (tile_n == 16 || tile_n == 128 || tile_n == 256),
               MOE355_EUNSUPPORTED);
  // 16-column tiles: the small-M kernel (M <= 64, K split inside the workgroup)
  MOE355_CHECK(tile_n != 16 || (tile_m <= 64 && M <= tile_m && splits == 1), MOE355_EUNSUPPORTED);
  DensePlan p;
  p.bm = tile_m;
  p.bnb = tile_n;
  set_splits(p, K, splits);
  return dense_gemm(a8, a_scale, sstride_m, sstride_kb, b8, b_scale, M, N, K, c, ldc, out_fp16, workspace,
                    workspace_bytes, stream, false, &p);
}

extern "C" int gemm_fp8_blockscale_plan(int M, int N, int K, int measured, int* tile_m, int* tile_n, int* splits) {
  MOE355_CHECK(M >= 0 && N >= 0 && K >= 0 && tile_m && tile_n && splits, MOE355_EINVAL);
  MOE355_CHECK(K % 16 == 0 && N % 8 == 0, MOE355_EUNSUPPORTED);
  const DensePlan p = measured ? dense_plan(M, N, K) : dense_rule_plan(M, N, K);
  *tile_m = p.bm;
  *tile_n = p.bnb;
  *splits = p.splits;
  return MOE355_OK;
}

extern "C" int gemm_fp8_blockscale_tiled_workspace(int M, int N, int K, int splits, size_t* bytes) {
  MOE355_CHECK(M >= 0 && N >= 0 && K >= 0 && splits >= 1 && bytes, MOE355_EINVAL);
  DensePlan p{16, 128, 1, 1};
  set_splits(p, K, splits);
  *bytes = (M == 0 || N == 0 || K == 0) ? 0 : dense_workspace_bytes(p, M, N);
  return MOE355_OK;
}

extern "C" int gemm_fp8_blockscale_wpreshuffle(const uint8_t* a8, const float* a_scale, int64_t sstride_m,
                                               int64_t sstride_kb, const uint8_t* b8, const float* b_scale, int M,
                                               int N, int K, uint16_t* c, int64_t ldc, int out_fp16,
                                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return dense_gemm(a8, a_scale, sstride_m, sstride_kb, b8, b_scale, M, N, K, c, ldc, out_fp16, workspace,
                    workspace_bytes, stream, true);
}

// Static device scratch for gemm_fp8_blockscale_noalloc: the split-K partial sums.
// Host code never uses this name as an address: the address on each device comes
// from hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) uint8_t scratch[MOE355_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The current device's copy of `scratch` (looked up on its first use).
int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE355_ELAUNCH;
  MOE355_CHECK(dev >= 0 && dev < kMaxScratchDevices, MOE355_EUNSUPPORTED);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return MOE355_ELAUNCH;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE355_OK;
}

}  // namespace

extern "C" int gemm_fp8_blockscale_noalloc(const uint8_t* a8, const float* a_scale, int64_t sstride_m,
                                           int64_t sstride_kb, const uint8_t* b8, const float* b_scale, int M, int N,
                                           int K, uint16_t* c, int64_t ldc, int out_fp16, hipStream_t stream) {
  // the shape checks of the workspace query come first (host only), then the size rule
  size_t need = 0;
  const int st = gemm_fp8_blockscale_workspace(M, N, K, &need);
  if (st != MOE355_OK) return st;
  MOE355_CHECK(need <= MOE355_STATIC_SCRATCH_BYTES, MOE355_ESCRATCH);
  void* ws = nullptr;
  if (need > 0 && (int64_t)M * N > 0) {
    const int s2 = device_scratch(&ws);
    if (s2 != MOE355_OK) return s2;
  }
  return dense_gemm(a8, a_scale, sstride_m, sstride_kb, b8, b_scale, M, N, K, c, ldc, out_fp16, ws, need, stream,
                    false);
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

extern "C" int moe_fp8_blockscale_fused(const uint8_t* a8, const float* a_scale, int64_t sstride_m, int64_t sstride_kb,
                                        const uint8_t* w1, const float* w1_scale, const uint8_t* w2,
                                        const float* w2_scale, const int32_t* sorted_ids, const float* sorted_weights,
                                        const int32_t* sorted_expert_ids, const int32_t* num_valid, int T, int H,
                                        int I, int E, int topk, int block_m, int64_t max_sorted,
                                        const float* fc2_smooth_scale, uint16_t* out, int64_t ld_out, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
  // the checks of the gate/up and down calls together
  MOE355_CHECK(T >= 0 && H > 0 && I > 0 && E > 0 && topk > 0 && ld_out >= H, MOE355_EINVAL);
  MOE355_CHECK(H % 256 == 0 && I % 128 == 0 && H <= 16384 && I <= 16384 && block_m != 256 && valid_block_m(block_m),
               MOE355_EUNSUPPORTED);
  MOE355_CHECK((int64_t)T * H < (1ll << 32) && (int64_t)2 * I * H < (1ll << 32) && max_sorted * I < (1ll << 32),
               MOE355_EUNSUPPORTED);
  const int cap = check_sorted_capacity(T, topk, E, block_m, max_sorted);
  if (cap != MOE355_OK) return cap;
  if (T == 0) return MOE355_OK;
  MOE355_CHECK(a8 && a_scale && w1 && w1_scale && w2 && w2_scale && sorted_ids && sorted_weights &&
                   sorted_expert_ids && num_valid && out && workspace && sstride_m >= 0 && sstride_kb >= 0,
               MOE355_EINVAL);
  MOE355_CHECK((int64_t)T * sstride_m * 4 < (1ll << 32), MOE355_EUNSUPPORTED);
  FusedWs L{};
  const int st = fused_ws_layout(T, H, I, E, topk, block_m, &L);
  if (st != MOE355_OK) return st;
  MOE355_CHECK(workspace_bytes >= L.total, MOE355_EINVAL);
  MOE355_CHECK(aligned16(a8) && aligned16(w1) && aligned16(w2) && aligned16(out) && aligned16(workspace) &&
                   ld_out % 8 == 0 && (reinterpret_cast<uintptr_t>(a_scale) & 3u) == 0 &&
                   aligned16(fc2_smooth_scale),
               MOE355_EMISALIGNED);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* h8 = ws + L.h8;
  float* hs = reinterpret_cast<float*>(ws + L.hs);
  FusedArgs f{};
  f.gu = g1u1_args(a8, a_scale, sstride_m, sstride_kb, w1, w1_scale, sorted_ids, sorted_expert_ids, num_valid, T, H, I,
                   topk, h8, hs, fc2_smooth_scale);
  f.dn = down_args(h8, hs, w2, w2_scale, sorted_ids, sorted_weights, sorted_expert_ids, num_valid, T, H, I, topk,
                   reinterpret_cast<float*>(ws + L.y));
  f.nt_gu = I / 128;
  f.nt_dn = H / 256;
  f.out = out;
  f.ld_out = ld_out;
  return launch_fused(f, block_m, stream);
}

#ifdef MOE355_PHASE_TRACE
extern "C" int moe355_phase_trace_read(uint32_t* host, size_t count) {
  MOE355_CHECK(host && count <= sizeof(g_phase_trace) / sizeof(uint32_t), MOE355_EINVAL);
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_phase_trace), count * sizeof(uint32_t), 0,
                             hipMemcpyDeviceToHost) == hipSuccess
             ? MOE355_OK
             : MOE355_ELAUNCH;
}
#endif
