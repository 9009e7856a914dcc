// MoE align/sort ("Accelerate DeepSeek-R1 Inference: Integrate AITER into
// SGLang", section "Complete MoE Implementation" / "MoE Sorting").
//
// Up to 16384 pairs: one workgroup does everything (see sort_small_kernel).
// Beyond that, three launches on the caller's stream, no host synchronisation:
//   count   one workgroup per chunk of 256 flat pairs: per-expert histogram in LDS
//   scan    one workgroup: per-expert prefix over chunks, padded segment offsets
//           (exclusive scan over experts), padding sentinels, block -> expert map
//   scatter one workgroup per chunk: stable rank of each pair among the pairs of
//           its expert (ballots over the expert-id bits inside a wave, per-wave
//           counts in LDS across waves, chunk prefix across chunks)
// The result is the unique stable order: experts ascending, pairs ascending.
#include "device_common.h"
#include "host_common.h"
#include "block_m_tuned.h"

namespace moe355 {
namespace {

constexpr int kChunk = 256;
constexpr int kMaxE = 1024;
constexpr int kScanThreads = 1024;

struct SortWs {
  int32_t* counts;   // [nchunks][E]  chunk histogram, then its exclusive prefix per expert
  int32_t* invalid;  // [nchunks]     ids outside [0, E) seen by the chunk
  int32_t* offs;     // [E]           segment start of each expert
};

inline int64_t nchunks_of(int T, int topk) { return ceil_div64((int64_t)T * topk, kChunk); }

inline size_t ws_bytes(int T, int topk, int E) {
  const int64_t nc = nchunks_of(T, topk);
  return (size_t)((nc * E + nc + E) * 4 + 256);
}

inline SortWs ws_layout(void* ws, int T, int topk, int E) {
  const int64_t nc = nchunks_of(T, topk);
  int32_t* p = static_cast<int32_t*>(ws);
  return SortWs{p, p + nc * E, p + nc * E + nc};
}

__global__ __launch_bounds__(kChunk) void sort_count_kernel(const int32_t* __restrict__ ids, int64_t ld, int T, int k,
                                                            int E, SortWs ws) {
  __shared__ int hist[kMaxE];
  __shared__ int bad;
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kChunk) hist[e] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  const int64_t p = (int64_t)blockIdx.x * kChunk + tid;
  if (p < (int64_t)T * k) {
    const int64_t t = p / k;
    const int j = (int)(p - t * k);
    const int e = ids[t * ld + j];
    if (e >= 0 && e < E)
      atomicAdd(&hist[e], 1);
    else
      atomicAdd(&bad, 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kChunk) ws.counts[(int64_t)blockIdx.x * E + e] = hist[e];
  if (tid == 0) ws.invalid[blockIdx.x] = bad;
}

// exclusive block scan of one int per thread (1024 threads = 16 waves)
__device__ int block_exclusive_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  int inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int n = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += n;
  }
  if (lane == kWave - 1) wave_tot[w] = inc;
  __syncthreads();
  if (w == 0) {
    int x = lane < kScanThreads / kWave ? wave_tot[lane] : 0;
    int xi = x;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int n = __shfl_up(xi, o, kWave);
      if (lane >= o) xi += n;
    }
    if (lane < kScanThreads / kWave) wave_tot[lane] = xi - x;  // exclusive wave base
    if (lane == kScanThreads / kWave - 1) wave_tot[kScanThreads / kWave] = xi;
  }
  __syncthreads();
  total = wave_tot[kScanThreads / kWave];
  return wave_tot[w] + inc - v;
}

__global__ __launch_bounds__(kScanThreads) void sort_scan_kernel(SortWs ws, int nchunks, int T, int k, int E, int BM,
                                                                 int32_t* __restrict__ sorted_ids,
                                                                 float* __restrict__ sorted_w,
                                                                 int32_t* __restrict__ sorted_eids,
                                                                 int32_t* __restrict__ num_valid) {
  __shared__ int wave_tot[kScanThreads / kWave + 1];
  __shared__ int bad;
  const int e = threadIdx.x;
  if (e == 0) bad = 0;
  __syncthreads();
  // per-chunk counts -> exclusive per-chunk offsets of expert e; loads issued in
  // batches so that their latencies overlap
  constexpr int kBatch = 16;
  int c = 0;
  if (e < E) {
    for (int ch0 = 0; ch0 < nchunks; ch0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) v[i] = ch0 + i < nchunks ? ws.counts[(int64_t)(ch0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (ch0 + i < nchunks) ws.counts[(int64_t)(ch0 + i) * E + e] = c;
        c += v[i];
      }
    }
  }
  for (int ch = e; ch < nchunks; ch += kScanThreads)
    if (ws.invalid[ch]) atomicAdd(&bad, 1);
  const int padded = (c + BM - 1) / BM * BM;
  int total = 0;
  const int off = block_exclusive_scan(padded, wave_tot, total);
  if (e < E) {
    ws.offs[e] = off;
    const int sentinel = T * k;
    for (int i = c; i < padded; ++i) {
      sorted_ids[off + i] = sentinel;
      sorted_w[off + i] = 0.0f;
    }
    for (int b = off / BM; b < (off + padded) / BM; ++b) sorted_eids[b] = e;
  }
  if (e == 0) num_valid[0] = bad ? -1 : total;
}

__global__ __launch_bounds__(kChunk) void sort_scatter_kernel(const int32_t* __restrict__ ids,
                                                              const float* __restrict__ weights, int64_t ld, int T,
                                                              int k, int E, int nbits, SortWs ws,
                                                              int32_t* __restrict__ sorted_ids,
                                                              float* __restrict__ sorted_w) {
  constexpr int kWaves = kChunk / kWave;
  __shared__ int wcnt[kWaves][kMaxE];
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  for (int i = tid; i < kWaves * E; i += kChunk) wcnt[i / E][i % E] = 0;
  const int64_t p = (int64_t)blockIdx.x * kChunk + tid;
  int e = -1;
  float wt = 0.0f;
  if (p < (int64_t)T * k) {
    const int64_t t = p / k;
    const int j = (int)(p - t * k);
    e = ids[t * ld + j];
    wt = weights[t * ld + j];
    if (e < 0 || e >= E) e = -1;
  }
  // lanes of this wave holding the same expert
  uint64_t peers = __ballot(e >= 0);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool on = e >= 0 && ((e >> bit) & 1);
    const uint64_t bal = __ballot(on);
    peers &= on ? bal : ~bal;
  }
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int rank_w = __popcll(peers & lt);
  __syncthreads();
  if (e >= 0 && rank_w == 0) wcnt[w][e] = __popcll(peers);
  __syncthreads();
  if (e >= 0) {
    int before = 0;
    for (int ww = 0; ww < w; ++ww) before += wcnt[ww][e];
    const int pos = ws.offs[e] + ws.counts[(int64_t)blockIdx.x * E + e] + before + rank_w;
    sorted_ids[pos] = (int32_t)p;
    sorted_w[pos] = wt;
  }
}

// Small inputs (at most kSmallMaxPairs pairs, e.g. decode): the whole sort in one
// 1024-thread workgroup -- histogram, padded scan, then the pairs in chunks of
// 1024 in flat order, each ranked stably (ballots inside a wave, per-wave counts
// across waves) on top of a running per-expert position.
constexpr int kSmallMaxPairs = 16384;
constexpr int kSmallWaves = kScanThreads / kWave;

__global__ __launch_bounds__(kScanThreads) void sort_small_kernel(const int32_t* __restrict__ ids,
                                                                  const float* __restrict__ weights, int64_t ld,
                                                                  int T, int k, int E, int BM, int nbits,
                                                                  int32_t* __restrict__ sorted_ids,
                                                                  float* __restrict__ sorted_w,
                                                                  int32_t* __restrict__ sorted_eids,
                                                                  int32_t* __restrict__ num_valid) {
  __shared__ int pos[kMaxE];                  // counts, then the next free slot of each expert
  __shared__ int wcnt[kSmallWaves][kMaxE];    // per-wave counts of one chunk (kept all-zero between uses)
  __shared__ int wave_tot[kSmallWaves + 1];
  __shared__ int bad;
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  const int np = T * k;
  for (int e = tid; e < E; e += kScanThreads) pos[e] = 0;
  for (int i = tid; i < kSmallWaves * E; i += kScanThreads) wcnt[i / E][i % E] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int p = tid; p < np; p += kScanThreads) {
    const int e = ids[(int64_t)(p / k) * ld + p % k];
    if (e >= 0 && e < E)
      atomicAdd(&pos[e], 1);
    else
      atomicAdd(&bad, 1);
  }
  __syncthreads();
  const int c = tid < E ? pos[tid] : 0;
  const int padded = (c + BM - 1) / BM * BM;
  int total = 0;
  const int off = block_exclusive_scan(padded, wave_tot, total);
  if (tid < E) {
    const int sentinel = T * k;
    for (int i = c; i < padded; ++i) {
      sorted_ids[off + i] = sentinel;
      sorted_w[off + i] = 0.0f;
    }
    for (int b = off / BM; b < (off + padded) / BM; ++b) sorted_eids[b] = tid;
    pos[tid] = off;
  }
  if (tid == 0) num_valid[0] = bad ? -1 : total;
  __syncthreads();
  for (int base = 0; base < np; base += kScanThreads) {
    const int p = base + tid;
    int e = -1;
    float wt = 0.0f;
    if (p < np) {
      e = ids[(int64_t)(p / k) * ld + p % k];
      wt = weights[(int64_t)(p / k) * ld + p % k];
      if (e < 0 || e >= E) e = -1;
    }
    uint64_t peers = __ballot(e >= 0);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = e >= 0 && ((e >> bit) & 1);
      const uint64_t bal = __ballot(on);
      peers &= on ? bal : ~bal;
    }
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    const int rank_w = __popcll(peers & lt);
    const bool leader = e >= 0 && rank_w == 0;
    if (leader) wcnt[w][e] = __popcll(peers);
    __syncthreads();
    if (e >= 0) {
      int before = 0;
      for (int ww = 0; ww < w; ++ww) before += wcnt[ww][e];
      const int at = pos[e] + before + rank_w;
      sorted_ids[at] = p;
      sorted_w[at] = wt;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&pos[e], __popcll(peers));
      wcnt[w][e] = 0;
    }
    __syncthreads();
  }
}

}  // namespace
}  // namespace moe355

using namespace moe355;

extern "C" int moe_sort_sizes(int T, int topk, int E, int block_m, int64_t* max_sorted, int64_t* max_blocks,
                              size_t* workspace_bytes) {
  MOE355_CHECK(T >= 0 && topk > 0 && E > 0, MOE355_EINVAL);
  MOE355_CHECK(valid_block_m(block_m) && E <= kMaxE && topk <= 32, MOE355_EUNSUPPORTED);
  MOE355_CHECK((int64_t)T * topk + (int64_t)E * block_m < (1ll << 30), MOE355_EUNSUPPORTED);
  const int64_t ms = ceil_div64((int64_t)T * topk + (int64_t)E * (block_m - 1), block_m) * block_m;
  if (max_sorted) *max_sorted = ms;
  if (max_blocks) *max_blocks = ms / block_m;
  if (workspace_bytes) *workspace_bytes = ws_bytes(T, topk, E);
  return MOE355_OK;
}

// M tile of the grouped GEMMs by the expected pairs per expert, T*topk/E (uniform
// routing), from a sweep of the whole layer on MI355X with V3 shapes: weight
// streaming wants the smallest tile while experts hold a few rows, the 128-row
// 8-wave tile wins once an expert holds a few dozen.
extern "C" int moe_block_m(int T, int topk, int E, int* block_m) {
  MOE355_CHECK(T >= 0 && topk > 0 && E > 0 && block_m, MOE355_EINVAL);
  const int64_t pairs = (int64_t)T * topk;
  // measured table (block_m_tuned.h) by mean pairs per expert, else the rule: 16-row tiles
  // while experts average under 4 pairs, 32 under 16, 128 above
  const int n = (int)(sizeof(kBlockMTuned) / sizeof(kBlockMTuned[0]));
  if (kBlockMTuned[0].block_m > 0) {
    const double ppe = (double)pairs / E;
    int bm = kBlockMTuned[n - 1].block_m;
    for (int i = n - 1; i >= 0; --i)
      if (ppe <= kBlockMTuned[i].ppe_max) bm = kBlockMTuned[i].block_m;
    *block_m = bm;
    return MOE355_OK;
  }
  *block_m = pairs < 4ll * E ? 16 : pairs < 16ll * E ? 32 : 128;
  return MOE355_OK;
}

extern "C" int moe_sort(const int32_t* topk_ids, const float* topk_weights, int64_t ld_topk, int T, int topk, int E,
                        int block_m, int32_t* sorted_ids, float* sorted_weights, int32_t* sorted_expert_ids,
                        int32_t* num_valid, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int64_t ms = 0, mb = 0;
  size_t need = 0;
  const int st = moe_sort_sizes(T, topk, E, block_m, &ms, &mb, &need);
  if (st != MOE355_OK) return st;
  MOE355_CHECK(ld_topk >= topk, MOE355_EINVAL);
  if (T == 0) return MOE355_OK;
  MOE355_CHECK(topk_ids && topk_weights && sorted_ids && sorted_weights && sorted_expert_ids && num_valid && workspace,
               MOE355_EINVAL);
  MOE355_CHECK(workspace_bytes >= need, MOE355_EINVAL);
  MOE355_CHECK((reinterpret_cast<uintptr_t>(workspace) & 3u) == 0, MOE355_EMISALIGNED);
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  if ((int64_t)T * topk <= kSmallMaxPairs) {
    hipLaunchKernelGGL(sort_small_kernel, dim3(1), dim3(kScanThreads), 0, stream, topk_ids, topk_weights, ld_topk, T,
                       topk, E, block_m, nbits, sorted_ids, sorted_weights, sorted_expert_ids, num_valid);
    return launch_status();
  }
  const int nc = (int)nchunks_of(T, topk);
  const SortWs ws = ws_layout(workspace, T, topk, E);
  hipLaunchKernelGGL(sort_count_kernel, dim3(nc), dim3(kChunk), 0, stream, topk_ids, ld_topk, T, topk, E, ws);
  hipLaunchKernelGGL(sort_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, ws, nc, T, topk, E, block_m, sorted_ids,
                     sorted_weights, sorted_expert_ids, num_valid);
  hipLaunchKernelGGL(sort_scatter_kernel, dim3(nc), dim3(kChunk), 0, stream, topk_ids, topk_weights, ld_topk, T, topk,
                     E, nbits, ws, sorted_ids, sorted_weights);
  return launch_status();
}
