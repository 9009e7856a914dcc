/*
 * libmoe355 -- FP8 block-scale Mixture-of-Experts layer for MI355X (gfx950).
 *
 * The operations follow "Accelerate DeepSeek-R1 Inference: Integrate AITER
 * into SGLang" (rocm.blogs.amd.com): section "Complete MoE Implementation"
 * (Top-K routing, MoE Sorting, Blockscale FP8 MoE Computation) and section
 * "General Linear Layer" (FP8 block-scale GEMM).  FP8 is OCP E4M3
 * (e4m3fn: bias 7, no infinities, largest finite 448).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every pointer argument is a caller-owned DEVICE pointer unless noted.
 *    The library never allocates device memory and keeps no state between
 *    calls; workspace is passed in by the caller, sized by the *_sizes /
 *    *_workspace queries (which are host-only and touch no GPU).
 *  - Every compute call is asynchronous and ordered on `stream`
 *    (0 = the default stream).  No call synchronises the host.
 *  - bf16 tensors are passed as their uint16_t bit patterns, e4m3 tensors as
 *    uint8_t codes.  Scales are fp32 dequantisation multipliers:
 *    value = decode(code) * scale.
 *  - Strides (ld_*, sstride_*) are in elements.
 *  - Return value: MOE355_OK (0) or a negative status (below).  When an
 *    argument check fails nothing is launched and no memory is touched.
 *    A launch failure reported by the runtime returns MOE355_ELAUNCH.
 *  - A call with zero tokens / rows is a successful no-op.
 */
#ifndef MOE355_H
#define MOE355_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE355_OK 0
#define MOE355_EINVAL (-1)       /* null pointer, negative size, ld < width, workspace too small */
#define MOE355_EUNSUPPORTED (-2) /* shape or option outside what the kernels implement */
#define MOE355_EMISALIGNED (-3)  /* a base pointer or row stride breaks the call's alignment rule */
#define MOE355_ELAUNCH (-4)      /* the HIP runtime reported an error at launch */
#define MOE355_ESCRATCH (-5)     /* the call needs more than the library's static device scratch */

/* Human-readable text of a status code (static storage; never NULL). */
const char* moe355_strerror(int status);

/*
 * Biased grouped top-k routing ("Complete MoE Implementation" / "Top-K
 * routing": tokens choose a fixed number of expert groups, then their top-k
 * experts inside those groups; a correction bias steers the choice; optional
 * renormalisation; the routed scaling factor multiplies the weights).
 *
 * Per token t (fl32 = round to fp32, nearest-even):
 *   s_e  = fl32(1/(1+exp(-logits[t,e])))  (evaluated in binary64)
 *   b_e  = fl32(s_e + bias[e])
 *   group g = experts [g*E/n_group, (g+1)*E/n_group); score = fl32(top1 + top2 of b)
 *   keep the topk_group best groups (score desc, group index asc)
 *   topk_ids[t, 0..topk)  = best experts of the kept groups by (b desc, id asc), in that order
 *   topk_weights[t, j]    = s of that expert; if renorm: divided by the fp32
 *                           left-to-right sum of the row; then * routed_scaling_factor.
 *
 * logits        [T, E] router logits, row stride ld_logits >= E (elements): fp32, or
 *               bf16 bits when logits_bf16 is 1 (each widened exactly to fp32 first).
 * bias          fp32 [E] (the correction bias).
 * topk_weights  fp32 [T, topk] out, row stride ld_topk >= topk.
 * topk_ids      int32 [T, topk] out, same row stride ld_topk.
 * Supported: 1 <= E <= 1024, E % n_group == 0, E/n_group >= 2, n_group <= 64,
 *            1 <= topk_group <= n_group, 1 <= topk <= min(32, topk_group*E/n_group).
 */
int grouped_topk(const void* logits, int logits_bf16, int64_t ld_logits, const float* bias,
                 int T, int E, int n_group, int topk_group, int topk,
                 int renorm, float routed_scaling_factor,
                 float* topk_weights, int32_t* topk_ids, int64_t ld_topk,
                 hipStream_t stream);

/*
 * Host-only size query for moe_sort (no GPU access).
 *   max_sorted      = capacity of sorted_ids / sorted_weights: T*topk + E*(block_m-1),
 *                     rounded up to block_m;
 *   max_blocks      = max_sorted / block_m = capacity of sorted_expert_ids;
 *   workspace_bytes = device scratch moe_sort needs.
 * Any output pointer may be NULL.  block_m must be 16, 32, 64, 128 or 256.
 */
int moe_sort_sizes(int T, int topk, int E, int block_m,
                   int64_t* max_sorted, int64_t* max_blocks, size_t* workspace_bytes);

/*
 * Host-only tile choice for moe_sort and the grouped GEMMs (no GPU access): the
 * block_m whose whole DeepSeek-V3 layer measured fastest at this size, looked up by
 * the mean pairs per expert p = T*topk/E in a table compiled into the library
 * (generated from a committed sweep; for that sweep: p <= 2 -> 16, p <= 4 -> 32,
 * p <= 16 -> 64, else 128).  Routing that concentrates pairs on few experts favours a
 * larger block_m than this.
 */
int moe_block_m(int T, int topk, int E, int* block_m);

/*
 * MoE align/sort ("Complete MoE Implementation" / "MoE Sorting": token-expert
 * pairs bucketed per expert for the grouped GEMM).  Pairs are flattened as
 * p = t*topk + j.  For experts in ascending order, expert e's pairs occupy a
 * segment of sorted_ids in ascending p, padded with the sentinel T*topk (weight
 * 0.0f) up to a multiple of block_m; experts without pairs get no segment.
 *   sorted_ids        int32 [max_sorted] out: flat pair index or sentinel
 *   sorted_weights    fp32  [max_sorted] out: topk_weights of the pair, 0 for padding
 *   sorted_expert_ids int32 [max_blocks] out: expert of each block_m-row block
 *   num_valid         int32 [1] out: padded total P (entries at or beyond P are
 *                     left untouched); -1 if an id lies outside [0, E)
 * topk_ids / topk_weights: [T, topk] with row stride ld_topk.
 * workspace: device memory of at least workspace_bytes (moe_sort_sizes); its
 * contents need no initialisation and are scratch after the call.
 * block_m must equal the block_m later passed to the grouped GEMMs.
 */
int moe_sort(const int32_t* topk_ids, const float* topk_weights, int64_t ld_topk,
             int T, int topk, int E, int block_m,
             int32_t* sorted_ids, float* sorted_weights, int32_t* sorted_expert_ids,
             int32_t* num_valid, void* workspace, size_t workspace_bytes,
             hipStream_t stream);

/*
 * Dynamic 1x128 FP8 quantisation ("General Linear Layer": one scale per 1x128
 * of an activation row; "Blockscale FP8 MoE Computation": the bf16 hidden
 * states are quantised per 128 before the grouped GEMM).  Per row m and
 * group kb (columns [128*kb, min(K, 128*kb+128)); the last group of a row holds
 * the remaining K % 128 values when K is not a multiple of 128):
 *   amax  = max |x|;  scale = (amax == 0) ? 1 : fl32(amax / 448)
 *   q     = e4m3(fl32(x / scale))  nearest-even, saturating at +-448, sign kept
 * x      bf16 bits [M, K], row stride ld_x >= K.
 * q      e4m3 [M, K] out, row stride ld_q >= K.
 * scale  fp32 out, element (m, kb) at scale[m*sstride_m + kb*sstride_kb]:
 *        row-major [M, KB] is (KB, 1); K-block-major [KB, M] is (1, M); KB = ceil(K/128).
 * K % 8 == 0 (else MOE355_EUNSUPPORTED).  x and q 16-byte aligned, x's row stride a
 * multiple of 16 bytes and q's of 8 (each lane stores 8 codes), else MOE355_EMISALIGNED.
 */
int fp8_quant_1x128(const uint16_t* x, int64_t ld_x, int M, int K,
                    uint8_t* q, int64_t ld_q,
                    float* scale, int64_t sstride_m, int64_t sstride_kb,
                    hipStream_t stream);

/*
 * Gate/up grouped GEMM with SiLU(gate)*up ("Blockscale FP8 MoE Computation":
 * grouped GEMM over the sorted pairs with fused gate/up weights, g1u1).
 * For every valid row r of the sorted buffer (r < num_valid, sorted_ids[r] < T*topk),
 * token t = sorted_ids[r] / topk, expert e = sorted_expert_ids[r / block_m]:
 *   acc[n] = sum_kb a_scale(t,kb) * w1_scale[e, n/128, kb] * sum_{k in kb} a8[t,k] * w1[e,n,k]
 *   h[i]   = SiLU(acc[i]) * acc[I+i],  i < I            (fp32)
 *   h[i]   = fl32(h[i] * fc2_smooth_scale[e, i])         (only when fc2_smooth_scale is given)
 *   h8[r, :], h_scale[r, :] = 1x128 quantisation of h (same rule as fp8_quant_1x128)
 * a8        e4m3 [T, H] (row stride H); a_scale(t,kb) = a_scale[t*sstride_m + kb*sstride_kb].
 * w1        e4m3 [E, 2I, H]: rows [0, I) gate, [I, 2I) up;  w1_scale fp32 [E, 2I/128, H/128].
 * sorted_*  / num_valid as written by moe_sort with the same block_m; max_sorted
 *           is the capacity returned by moe_sort_sizes.
 * h8        e4m3 [max_sorted, I] out; h_scale fp32 [max_sorted, I/128] out.
 * fc2_smooth_scale  fp32 [E, I] (16-byte aligned) or NULL: per-expert channel factors
 *           applied to h before its quantisation (the pages pass an optional
 *           fc2_smooth_scale to the fused MoE call without defining it; this is the
 *           smoothing reading: the down projection's input is scaled per channel and the
 *           caller folds the inverse factors into w2).
 *           Padding rows and rows at or beyond num_valid are not written (nothing
 *           is written when num_valid is -1).
 * H % 128 == 0, I % 128 == 0, block_m in {16, 32, 64, 128, 256}; a8, w1, h8 16-byte aligned.
 * T * sstride_m * 4 < 2^32 (the scale reads take 32-bit byte offsets), else MOE355_EUNSUPPORTED.
 */
int moe_fp8_blockscale_g1u1(const uint8_t* a8, const float* a_scale,
                            int64_t sstride_m, int64_t sstride_kb,
                            const uint8_t* w1, const float* w1_scale,
                            const int32_t* sorted_ids, const int32_t* sorted_expert_ids,
                            const int32_t* num_valid,
                            int T, int H, int I, int E, int topk, int block_m, int64_t max_sorted,
                            uint8_t* h8, float* h_scale, const float* fc2_smooth_scale,
                            hipStream_t stream);

/* Host-only workspace query for moe_down_combine (no GPU access). */
int moe_down_combine_workspace(int T, int H, int topk, size_t* bytes);

/*
 * Down-projection grouped GEMM and top-k-weighted combine ("Blockscale FP8
 * MoE Computation": the second expert GEMM and the weighted sum of each
 * token's expert outputs into the [tokens, model_dim] output).
 *   y[r, n]  = sum_kb h_scale[r,kb] * w2_scale[e, n/128, kb] * sum_{k in kb} h8[r,k] * w2[e,n,k]
 *   out[t,n] = bf16(sum over j ascending of sorted_weights[r(t,j)] * y[r(t,j), n])
 * where r(t,j) is the sorted row holding pair t*topk+j (fp32 sums, bf16 nearest-even).
 * h8 / h_scale  as written by moe_fp8_blockscale_g1u1 ([max_sorted, I], [max_sorted, I/128]).
 * w2        e4m3 [E, H, I]; w2_scale fp32 [E, H/128, I/128].
 * out       bf16 bits [T, H] out, row stride ld_out >= H (16-byte aligned rows).
 * workspace device memory of at least moe_down_combine_workspace() bytes.
 * Every pair of the T*topk must appear in the sorted buffer (moe_sort guarantees it
 * for valid ids); when num_valid is -1 (an id outside [0, E)) out is not written.
 */
int moe_down_combine(const uint8_t* h8, const float* h_scale,
                     const uint8_t* w2, const float* w2_scale,
                     const int32_t* sorted_ids, const float* sorted_weights,
                     const int32_t* sorted_expert_ids, const int32_t* num_valid,
                     int T, int H, int I, int E, int topk, int block_m, int64_t max_sorted,
                     uint16_t* out, int64_t ld_out, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* Host-only workspace query for moe_fp8_blockscale_fused (no GPU access): bytes for the
 * intermediate h8 [max_sorted, I], its scales [max_sorted, I/128] and the per-pair
 * fp32 staging [T*topk, H] (max_sorted from moe_sort_sizes for this block_m). */
int moe_fp8_blockscale_fused_workspace(int T, int H, int I, int E, int topk, int block_m, size_t* bytes);

/*
 * The whole expert computation in one launch ("Blockscale FP8 MoE Computation": the
 * pages' fused call takes the sorted buffers to the [tokens, model_dim] output in one
 * kernel): moe_fp8_blockscale_g1u1 followed by moe_down_combine, run by one cooperative
 * launch of persistent workgroups with a grid-wide barrier between the gate/up tiles,
 * the down tiles and the combine.  Arguments are those two calls' (same meaning, same
 * layouts and rules); h8 / h_scale and the per-pair staging live in `workspace`
 * (moe_fp8_blockscale_fused_workspace bytes; contents need no initialisation).  Each
 * tile runs the same arithmetic as the two calls, so `out` equals theirs bit for bit.
 * block_m in {16, 32, 64, 128} (MOE355_EUNSUPPORTED for 256, or on a device without
 * cooperative launch).
 */
int moe_fp8_blockscale_fused(const uint8_t* a8, const float* a_scale,
                             int64_t sstride_m, int64_t sstride_kb,
                             const uint8_t* w1, const float* w1_scale,
                             const uint8_t* w2, const float* w2_scale,
                             const int32_t* sorted_ids, const float* sorted_weights,
                             const int32_t* sorted_expert_ids, const int32_t* num_valid,
                             int T, int H, int I, int E, int topk, int block_m, int64_t max_sorted,
                             const float* fc2_smooth_scale, uint16_t* out, int64_t ld_out,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Host-only workspace query for gemm_fp8_blockscale (no GPU access): the bytes of
 * fp32 partial sums its split-K path uses for this shape (0 when it does not split). */
int gemm_fp8_blockscale_workspace(int M, int N, int K, size_t* bytes);

/*
 * Dense FP8 block-scale GEMM ("General Linear Layer": Y = (XQ, 1x128 scales)
 * times (WQ, 128x128 scales)^T with WQ stored [N, K]):
 *   c[m,n] = bf16( sum_kb a_scale(m,kb) * b_scale[n/128, kb] * sum_{k in kb} a8[m,k] * b8[n,k] )
 * a8       e4m3 [M, K] (row stride K); a_scale(m,kb) = a_scale[m*sstride_m + kb*sstride_kb].
 * b8       e4m3 [N, K] (row stride K); b_scale fp32 [ceil(N/128), ceil(K/128)].
 *          K and N need not be multiples of 128 (the section sizes its scale arrays
 *          with ceil): K block kb covers k in [128*kb, min(K, 128*kb+128)) and
 *          b_scale row n/128 serves the last, shorter column block.
 * c        [M, N] out, row stride ldc >= N (16-byte aligned rows): bf16 bits, or fp16
 *          bits when out_fp16 is 1 (the pages' linear layer offers both output types);
 *          round to nearest even either way.
 * workspace device memory of gemm_fp8_blockscale_workspace() bytes, or NULL / 0: small M
 *          then splits K over more workgroups, keeps fp32 partial sums there and adds them
 *          in a fixed order (deterministic); without it one workgroup per output
 *          tile walks all of K.  The tiling (and so the workspace size) comes from a
 *          table of measured plans for the DeepSeek-V3 linear-layer shapes compiled into
 *          the library, else from a rule on M, N and K.  Contents need no initialisation.  K above 16384 (more
 *          than 128 K blocks) is always split and needs the workspace: without it
 *          MOE355_EUNSUPPORTED, with too little MOE355_EINVAL.
 * K % 16 == 0, N % 8 == 0 and M * sstride_m * 4 < 2^32 (else MOE355_EUNSUPPORTED);
 * a8, b8 16-byte aligned.
 */
int gemm_fp8_blockscale(const uint8_t* a8, const float* a_scale,
                        int64_t sstride_m, int64_t sstride_kb,
                        const uint8_t* b8, const float* b_scale,
                        int M, int N, int K, uint16_t* c, int64_t ldc, int out_fp16,
                        void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * gemm_fp8_blockscale with the tiling chosen by the caller ("General Linear Layer": the
 * pages pick the GEMM per DeepSeek-V3/R1 shape from a tuned table; this call is what a
 * sweep times to build one): output tiles of tile_m rows (16, 32, 64 or 128) by tile_n
 * columns (128 or 256), and K split into `splits` runs of whole 128-wide blocks whose
 * fp32 partial sums are added in a fixed order.  splits > 1 needs a workspace of
 * gemm_fp8_blockscale_tiled_workspace() bytes (MOE355_EINVAL without it); a run of more
 * than 128 K blocks is MOE355_EUNSUPPORTED.  tile_n 16 selects the small-M kernel: one
 * workgroup per 16 columns whose waves split K among themselves and add their fp32
 * partial tiles in LDS in a fixed order (M <= tile_m <= 64, splits 1, no workspace,
 * any K).  Arguments, results and other errors are those of gemm_fp8_blockscale (the
 * arithmetic per output element is the same block-scaled sum whatever the tiling; only
 * the order of the fp32 additions differs between K splits).
 */
int gemm_fp8_blockscale_tiled(const uint8_t* a8, const float* a_scale,
                              int64_t sstride_m, int64_t sstride_kb,
                              const uint8_t* b8, const float* b_scale,
                              int M, int N, int K, uint16_t* c, int64_t ldc, int out_fp16,
                              int tile_m, int tile_n, int splits,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);
/* Host-only: the workspace gemm_fp8_blockscale_tiled needs for this shape and split count. */
int gemm_fp8_blockscale_tiled_workspace(int M, int N, int K, int splits, size_t* bytes);

/* Host-only: the tiling gemm_fp8_blockscale runs for this shape (with its workspace):
 * measured 1 -> the plan the call uses (the compiled table of measured plans, else the
 * rule); measured 0 -> the rule alone (what a sweep compares the candidates against).
 * Arguments and errors as gemm_fp8_blockscale_workspace. */
int gemm_fp8_blockscale_plan(int M, int N, int K, int measured, int* tile_m, int* tile_n, int* splits);

/*
 * gemm_fp8_blockscale for callers that cannot allocate device memory (code under
 * HIP-graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments, results and errors as gemm_fp8_blockscale with its workspace,
 * but the split-K partial sums live in a static device array of the library
 * (MOE355_STATIC_SCRATCH_BYTES per GPU, held by every GPU the library runs on
 * until the process ends).  The call allocates nothing; a shape whose split-K
 * partials need more than that array (gemm_fp8_blockscale_workspace) returns
 * MOE355_ESCRATCH before anything is launched.  All calls on one GPU share its
 * array: calls that overlap in time on one GPU (other streams, other threads) race.
 * The first call on a GPU looks up the array's address there (it must be the
 * current device); a failure of that lookup returns MOE355_ELAUNCH.
 */
#define MOE355_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
int gemm_fp8_blockscale_noalloc(const uint8_t* a8, const float* a_scale,
                                int64_t sstride_m, int64_t sstride_kb,
                                const uint8_t* b8, const float* b_scale,
                                int M, int N, int K, uint16_t* c, int64_t ldc, int out_fp16,
                                hipStream_t stream);

/*
 * Pre-shuffled weights ("General Linear Layer": the linear path runs on weights
 * permuted once at load time into an MFMA-friendly order; the pages use such a
 * layout with their pre-shuffle GEMM).  The permutation is this library's own:
 * w [rows, K] e4m3 (rows and K multiples of 128) is written to out as 128-row x
 * 128-byte tiles; tile (t, kb) -- rows [128t, 128t+128), bytes [128kb, 128kb+128)
 * of each row -- starts at byte (t*K/128 + kb)*16384, and inside it row rr takes
 * bytes [rr*128, rr*128+128) with its 16-byte chunk c in slot c ^ (rr & 7).
 * An expert tensor [E, R, K] is passed as rows = E*R (R % 128 == 0).  Scales are
 * not permuted.  out must not overlap w (else MOE355_EINVAL); rows or K not a
 * multiple of 128 give MOE355_EUNSUPPORTED; w, out 16-byte aligned.
 */
int shuffle_weight_128x128(const uint8_t* w, int64_t rows, int K, uint8_t* out,
                           hipStream_t stream);

/*
 * The three GEMM calls on weights in the shuffle_weight_128x128 layout: the same
 * arguments, results and error behaviour as gemm_fp8_blockscale (b8 = shuffled
 * [N, K]; N and K multiples of 128, else MOE355_EUNSUPPORTED),
 * moe_fp8_blockscale_g1u1 (w1 = shuffled [E*2I, H]) and moe_down_combine
 * (w2 = shuffled [E*H, I]).  The arithmetic and its order are unchanged, so the
 * outputs equal those of the unshuffled calls bit for bit.
 */
int gemm_fp8_blockscale_wpreshuffle(const uint8_t* a8, const float* a_scale,
                                    int64_t sstride_m, int64_t sstride_kb,
                                    const uint8_t* b8, const float* b_scale,
                                    int M, int N, int K, uint16_t* c, int64_t ldc, int out_fp16,
                                    void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);
int moe_fp8_blockscale_g1u1_wpreshuffle(const uint8_t* a8, const float* a_scale,
                                        int64_t sstride_m, int64_t sstride_kb,
                                        const uint8_t* w1, const float* w1_scale,
                                        const int32_t* sorted_ids, const int32_t* sorted_expert_ids,
                                        const int32_t* num_valid,
                                        int T, int H, int I, int E, int topk, int block_m,
                                        int64_t max_sorted, uint8_t* h8, float* h_scale,
                                        const float* fc2_smooth_scale, hipStream_t stream);
int moe_down_combine_wpreshuffle(const uint8_t* h8, const float* h_scale,
                                 const uint8_t* w2, const float* w2_scale,
                                 const int32_t* sorted_ids, const float* sorted_weights,
                                 const int32_t* sorted_expert_ids, const int32_t* num_valid,
                                 int T, int H, int I, int E, int topk, int block_m, int64_t max_sorted,
                                 uint16_t* out, int64_t ld_out, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE355_H */
