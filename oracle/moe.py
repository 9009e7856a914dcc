"""FP8 block-scale MoE expert computation (CPU oracle; test infrastructure only).

"Accelerate DeepSeek-R1 Inference: Integrate AITER into SGLang", section
"Complete MoE Implementation" / "Blockscale FP8 MoE Computation": a grouped
GEMM over the sorted token-expert pairs with fused gate/up weights (g1u1:
w1 has twice the rows of w2's inner dimension), SiLU(gate) * up, a down
projection, and the combine of each token's top-k expert outputs weighted
by sorted_weight_buf into the [tokens, model_dim] output.

Layouts: w1 [E, 2I, H] (rows [0, I) gate, [I, 2I) up), w1_scale
[E, 2I/128, H/128]; w2 [E, H, I], w2_scale [E, H/128, I/128]; a8 [T, H] with
a_scale [T, H/128].

Readings taken where the page hides the step inside its fused kernel:
  * the intermediate h = fl32(SiLU(g) * u), SiLU(g) = g / (1 + exp(-g)) in
    binary64, is requantised with the same dynamic 1x128 rule as the
    activations before the down projection (both products on FP8);
  * the routing weight multiplies each pair's down-projection output, and a
    token's k weighted outputs are summed in ascending j, in binary64;
  * the optional fc2_smooth_scale (passed to the fused call, never defined on
    the page) is read as per-expert channel factors [E, I] on h before its
    requantisation: h_i = fl32(h_i * s[e, i]), an fp32 product.
"""
import numpy as np

from . import gemm, pool, quant

# rows of one expert handed to a worker at a time (rows are independent)
ROW_CHUNK = 512


def silu_mul_f32(g, u):
    """fl32(SiLU(g) * u) with the products in binary64."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    with np.errstate(over="ignore"):
        return (g / (1.0 + np.exp(-g)) * u).astype(np.float32)


def smooth_f32(h, smooth_e):
    """fl32(h_i * s_i) per channel (fp32 operands; the product is exact in binary64)."""
    if smooth_e is None:
        return h
    prod = np.asarray(h, np.float32).astype(np.float64) * np.asarray(smooth_e, np.float32).astype(np.float64)
    return prod.astype(np.float32)


def expert_ffn_h(a8_rows, a_scale_rows, w1_e, w1_scale_e, smooth_e=None):
    """Gate/up GEMM for rows of one expert -> (h float32 [R, I], acc float64 [R, 2I])."""
    acc = gemm.gemm_blockscale(a8_rows, a_scale_rows, w1_e, w1_scale_e)
    I = acc.shape[1] // 2
    return smooth_f32(silu_mul_f32(acc[:, :I], acc[:, I:]), smooth_e), acc


def g1u1(a8, a_scale, w1, w1_scale, sorted_ids, sorted_expert_ids, num_valid, topk, block_m,
         fc2_smooth_scale=None, workers=1):
    """Gate/up stage over the sorted buffer.

    Returns (h8 uint8 [P, I], h_scale float32 [P, I/128], h float32 [P, I], valid bool [P]);
    rows holding the sentinel are left zero and marked invalid.  workers > 1 evaluates
    the blocks on a thread pool (same result: every block writes its own rows).
    """
    T = a8.shape[0]
    E, twoI, H = w1.shape
    I = twoI // 2
    P = int(num_valid)
    h = np.zeros((P, I), dtype=np.float32)
    valid = np.asarray(sorted_ids[:P]) < T * topk

    def block(blk):
        rows = np.arange(blk * block_m, (blk + 1) * block_m)
        rows = rows[valid[rows]]
        if len(rows) == 0:
            return
        e = int(sorted_expert_ids[blk])
        tok = np.asarray(sorted_ids)[rows] // topk
        h[rows], _ = expert_ffn_h(a8[tok], a_scale[tok], w1[e], w1_scale[e],
                                  None if fc2_smooth_scale is None else fc2_smooth_scale[e])

    pool.run([lambda b=b: block(b) for b in range(P // block_m)], workers)
    h8, hs = quant.quant_1x128(h)
    h8[~valid] = 0
    hs[~valid] = 0
    return h8, hs, h, valid


def down_combine(h8, h_scale, w2, w2_scale, sorted_ids, sorted_weights, sorted_expert_ids,
                 num_valid, T, topk, block_m, workers=1):
    """Down projection + weighted combine -> ref float64 [T, H] (before the bf16 store).

    workers > 1 evaluates the blocks on a thread pool (same result: every block
    writes the rows of its own pairs; the combine runs afterwards in ascending j)."""
    E, H, I = w2.shape
    P = int(num_valid)
    sid = np.asarray(sorted_ids)
    y = np.zeros((T * topk, H), dtype=np.float64)       # per pair, weight applied

    def block(blk):
        rows = np.arange(blk * block_m, (blk + 1) * block_m)
        rows = rows[sid[rows] < T * topk]
        if len(rows) == 0:
            return
        e = int(sorted_expert_ids[blk])
        yy = gemm.gemm_blockscale(h8[rows], h_scale[rows], w2[e], w2_scale[e])
        y[sid[rows]] = np.asarray(sorted_weights, dtype=np.float64)[rows, None] * yy

    pool.run([lambda b=b: block(b) for b in range(P // block_m)], workers)
    out = np.zeros((T, H), dtype=np.float64)
    y = y.reshape(T, topk, H)
    for j in range(topk):
        out += y[:, j, :]
    return out


def layer_tokens(a8, a_scale, w1, w1_scale, w2, w2_scale, topk_ids, topk_weights, fc2_smooth_scale=None,
                 workers=1):
    """Token-major evaluation of the expert part of the layer for a set of token rows.

    a8 [R, H], a_scale [R, H/128], topk_ids / topk_weights [R, k] are the rows of
    the tokens to evaluate.  No sort buffer is used: slot j of row i applies
    expert topk_ids[i, j] to row i.  Each expert is evaluated once on all rows
    routed to it (rows are independent, so this equals one row at a time).
    Returns (ref float64 [R, H], h float32 [R, k, I], h8 uint8 [R, k, I],
    h_scale float32 [R, k, I/128]); ref sums the k weighted outputs in
    ascending j.  workers > 1 evaluates (expert, up to ROW_CHUNK of its rows) pieces
    on a thread pool; the pieces write disjoint rows, so the result is the same.
    """
    R, k = topk_ids.shape
    E, H, I = w2.shape
    y = np.zeros((R, k, H), dtype=np.float64)
    hh = np.zeros((R, k, I), dtype=np.float32)
    h8s = np.zeros((R, k, I), dtype=np.uint8)
    hss = np.zeros((R, k, I // 128), dtype=np.float32)

    def piece(e, ii, jj):
        h, _ = expert_ffn_h(a8[ii], a_scale[ii], w1[e], w1_scale[e],
                            None if fc2_smooth_scale is None else fc2_smooth_scale[e])
        h8, hs = quant.quant_1x128(h)
        y[ii, jj] = gemm.gemm_blockscale(h8, hs, w2[e], w2_scale[e])
        hh[ii, jj], h8s[ii, jj], hss[ii, jj] = h, h8, hs

    tasks = []
    for e in np.unique(topk_ids):
        ii, jj = np.nonzero(topk_ids == e)
        for s0, s1 in pool.row_chunks(len(ii), ROW_CHUNK if workers > 1 else max(1, len(ii))):
            tasks.append(lambda e=int(e), ii=ii[s0:s1], jj=jj[s0:s1]: piece(e, ii, jj))
    pool.run(tasks, workers)
    ref = np.zeros((R, H), dtype=np.float64)
    for j in range(k):
        ref += np.asarray(topk_weights[:, j], dtype=np.float64)[:, None] * y[:, j]
    return ref, hh, h8s, hss
