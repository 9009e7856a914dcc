"""MoE align/sort (CPU oracle; test infrastructure only).

"Accelerate DeepSeek-R1 Inference: Integrate AITER into SGLang", section
"Complete MoE Implementation" / "MoE Sorting": token-expert pairs are
bucketed per expert for the grouped GEMM, which consumes
sorted_token_ids, sorted_weight_buf, sorted_expert_ids and num_valid_ids.

Reading taken for the encoding (the page gives only the names), with
pairs flattened as p = t*topk + j and block size BM:
  c_e   = number of pairs routed to expert e
  p_e   = ceil(c_e / BM) * BM      (experts with no pair get no block)
  off_e = sum of p_e' over e' < e,  P = sum of all p_e
  sorted_ids[off_e + i]    = i-th pair of expert e in ascending p, i < c_e
  sorted_weights[same]     = topk_weights of that pair
  padding slots            = sentinel T*topk with weight 0.0
  sorted_expert_ids[blk]   = expert owning rows [blk*BM, (blk+1)*BM)
  num_valid                = P
"""
import numpy as np


def max_sizes(T, topk, E, block_m):
    """Worst-case padded length and block count: T*k + E*(BM-1), rounded to BM."""
    max_sorted = T * topk + E * (block_m - 1)
    max_sorted = -(-max_sorted // block_m) * block_m
    return max_sorted, max_sorted // block_m


def moe_sort(ids, weights, E, block_m):
    """ids int32 [T, k], weights float32 [T, k] -> (sorted_ids, sorted_weights, sorted_expert_ids, P)."""
    ids = np.asarray(ids)
    weights = np.asarray(weights, dtype=np.float32)
    T, k = ids.shape
    flat_ids = ids.reshape(-1).astype(np.int64)
    flat_w = weights.reshape(-1)
    sentinel = T * k
    sorted_ids, sorted_w, sorted_eid = [], [], []
    for e in range(E):
        pairs = np.nonzero(flat_ids == e)[0]          # ascending flat index
        c = len(pairs)
        if c == 0:
            continue
        p = -(-c // block_m) * block_m
        sorted_ids.append(pairs.astype(np.int32))
        sorted_w.append(flat_w[pairs])
        sorted_ids.append(np.full(p - c, sentinel, dtype=np.int32))
        sorted_w.append(np.zeros(p - c, dtype=np.float32))
        sorted_eid.append(np.full(p // block_m, e, dtype=np.int32))
    if sorted_ids:
        sid = np.concatenate(sorted_ids)
        sw = np.concatenate(sorted_w).astype(np.float32)
        seid = np.concatenate(sorted_eid)
    else:
        sid = np.zeros(0, np.int32)
        sw = np.zeros(0, np.float32)
        seid = np.zeros(0, np.int32)
    return sid, sw, seid, int(len(sid))
