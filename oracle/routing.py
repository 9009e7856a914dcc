"""Biased grouped top-k routing (CPU oracle; test infrastructure only).

"Accelerate DeepSeek-R1 Inference: Integrate AITER into SGLang", section
"Complete MoE Implementation" / "Top-K routing": each token may only pick
experts from a fixed number of expert groups and then takes its top-k
experts from the chosen groups; a correction bias is added to the scores;
the weights are optionally renormalised and multiplied by the routed
scaling factor (the test there multiplies the reference weights by the
factor; the API comment says the factor multiplies topk_weights).

Readings taken where the page is silent (all per token, fl32 = round to
float32, nearest-even):
  1. score      s_e = fl32(1 / (1 + exp(-x_e)))  evaluated in binary64
  2. biased     b_e = fl32(s_e + bias_e)
  3. groups are E/G contiguous experts; group score gs_g = fl32(m1 + m2),
     m1 >= m2 the two largest b_e of the group
  4. keep the topk_group groups first in the order (gs desc, g asc)
  5. candidates are the experts of the kept groups only; order them by
     (b desc, e asc) and take the first topk, in that order
  6. weights use the unbiased score: w_j = s_{id_j}
  7. renorm: S = fl32 left-to-right sum of w_0..w_{k-1}; w_j = fl32(w_j / S)
  8. w_j = fl32(w_j * routed_scaling_factor), with or without renorm
Ties on a key go to the lower index.  Equal values (including +0 / -0)
compare equal.
"""
import numpy as np


def sigmoid_f32(x):
    """fl32 of the binary64 logistic function."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    with np.errstate(over="ignore"):
        return (1.0 / (1.0 + np.exp(-x64))).astype(np.float32)


def grouped_topk(logits, bias, n_group, topk_group, topk, renorm, routed_scaling_factor):
    """logits float32 [T, E], bias float32 [E] -> (weights float32 [T, k], ids int32 [T, k])."""
    logits = np.asarray(logits, dtype=np.float32)
    bias = np.asarray(bias, dtype=np.float32)
    T, E = logits.shape
    assert E % n_group == 0 and E // n_group >= 2
    assert 1 <= topk_group <= n_group and 1 <= topk <= topk_group * (E // n_group)
    gsz = E // n_group

    s = sigmoid_f32(logits)                                          # step 1
    b = np.add(s, bias[None, :], dtype=np.float32)                   # step 2

    # step 3: top-2 sum per group (sorting values; ties do not matter here)
    bg = b.reshape(T, n_group, gsz)
    top2 = -np.sort(-bg, axis=2)[:, :, :2]
    gs = np.add(top2[:, :, 0], top2[:, :, 1], dtype=np.float32)      # [T, G]

    # step 4: stable sort on (-gs) keeps equal scores in ascending group order
    gorder = np.argsort(-gs, axis=1, kind="stable")
    kept = gorder[:, :topk_group]                                    # [T, tg]

    ids = np.empty((T, topk), dtype=np.int32)
    for t in range(T):
        # step 5: candidate experts, ascending expert index, then stable sort on -b
        cand = np.sort(np.concatenate([np.arange(g * gsz, (g + 1) * gsz) for g in kept[t]]))
        order = np.argsort(-b[t, cand], kind="stable")
        ids[t] = cand[order[:topk]]

    w = np.take_along_axis(s, ids.astype(np.int64), axis=1).astype(np.float32)   # step 6
    if renorm:                                                       # step 7
        S = w[:, 0].copy()
        for j in range(1, topk):
            S = np.add(S, w[:, j], dtype=np.float32)
        w = np.divide(w, S[:, None], dtype=np.float32)
    w = np.multiply(w, np.float32(routed_scaling_factor), dtype=np.float32)      # step 8
    return w, ids


def biased_scores(logits, bias):
    """(s, b) of steps 1-2, exposed for the property checks in the tests."""
    s = sigmoid_f32(logits)
    return s, np.add(s, np.asarray(bias, dtype=np.float32)[None, :], dtype=np.float32)
