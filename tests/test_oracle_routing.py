"""Pins of the oracle's biased grouped top-k."""
import math

import numpy as np
import pytest
import torch

from oracle import routing


def _check_row(x, bias, ids, w, G, tg, k, renorm, factor):
    """Brute-force property check of one token's routing (pure Python floats, fp32 where stated)."""
    E = len(x)
    gsz = E // G
    s = [np.float32(1.0 / (1.0 + math.exp(-float(v)))) for v in x]
    b = [np.float32(s[e] + bias[e]) for e in range(E)]
    gs = []
    for g in range(G):
        vals = sorted((b[e] for e in range(g * gsz, (g + 1) * gsz)), reverse=True)
        gs.append(np.float32(vals[0] + vals[1]))
    groups = sorted(range(G), key=lambda g: (-gs[g], g))[:tg]
    ids = [int(v) for v in ids]
    assert len(set(ids)) == k                                 # k distinct experts
    assert {e // gsz for e in ids} <= set(groups)             # all inside the kept groups
    cand = [e for e in range(E) if e // gsz in groups]
    best = sorted(cand, key=lambda e: (-b[e], e))[:k]
    assert ids == best                                        # exactly the best k, in key order
    ww = [s[e] for e in ids]
    if renorm:
        S = np.float32(0.0)
        S = ww[0]
        for v in ww[1:]:
            S = np.float32(S + v)
        ww = [np.float32(v / S) for v in ww]
    ww = [np.float32(v * np.float32(factor)) for v in ww]
    assert np.array_equal(np.array(ww, np.float32), np.asarray(w, np.float32))
    if renorm:
        assert abs(float(np.sum(np.asarray(w, np.float64))) - factor) <= 1e-6 * factor * k


@pytest.mark.parametrize("T,E,G,tg,k", [(16, 16, 4, 2, 4), (32, 64, 8, 4, 8), (8, 256, 8, 4, 8), (12, 24, 3, 2, 5)])
@pytest.mark.parametrize("renorm", [True, False])
def test_properties_random(rng, T, E, G, tg, k, renorm):
    x = rng.standard_normal((T, E)).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
    w, ids = routing.grouped_topk(x, bias, G, tg, k, renorm, 2.5)
    for t in range(T):
        _check_row(x[t], bias, ids[t], w[t], G, tg, k, renorm, 2.5)


def test_single_group_is_plain_topk(rng):
    # G = tg = 1: the choice is the plain top-k of the biased scores (distinct values)
    x = rng.standard_normal((50, 40)).astype(np.float32)
    bias = (rng.standard_normal(40) * 0.1).astype(np.float32)
    w, ids = routing.grouped_topk(x, bias, 1, 1, 6, False, 1.0)
    s, b = routing.biased_scores(x, bias)
    vals, tids = torch.topk(torch.from_numpy(b), 6, dim=1)
    assert np.array_equal(ids, tids.numpy().astype(np.int32))
    assert np.array_equal(w, np.take_along_axis(s, tids.numpy(), 1))


def test_zero_bias_is_topk_of_logits(rng):
    x = rng.standard_normal((20, 32)).astype(np.float32)
    w, ids = routing.grouped_topk(x, np.zeros(32, np.float32), 1, 1, 4, True, 1.0)
    _, tids = torch.topk(torch.from_numpy(x), 4, dim=1)
    assert np.array_equal(ids, tids.numpy().astype(np.int32))


def test_group_restriction_worked_example():
    # E=8 in 4 groups of 2, keep 2 groups, top-2.  Expert 6 has the largest score
    # but its group {6,7} scores s(5)+s(-5) ~ 1.0 < s(0)+s(1) ~ 1.23 < s(2)+s(3) ~ 1.83,
    # so the kept groups are {2,3} and {0,1} and the answer is experts 3, 2.
    x = np.array([[0, 1, 2, 3, -1, -2, 5, -5]], np.float32)
    w, ids = routing.grouped_topk(x, np.zeros(8, np.float32), 4, 2, 2, True, 2.5)
    assert list(ids[0]) == [3, 2]
    # renormalised weights: ratio s(3)/s(2) = (1+e^-2)/(1+e^-3), sum = 2.5
    assert abs(w[0, 0] / w[0, 1] - (1 + math.exp(-2)) / (1 + math.exp(-3))) < 1e-6
    assert abs(float(w[0].sum()) - 2.5) < 1e-6
    # without the group step the answer would include expert 6
    w1, ids1 = routing.grouped_topk(x, np.zeros(8, np.float32), 1, 1, 2, True, 2.5)
    assert list(ids1[0]) == [6, 3]


def test_bias_steers_choice_but_weights_unbiased():
    x = np.zeros((1, 4), np.float32)                   # all scores 0.5
    bias = np.array([0.0, 0.3, 0.0, 0.2], np.float32)
    w, ids = routing.grouped_topk(x, bias, 1, 1, 2, False, 1.0)
    assert list(ids[0]) == [1, 3]
    assert np.all(w == np.float32(0.5))                # weights from the unbiased sigmoid


def test_ties_lower_index_wins():
    x = np.zeros((1, 8), np.float32)                   # every expert equal
    w, ids = routing.grouped_topk(x, np.zeros(8, np.float32), 4, 2, 3, True, 1.0)
    # all groups tie -> groups 0 and 1 are kept; experts tie -> 0, 1, 2
    assert list(ids[0]) == [0, 1, 2]
    assert np.all(w[0] == np.float32(np.float32(0.5) / np.float32(1.5)))


def test_group_tie_lower_group_wins():
    x = np.array([[1, 0, 1, 0, -1, -1]], np.float32)     # groups of 2: g0 and g1 tie, g2 lower
    w, ids = routing.grouped_topk(x, np.zeros(6, np.float32), 3, 1, 2, False, 1.0)
    assert list(ids[0]) == [0, 1]


def test_factor_applied_without_renorm():
    x = np.array([[2.0, -1.0, 0.5, 0.0]], np.float32)
    w, ids = routing.grouped_topk(x, np.zeros(4, np.float32), 2, 2, 2, False, 2.5)
    s = routing.sigmoid_f32(x)
    assert np.array_equal(w[0], np.float32(2.5) * s[0, ids[0]])
