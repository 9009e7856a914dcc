"""Pins of the oracle's MoE sort."""
import numpy as np
import pytest

from oracle import sort


def _brute(ids, weights, E, BM):
    T, k = ids.shape
    sid, sw, seid = [], [], []
    for e in range(E):
        seg = [(t * k + j, weights[t, j]) for t in range(T) for j in range(k) if ids[t, j] == e]
        if not seg:
            continue
        while len(seg) % BM:
            seg.append((T * k, 0.0))
        sid += [p for p, _ in seg]
        sw += [v for _, v in seg]
        seid += [e] * (len(seg) // BM)
    return sid, sw, seid


@pytest.mark.parametrize("T,k,E,BM", [(16, 4, 16, 16), (37, 8, 32, 32), (5, 2, 64, 64), (100, 3, 7, 128), (1, 1, 4, 16)])
def test_sort_properties_and_brute_force(rng, T, k, E, BM):
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    sid, sw, seid, P = sort.moe_sort(ids, w, E, BM)
    bsid, bsw, bseid = _brute(ids, w, E, BM)
    assert list(sid) == bsid and list(seid) == bseid and np.array_equal(sw, np.float32(bsw))
    # invariants
    assert P == len(sid) and P % BM == 0
    assert P <= sort.max_sizes(T, k, E, BM)[0]
    real = sid[sid < T * k]
    assert sorted(real.tolist()) == list(range(T * k))                  # every pair exactly once
    assert np.all(sw[sid == T * k] == 0)
    for blk, e in enumerate(seid):
        rows = sid[blk * BM:(blk + 1) * BM]
        r = rows[rows < T * k]
        assert len(r) > 0 and np.all(ids.reshape(-1)[r] == e)            # block owns one expert
        assert np.all(np.diff(r) > 0)                                      # ascending
        assert np.all(w.reshape(-1)[r] == sw[blk * BM:(blk + 1) * BM][rows < T * k])
    assert np.all(np.diff(seid) >= 0)


def test_all_pairs_one_expert_and_empty():
    ids = np.full((10, 1), 3, np.int32)
    w = np.ones((10, 1), np.float32)
    sid, sw, seid, P = sort.moe_sort(ids, w, 8, 16)
    assert P == 16 and list(seid) == [3] and list(sid[:10]) == list(range(10)) and np.all(sid[10:] == 10)
    sid, sw, seid, P = sort.moe_sort(np.zeros((0, 2), np.int32), np.zeros((0, 2), np.float32), 8, 16)
    assert P == 0 and len(seid) == 0
