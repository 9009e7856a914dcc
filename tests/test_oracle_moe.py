"""Pins of the oracle's expert stages and their composition."""
import math

import numpy as np
import torch

from oracle import fp8, moe, quant, routing, sort


def test_silu_mul_closed_forms():
    g = np.array([0.0, math.log(3.0), -math.log(3.0), 50.0, -800.0], np.float64)
    u = np.array([5.0, 2.0, 2.0, 1.0, 1.0])
    h = moe.silu_mul_f32(g, u)
    # SiLU(0)=0; sigmoid(ln 3) = 3/4; sigmoid(-ln 3) = 1/4; SiLU(50) ~ 50; SiLU(-800) -> -0
    exp = np.float32([0.0, 0.75 * math.log(3.0) * 2, -0.25 * math.log(3.0) * 2, 50.0, 0.0])
    assert np.allclose(h, exp, rtol=1e-6, atol=0)
    t = torch.nn.functional.silu(torch.tensor(g)) * torch.tensor(u)
    assert np.array_equal(h, t.numpy().astype(np.float32))


def _small_layer(rng, T=6, H=256, I=128, E=4, k=2):
    x = (rng.standard_normal((T, H))).astype(np.float32)
    a8, sa = quant.quant_1x128(x)
    w1 = rng.integers(0, 0x7F, (E, 2 * I, H)).astype(np.uint8) & 0x3F | (rng.integers(0, 2, (E, 2 * I, H)).astype(np.uint8) << 7)
    w2 = rng.integers(0, 0x7F, (E, H, I)).astype(np.uint8) & 0x3F | (rng.integers(0, 2, (E, H, I)).astype(np.uint8) << 7)
    s1 = (rng.random((E, 2 * I // 128, H // 128)) * 0.01).astype(np.float32)
    s2 = (rng.random((E, H // 128, I // 128)) * 0.01).astype(np.float32)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    G = 2 if E >= 4 else 1
    w, ids = routing.grouped_topk(logits, np.zeros(E, np.float32), G, G, k, True, 2.5)
    return a8, sa, w1, s1, w2, s2, w, ids


def test_sorted_path_equals_token_major(rng):
    a8, sa, w1, s1, w2, s2, w, ids = _small_layer(rng)
    T, k = ids.shape
    for BM in (16, 64):
        sid, sw, seid, P = sort.moe_sort(ids, w, w1.shape[0], BM)
        h8, hs, h, valid = moe.g1u1(a8, sa, w1, s1, sid, seid, P, k, BM)
        out = moe.down_combine(h8, hs, w2, s2, sid, sw, seid, P, T, k, BM)
        ref, _, h8t, hst = moe.layer_tokens(a8, sa, w1, s1, w2, s2, ids, w)
        assert np.array_equal(out, ref)
        # one row at a time gives the same bits
        for t in range(T):
            r1, _, _, _ = moe.layer_tokens(a8[t:t + 1], sa[t:t + 1], w1, s1, w2, s2, ids[t:t + 1], w[t:t + 1])
            assert np.array_equal(r1[0], ref[t])
        for r in np.nonzero(valid)[0]:
            t, j = divmod(int(sid[r]), k)
            assert np.array_equal(h8[r], h8t[t, j]) and np.array_equal(hs[r], hst[t, j])


def test_gate_up_selection_gives_silu_times_value(rng):
    # gate row i and up row i both pick input column i: h_i = SiLU(a_i) * a_i
    T, H, I, E = 3, 256, 128, 1
    x = rng.standard_normal((T, H)).astype(np.float32)
    a8, sa = quant.quant_1x128(x)
    w1 = np.zeros((E, 2 * I, H), np.uint8)
    w1[0, np.arange(I), np.arange(I)] = 0x38
    w1[0, I + np.arange(I), np.arange(I)] = 0x38
    s1 = np.ones((E, 2, 2), np.float32)
    ids = np.zeros((T, 1), np.int32)
    sid, sw, seid, P = sort.moe_sort(ids, np.ones((T, 1), np.float32), E, 16)
    h8, hs, h, valid = moe.g1u1(a8, sa, w1, s1, sid, seid, P, 1, 16)
    a = torch.tensor(fp8.decode(a8[:, :I]) * sa[:, :1].astype(np.float64))
    expect = (torch.nn.functional.silu(a) * a).numpy().astype(np.float32)
    assert np.array_equal(h[:T], expect)


def test_topk1_identity_down_returns_dequantised_h(rng):
    # topk=1 with renorm and factor 1 gives weight exactly 1; w2 = identity (H = I), unit scales
    T, H, I, E = 4, 128, 128, 2
    a8, sa, w1, s1, _, _, _, _ = _small_layer(rng, T=T, H=H, I=I, E=E, k=1)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    w, ids = routing.grouped_topk(logits, np.zeros(E, np.float32), 1, 1, 1, True, 1.0)
    assert np.all(w == 1.0)
    w2 = np.zeros((E, H, I), np.uint8)
    w2[:, np.arange(H), np.arange(I)] = 0x38
    s2 = np.ones((E, 1, 1), np.float32)
    sid, sw, seid, P = sort.moe_sort(ids, w, E, 16)
    h8, hs, h, valid = moe.g1u1(a8, sa, w1, s1, sid, seid, P, 1, 16)
    out = moe.down_combine(h8, hs, w2, s2, sid, sw, seid, P, T, 1, 16)
    for r in np.nonzero(valid)[0]:
        assert np.array_equal(out[sid[r]], quant.dequant_1x128(h8[r:r + 1], hs[r:r + 1])[0])


def test_smoothing_by_powers_of_two_moves_only_the_scales(rng):
    # a factor 2^j on a whole 128-column group of h multiplies the group's amax, hence
    # its 1x128 scale, by 2^j exactly, and leaves every e4m3 code unchanged
    T, H, I, E = 6, 256, 256, 4
    a8, sa, w1, s1, w2, s2, w, ids = _small_layer(rng, T=T, H=H, I=I, E=E, k=2)
    sid, sw, seid, P = sort.moe_sort(ids, w, E, 16)
    h8, hs, h, valid = moe.g1u1(a8, sa, w1, s1, sid, seid, P, 2, 16)
    j = rng.integers(-3, 4, (E, I // 128))
    smooth = np.repeat(np.ldexp(np.float32(1), j), 128, axis=1).astype(np.float32)
    h8s, hss, hsm, _ = moe.g1u1(a8, sa, w1, s1, sid, seid, P, 2, 16, fc2_smooth_scale=smooth)
    rows = np.nonzero(valid)[0]
    e_of_row = np.asarray(seid)[rows // 16]
    assert np.array_equal(h8s[rows], h8[rows])
    assert np.array_equal(hss[rows], (hs[rows] * np.ldexp(np.float32(1), j[e_of_row])).astype(np.float32))
    # all-ones factors are the unsmoothed layer
    h81, hs1, _, _ = moe.g1u1(a8, sa, w1, s1, sid, seid, P, 2, 16, fc2_smooth_scale=np.ones((E, I), np.float32))
    assert np.array_equal(h81, h8) and np.array_equal(hs1, hs)


def test_smoothing_zero_channel_zeroes_its_codes(rng):
    # a zero factor silences exactly its channel: code 0 there, the other channels keep
    # their values up to the group's re-derived scale
    T, H, I, E = 5, 128, 128, 2
    a8, sa, w1, s1, w2, s2, w, ids = _small_layer(rng, T=T, H=H, I=I, E=E, k=1)
    sid, sw, seid, P = sort.moe_sort(ids, w, E, 16)
    smooth = np.ones((E, I), np.float32)
    smooth[:, 7] = 0.0
    h8, hs, h, valid = moe.g1u1(a8, sa, w1, s1, sid, seid, P, 1, 16, fc2_smooth_scale=smooth)
    rows = np.nonzero(valid)[0]
    assert np.all(h8[rows, 7] & 0x7F == 0)
    _, _, hraw, _ = moe.g1u1(a8, sa, w1, s1, sid, seid, P, 1, 16)
    keep = np.arange(I) != 7
    assert np.array_equal(h[np.ix_(rows, keep)], hraw[np.ix_(rows, keep)])


def test_worker_pool_gives_identical_results(rng):
    # the thread-pool evaluation of independent experts / blocks / row groups equals the
    # serial one bit for bit (block sums are exact, every piece writes its own rows)
    from oracle import moe as omoe
    a8, sa, w1, s1, w2, s2, w, ids = _small_layer(rng, T=40, E=4, k=2)
    T, k = ids.shape
    old = omoe.ROW_CHUNK
    try:
        omoe.ROW_CHUNK = 7                       # several pieces per expert
        r1 = moe.layer_tokens(a8, sa, w1, s1, w2, s2, ids, w)
        r4 = moe.layer_tokens(a8, sa, w1, s1, w2, s2, ids, w, workers=4)
    finally:
        omoe.ROW_CHUNK = old
    for x1, x4 in zip(r1, r4):
        assert np.array_equal(x1, x4)
    sid, sw, seid, P = sort.moe_sort(ids, w, w1.shape[0], 16)
    g1 = moe.g1u1(a8, sa, w1, s1, sid, seid, P, k, 16)
    g4 = moe.g1u1(a8, sa, w1, s1, sid, seid, P, k, 16, workers=4)
    for x1, x4 in zip(g1, g4):
        assert np.array_equal(x1, x4)
    d1 = moe.down_combine(g1[0], g1[1], w2, s2, sid, sw, seid, P, T, k, 16)
    d4 = moe.down_combine(g1[0], g1[1], w2, s2, sid, sw, seid, P, T, k, 16, workers=4)
    assert np.array_equal(d1, d4)
    x = rng.standard_normal((700, 384)).astype(np.float32)
    q1, s_1 = quant.quant_1x128(x)
    q4, s_4 = quant.quant_1x128(x, workers=4)
    assert np.array_equal(q1, q4) and np.array_equal(s_1, s_4)
