"""GPU parity on the tiny MoE layer and small dense shapes (every output element checked)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as ofp8
from tests.helpers import assert_rel_max, check_requant, f32_of_bf16, np_u8, oracle_routing

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def m():
    import fp8_block_scaled_grouped_amd as mod
    mod.lib()
    return mod


@pytest.fixture(scope="module")
def tiny():
    from fp8_block_scaled_grouped_amd import inputs
    cfg = inputs.MOE_CONFIGS["tiny"]
    return cfg, inputs.make_moe_inputs(cfg, "cpu", seed=0)


def _edge_rows(K):
    rows = [np.zeros(K), -np.zeros(K), np.linspace(-3, 3, K), np.full(K, 1e-30), np.full(K, -2.0 ** -140)]
    v = ofp8.decode(np.arange(127, dtype=np.uint8))
    mids = ((v[:-1] + v[1:]) / 2)
    rows.append(np.resize(np.concatenate([mids, -mids, [448.0]]), K))   # exact midpoints, amax 448
    rows.append(np.resize(np.array([1e30, -1e30, 3e38, 1.0]), K))
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("M,K", [(16, 256), (37, 1280), (1, 128), (300, 7168), (19, 200), (3, 72), (40, 7176)])
@pytest.mark.parametrize("layout", ["row", "kblock"])
def test_quant_bitexact(m, M, K, layout):
    print("quant", M, K, layout, flush=True)
    g = torch.Generator().manual_seed(M * 131 + K)
    x = (torch.randn((M, K), generator=g) * torch.exp2(torch.randint(-30, 30, (M, 1), generator=g).float()))
    x = x.to(torch.bfloat16)
    if M >= 7:
        x[:7] = torch.from_numpy(_edge_rows(K)).to(torch.bfloat16)
    q, s = m.fp8_quant_1x128(x.to(DEV), scale_layout=layout)
    torch.cuda.synchronize()
    qr, sr = oracle.quant.quant_1x128(f32_of_bf16(x))
    s = s.cpu().numpy()
    if layout == "kblock":
        s = s.T
    assert np.array_equal(np_u8(q), qr)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))


def test_quant_strided_rows(m):
    x = torch.randn((8, 512 + 64)).to(torch.bfloat16).to(DEV)[:, :512]
    qbuf = torch.zeros((8, 640), dtype=torch.uint8, device=DEV)
    q, s = m.fp8_quant_1x128(x, q=qbuf[:, :512])
    torch.cuda.synchronize()
    qr, sr = oracle.quant.quant_1x128(f32_of_bf16(x))
    assert np.array_equal(np_u8(qbuf[:, :512]), qr) and np.all(np_u8(qbuf[:, 512:]) == 0)
    assert np.array_equal(s.cpu().numpy(), sr)


@pytest.mark.parametrize("ld_extra", [0, 10])
def test_topk_bitexact_tiny(m, tiny, ld_extra):
    cfg, x = tiny
    k = cfg.topk
    wbuf = torch.full((cfg.T, k + ld_extra), -7.0, device=DEV)
    ibuf = torch.full((cfg.T, k + ld_extra), -7, dtype=torch.int32, device=DEV)
    m.grouped_topk(x["logits"].to(DEV), x["bias"].to(DEV), cfg.n_group, cfg.topk_group, k, cfg.renorm,
                   cfg.routed_scaling_factor, wbuf[:, :k], ibuf[:, :k])
    torch.cuda.synchronize()
    w, ids = oracle_routing(x, cfg)
    assert np.array_equal(ibuf[:, :k].cpu().numpy(), ids)
    assert np.array_equal(wbuf[:, :k].cpu().numpy().view(np.uint32), w.view(np.uint32))
    assert np.all(ibuf[:, k:].cpu().numpy() == -7)


@pytest.mark.parametrize("T,E,G,tg,k,renorm", [(1, 16, 4, 2, 4, True), (33, 64, 8, 3, 6, False), (5, 1024, 64, 8, 32, True),
                                               (100, 256, 8, 4, 8, True), (7, 24, 3, 2, 5, True),
                                               # group shapes off the register path (12 or 24 experts per group)
                                               (20, 96, 4, 2, 6, True), (9, 48, 4, 3, 5, False), (3, 1000, 8, 2, 9, True)])
def test_topk_bitexact_shapes(m, T, E, G, tg, k, renorm):
    g = torch.Generator().manual_seed(T * 7 + E)
    logits = torch.randn((T, E), generator=g)
    bias = torch.randn((E,), generator=g) * 0.1
    w, ids = m.grouped_topk(logits.to(DEV), bias.to(DEV), G, tg, k, renorm, 2.5)
    torch.cuda.synchronize()
    wr, ir = oracle.routing.grouped_topk(logits.numpy(), bias.numpy(), G, tg, k, renorm, 2.5)
    assert np.array_equal(ids.cpu().numpy(), ir)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), wr.view(np.uint32))


def test_topk_ties(m):
    logits = torch.zeros((3, 16))
    logits[1, ::2] = 1.0
    logits[2] = torch.tensor([1.0, 1.0, 0, 0] * 4)
    w, ids = m.grouped_topk(logits.to(DEV), torch.zeros(16, device=DEV), 4, 2, 4, True, 1.0)
    torch.cuda.synchronize()
    wr, ir = oracle.routing.grouped_topk(logits.numpy(), np.zeros(16, np.float32), 4, 2, 4, True, 1.0)
    assert np.array_equal(ids.cpu().numpy(), ir)
    assert np.array_equal(w.cpu().numpy(), wr)


def _check_sort(m, ids, w, E, BM, ld_extra=0):
    T, k = ids.shape
    ib = torch.zeros((T, k + ld_extra), dtype=torch.int32)
    wb = torch.zeros((T, k + ld_extra), dtype=torch.float32)
    ib[:, :k] = torch.from_numpy(ids)
    wb[:, :k] = torch.from_numpy(w)
    ib, wb = ib.to(DEV), wb.to(DEV)
    sid, sw, seid, nv = m.moe_sort(ib[:, :k], wb[:, :k], E, BM)
    torch.cuda.synchronize()
    rsid, rsw, rseid, P = oracle.sort.moe_sort(ids, w, E, BM)
    assert int(nv.item()) == P
    assert np.array_equal(sid.cpu().numpy()[:P], rsid)
    assert np.array_equal(sw.cpu().numpy()[:P].view(np.uint32), rsw.view(np.uint32))
    assert np.array_equal(seid.cpu().numpy()[:P // BM], rseid)


@pytest.mark.parametrize("BM", [16, 32, 64, 128, 256])
def test_sort_bitexact_tiny_routing(m, tiny, BM):
    cfg, x = tiny
    w, ids = oracle_routing(x, cfg)
    _check_sort(m, ids, w, cfg.E, BM, ld_extra=10)


@pytest.mark.parametrize("T,k,E,BM", [(1, 1, 4, 16), (1000, 8, 256, 64), (300, 3, 1024, 16), (4096, 8, 256, 128),
                                      (2048, 8, 256, 32), (2049, 8, 256, 16), (5000, 4, 1000, 64),
                                      (4096, 8, 256, 256), (3000, 8, 64, 256)])
def test_sort_bitexact_random(m, T, k, E, BM):
    rng = np.random.default_rng(T + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    _check_sort(m, ids, w, E, BM)


def test_sort_all_one_expert_and_skewed(m):
    T, k, E = 777, 2, 32
    ids = np.stack([np.full(T, 5), np.full(T, 6)], 1).astype(np.int32)
    _check_sort(m, ids, np.ones((T, k), np.float32), E, 128)
    rng = np.random.default_rng(3)
    hot = rng.random((T, 4)) < 0.9
    ids = np.where(hot, np.arange(4)[None, :], rng.integers(4, E, (T, 4))).astype(np.int32)
    ids = np.stack([rng.permutation(E)[:4] if len(set(r)) < 4 else r for r in ids]).astype(np.int32)
    _check_sort(m, ids, rng.random((T, 4)).astype(np.float32), E, 64)


def _tiny_stage_inputs(tiny, BM):
    cfg, x = tiny
    w, ids = oracle_routing(x, cfg)
    sid, sw, seid, P = oracle.sort.moe_sort(ids, w, cfg.E, BM)
    ms = oracle.sort.max_sizes(cfg.T, cfg.topk, cfg.E, BM)[0]
    pad = lambda a, fill: np.concatenate([a, np.full(ms - len(a), fill, a.dtype)])
    a8, sa = oracle.quant.quant_1x128(f32_of_bf16(x["hidden"]))
    return cfg, x, w, ids, (pad(sid, cfg.T * cfg.topk), pad(sw, np.float32(0)), pad(seid, 0), P), a8, sa


@pytest.mark.parametrize("BM", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("smooth", [False, True], ids=["plain", "smooth"])
def test_g1u1_stage_tiny(m, tiny, BM, smooth):
    cfg, x, w, ids, (sid, sw, seid, P), a8, sa = _tiny_stage_inputs(tiny, BM)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    sm = None
    if smooth:  # per-expert channel factors spanning 2^-3 .. 2^3
        sm = np.exp2(np.random.default_rng(BM).uniform(-3, 3, (cfg.E, cfg.I))).astype(np.float32)
    h8, hs = m.moe_fp8_blockscale_g1u1(t(a8), t(sa), x["w1"].to(DEV), x["w1_scale"].to(DEV), t(sid), t(seid),
                                       t(np.array([P], np.int32)), cfg.topk, BM,
                                       fc2_smooth_scale=None if sm is None else t(sm))
    torch.cuda.synchronize()
    _, _, h_ref, valid = oracle.moe.g1u1(a8, sa, x["w1"].numpy(), x["w1_scale"].numpy(), sid, seid, P, cfg.topk, BM,
                                         fc2_smooth_scale=sm)
    rows = np.nonzero(valid)[0]
    check_requant(np_u8(h8)[rows], hs.cpu().numpy()[rows], h_ref[rows])


@pytest.mark.parametrize("BM", [16, 64, 256])
def test_down_stage_tiny(m, tiny, BM):
    cfg, x, w, ids, (sid, sw, seid, P), a8, sa = _tiny_stage_inputs(tiny, BM)
    h8, hs, _, valid = oracle.moe.g1u1(a8, sa, x["w1"].numpy(), x["w1_scale"].numpy(), sid, seid, P, cfg.topk, BM)
    ms = len(sid)
    h8p = np.zeros((ms, cfg.I), np.uint8)
    hsp = np.ones((ms, cfg.I // 128), np.float32)
    h8p[:P], hsp[:P] = h8, hs
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    out = m.moe_down_combine(t(h8p), t(hsp), x["w2"].to(DEV), x["w2_scale"].to(DEV), t(sid), t(sw), t(seid),
                             t(np.array([P], np.int32)), cfg.T, cfg.topk, BM)
    torch.cuda.synchronize()
    ref = oracle.moe.down_combine(h8, hs, x["w2"].numpy(), x["w2_scale"].numpy(), sid, sw, seid, P, cfg.T, cfg.topk, BM)
    assert_rel_max(f32_of_bf16(out), ref, what="down_combine tiny")
    # also tight: bf16 rounding of an fp32 sum
    assert np.all(np.abs(f32_of_bf16(out) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4 * np.abs(ref).max())


@pytest.mark.parametrize("BM", [16, 32])
@pytest.mark.parametrize("layout", ["row", "kblock"])
def test_layer_tiny(m, tiny, BM, layout):
    cfg, x = tiny
    g = {k: v.to(DEV) for k, v in x.items()}
    layer = m.MoELayer(cfg, g["bias"], g["w1"], g["w1_scale"], g["w2"], g["w2_scale"], block_m=BM,
                       scale_layout=layout)
    out = layer.forward(g["hidden"], g["logits"])
    torch.cuda.synchronize()
    w, ids = oracle_routing(x, cfg)
    assert np.array_equal(layer.topk_ids.cpu().numpy(), ids)
    a8, sa = oracle.quant.quant_1x128(f32_of_bf16(x["hidden"]))
    ref, _, _, _ = oracle.moe.layer_tokens(a8, sa, x["w1"].numpy(), x["w1_scale"].numpy(), x["w2"].numpy(),
                                           x["w2_scale"].numpy(), ids, w)
    assert_rel_max(f32_of_bf16(out), ref, what="tiny layer")


@pytest.mark.parametrize("BM", [16, 32, 64, 128])
@pytest.mark.parametrize("smooth", [False, True], ids=["plain", "smooth"])
def test_layer_tiny_fused(m, tiny, BM, smooth):
    # the single-launch expert computation equals the two calls bit for bit, and the oracle
    cfg, x = tiny
    g = {k: v.to(DEV) for k, v in x.items()}
    sm = None
    if smooth:
        sm = torch.from_numpy(np.exp2(np.random.default_rng(BM).uniform(-3, 3, (cfg.E, cfg.I))).astype(np.float32))
    args = (cfg, g["bias"], g["w1"], g["w1_scale"], g["w2"], g["w2_scale"])
    kw = dict(block_m=BM, fc2_smooth_scale=None if sm is None else sm.to(DEV))
    two = m.MoELayer(*args, **kw).forward(g["hidden"], g["logits"]).clone()
    one = m.MoELayer(*args, fused=True, **kw).forward(g["hidden"], g["logits"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(two.view(torch.int16), one.view(torch.int16))
    w, ids = oracle_routing(x, cfg)
    a8, sa = oracle.quant.quant_1x128(f32_of_bf16(x["hidden"]))
    ref, _, _, _ = oracle.moe.layer_tokens(a8, sa, x["w1"].numpy(), x["w1_scale"].numpy(), x["w2"].numpy(),
                                           x["w2_scale"].numpy(), ids, w, None if sm is None else sm.numpy())
    assert_rel_max(f32_of_bf16(one), ref, what="tiny fused layer")


def test_layer_tiny_deterministic(m, tiny):
    cfg, x = tiny
    g = {k: v.to(DEV) for k, v in x.items()}
    layer = m.MoELayer(cfg, g["bias"], g["w1"], g["w1_scale"], g["w2"], g["w2_scale"])
    a = layer.forward(g["hidden"], g["logits"]).clone()
    b = layer.forward(g["hidden"], g["logits"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# (5, 1024, 4096): 16 splits of 2 K blocks; (33, 256, 1664): 3 splits of 5, 5, 3 K blocks
@pytest.mark.parametrize("M,N,K", [(1, 384, 512), (37, 384, 512), (128, 256, 1024), (200, 128, 256), (16, 2048, 7168),
                                   (5, 1024, 4096), (33, 256, 1664),
                                   # 256-row tiles (M of 512 and more): ragged M, two K lengths
                                   (600, 512, 1024), (1030, 768, 2048)])
@pytest.mark.parametrize("layout", ["row", "kblock"])
@pytest.mark.parametrize("split", [True, False], ids=["ws", "nows"])
def test_dense_small(m, M, N, K, layout, split):
    from fp8_block_scaled_grouped_amd import inputs
    d = inputs.make_dense_inputs(M, N, K, "cpu", seed=M + N)
    a8, sa = oracle.quant.quant_1x128(f32_of_bf16(d["a"]))
    sa_dev = torch.from_numpy(sa if layout == "row" else np.ascontiguousarray(sa.T)).to(DEV)
    ws = None
    if split:
        # garbage in the workspace must not matter; two calls in a row on the same workspace
        nws = m.gemm_fp8_blockscale_workspace(M, N, K)
        ws = torch.full((max(nws, 16),), 0x7F, dtype=torch.uint8, device=DEV)
    args = (torch.from_numpy(a8).to(DEV), sa_dev, d["b"].to(DEV), d["b_scale"].to(DEV))
    c = m.gemm_fp8_blockscale(*args, scale_layout=layout, workspace=ws if split else False).clone()
    c2 = m.gemm_fp8_blockscale(*args, scale_layout=layout, workspace=ws if split else False)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), c2.view(torch.int16))
    ref = oracle.gemm.gemm_blockscale(a8, sa, d["b"].numpy(), d["b_scale"].numpy())
    assert_rel_max(f32_of_bf16(c), ref, what="dense %dx%dx%d" % (M, N, K))


# K and N off multiples of 128 (ceil-sized scales): partial N only, partial K only (16
# bytes past the last full block), both with 128-row tiles, K below one block, split-K
# with the partial block in the last split
@pytest.mark.parametrize("M,N,K", [(5, 576, 1024), (37, 256, 1040), (130, 200, 208), (1, 136, 64),
                                   (8, 1000, 4112), (64, 4104, 7184), (300, 520, 400), (700, 512, 1040)])
@pytest.mark.parametrize("split", [True, False], ids=["ws", "nows"])
def test_dense_partial_blocks(m, M, N, K, split):
    from fp8_block_scaled_grouped_amd import inputs
    print("dense partial", M, N, K, split, flush=True)
    d = inputs.make_dense_inputs(M, N, K, "cpu", seed=M + 7 * N + K)
    x = f32_of_bf16(d["a"])
    a8, sa = oracle.quant.quant_1x128(x)
    # the library's own quantisation of the partial last group agrees bit for bit
    q_dev, s_dev = m.fp8_quant_1x128(d["a"].to(DEV))
    c = m.gemm_fp8_blockscale(torch.from_numpy(a8).to(DEV), torch.from_numpy(sa).to(DEV), d["b"].to(DEV),
                              d["b_scale"].to(DEV), workspace=None if split else False)
    torch.cuda.synchronize()
    assert np.array_equal(np_u8(q_dev), a8)
    assert np.array_equal(s_dev.cpu().numpy().view(np.uint32), sa.view(np.uint32))
    ref = oracle.gemm.gemm_blockscale(a8, sa, d["b"].numpy(), d["b_scale"].numpy())
    assert_rel_max(f32_of_bf16(c), ref, what="dense partial %dx%dx%d" % (M, N, K))


# more than 128 K blocks: always split (a workgroup holds the scales of at most 128),
# also at M above 64; with partial N / K as well
@pytest.mark.parametrize("M,N,K", [(37, 256, 18432), (300, 512, 16512), (1, 576, 24576), (130, 136, 16400),
                                   (600, 512, 16512)])
def test_dense_long_k(m, M, N, K):
    from fp8_block_scaled_grouped_amd import inputs
    print("dense long K", M, N, K, flush=True)
    assert m.gemm_fp8_blockscale_workspace(M, N, K) > 0
    d = inputs.make_dense_inputs(M, N, K, "cpu", seed=M + N + K)
    a8, sa = oracle.quant.quant_1x128(f32_of_bf16(d["a"]))
    c = m.gemm_fp8_blockscale(torch.from_numpy(a8).to(DEV), torch.from_numpy(sa).to(DEV), d["b"].to(DEV),
                              d["b_scale"].to(DEV))
    torch.cuda.synchronize()
    ref = oracle.gemm.gemm_blockscale(a8, sa, d["b"].numpy(), d["b_scale"].numpy())
    assert_rel_max(f32_of_bf16(c), ref, what="dense long K %dx%dx%d" % (M, N, K))
    with pytest.raises(m.Moe355Error):
        m.gemm_fp8_blockscale(torch.from_numpy(a8).to(DEV), torch.from_numpy(sa).to(DEV), d["b"].to(DEV),
                              d["b_scale"].to(DEV), workspace=False)


def test_dense_partial_n_leaves_padding_columns(m):
    # c with a wider row stride: columns past N keep their contents
    from fp8_block_scaled_grouped_amd import inputs
    M, N, K = 20, 264, 336
    d = inputs.make_dense_inputs(M, N, K, DEV, seed=11)
    a8, sa = m.fp8_quant_1x128(d["a"])
    cbuf = torch.full((M, 512), 5.0, dtype=torch.bfloat16, device=DEV)
    m.gemm_fp8_blockscale(a8, sa, d["b"], d["b_scale"], c=cbuf[:, :N])
    c2 = m.gemm_fp8_blockscale(a8, sa, d["b"], d["b_scale"])
    torch.cuda.synchronize()
    assert bool((cbuf[:, N:] == 5.0).all())
    assert torch.equal(cbuf[:, :N].view(torch.int16), c2.view(torch.int16))


def test_shuffle_weight_bitexact(m):
    w = np.random.default_rng(3).integers(0, 256, size=(3, 256, 384), dtype=np.uint8)
    out = m.shuffle_weight_128x128(torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.layout.shuffle_128x128(w))


# pre-shuffled weights: every tile shape (BM 16/64/128, 128 and 256 B rows), split-K or not;
# the arithmetic is unchanged, so the output equals the plain call's bit for bit
@pytest.mark.parametrize("M,N,K", [(1, 2048, 7168), (37, 384, 512), (200, 128, 256), (130, 512, 1024),
                                   (64, 256, 4096)])
def test_dense_preshuffled_bitwise(m, M, N, K):
    from fp8_block_scaled_grouped_amd import inputs
    print("dense preshuffled", M, N, K, flush=True)
    d = inputs.make_dense_inputs(M, N, K, DEV, seed=M + N)
    a8, sa = m.fp8_quant_1x128(d["a"])
    bsh = m.shuffle_weight_128x128(d["b"])
    for ws in (None, False):
        c0 = m.gemm_fp8_blockscale(a8, sa, d["b"], d["b_scale"], workspace=ws)
        c1 = m.gemm_fp8_blockscale(a8, sa, bsh, d["b_scale"], workspace=ws, preshuffled=True)
        torch.cuda.synchronize()
        assert torch.equal(c0.view(torch.int16), c1.view(torch.int16))
    ref = oracle.gemm.gemm_blockscale(np_u8(a8), sa.cpu().numpy(), d["b"].cpu().numpy(), d["b_scale"].cpu().numpy())
    assert_rel_max(f32_of_bf16(c1), ref, what="dense preshuffled %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("BM", [16, 32, 64, 128, 256])
def test_layer_tiny_preshuffled_bitwise(m, tiny, BM):
    cfg, x = tiny
    g = {k: v.to(DEV) for k, v in x.items()}
    args = (cfg, g["bias"], g["w1"], g["w1_scale"], g["w2"], g["w2_scale"])
    plain = m.MoELayer(*args, block_m=BM)
    shuf = m.MoELayer(*args, block_m=BM, preshuffle=True)
    a = plain.forward(g["hidden"], g["logits"]).clone()
    b = shuf.forward(g["hidden"], g["logits"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # the requantised intermediate of every valid sorted row as well
    P = int(plain.sort_out[3].item())
    valid = plain.sort_out[0][:P] < cfg.T * cfg.topk
    assert torch.equal(plain.h8[:P][valid], shuf.h8[:P][valid])
    assert torch.equal(plain.h_scale[:P][valid], shuf.h_scale[:P][valid])
    w, ids = oracle_routing(x, cfg)
    a8, sa = oracle.quant.quant_1x128(f32_of_bf16(x["hidden"]))
    ref, _, _, _ = oracle.moe.layer_tokens(a8, sa, x["w1"].numpy(), x["w1_scale"].numpy(), x["w2"].numpy(),
                                           x["w2_scale"].numpy(), ids, w)
    assert_rel_max(f32_of_bf16(b), ref, what="tiny layer, pre-shuffled weights")


@pytest.mark.parametrize("BM", [16, 128])
def test_layer_graph_replay_matches_eager(m, tiny, BM):
    # the five calls allocate nothing and never synchronise: captured once as a graph, every
    # replay (with eager work and synchronisations between replays) reproduces the eager output
    # (with the quantisation on the layer's side stream: the capture forks and joins it)
    cfg, x = tiny
    g = {k: v.to(DEV) for k, v in x.items()}
    layer = m.MoELayer(cfg, g["bias"], g["w1"], g["w1_scale"], g["w2"], g["w2_scale"], block_m=BM,
                       overlap_quant=True)
    eager = layer.forward(g["hidden"], g["logits"]).clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward(g["hidden"], g["logits"])
    for i in range(3):
        layer.out.fill_(float(i + 7))
        other = m.MoELayer(cfg, g["bias"], g["w1"], g["w1_scale"], g["w2"], g["w2_scale"], block_m=16)
        other.forward(g["hidden"], g["logits"])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.out.view(torch.int16), eager.view(torch.int16)), "replay %d" % i


@pytest.mark.parametrize("BM", [16, 128])
def test_layer_quant_overlap_matches_serial(m, tiny, BM):
    # quantisation on the layer's side stream gives the serial layer's output bit for bit,
    # also over two back-to-back calls on different inputs (the second call's quantisation
    # must wait for the first call's GEMMs, which read the same a8 buffer)
    cfg, x = tiny
    g = {k: v.to(DEV) for k, v in x.items()}
    h2 = (g["hidden"].float() * -0.75).to(torch.bfloat16)
    lg2 = g["logits"].flip(1).contiguous()
    over = m.MoELayer(cfg, g["bias"], g["w1"], g["w1_scale"], g["w2"], g["w2_scale"], block_m=BM,
                      overlap_quant=True)
    serial = m.MoELayer(cfg, g["bias"], g["w1"], g["w1_scale"], g["w2"], g["w2_scale"], block_m=BM)
    assert over.side is not None and serial.side is None
    o1 = over.forward(g["hidden"], g["logits"]).clone()
    o2 = over.forward(h2, lg2).clone()
    s1 = serial.forward(g["hidden"], g["logits"]).clone()
    s2 = serial.forward(h2, lg2).clone()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), s1.view(torch.int16))
    assert torch.equal(o2.view(torch.int16), s2.view(torch.int16))
    assert not torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_binding_rejects_wrong_shapes(m, tiny):
    # a shape mistake raises in the binding before any pointer reaches a kernel
    cfg, x = tiny
    g = {k: v.to(DEV) for k, v in x.items()}
    layer = m.MoELayer(cfg, g["bias"], g["w1"], g["w1_scale"], g["w2"], g["w2_scale"])
    layer.forward(g["hidden"], g["logits"])
    sid, sw, seid, nv = layer.sort_out
    with pytest.raises(ValueError):
        m.moe_fp8_blockscale_g1u1(layer.a8, layer.a_scale, g["w1"], g["w1_scale"][:, :1].contiguous(), sid, seid, nv,
                                  cfg.topk, layer.block_m, layer.h8, layer.h_scale)
    with pytest.raises(ValueError):
        m.moe_down_combine(layer.h8[:-1], layer.h_scale, g["w2"], g["w2_scale"], sid, sw, seid, nv, cfg.T, cfg.topk,
                           layer.block_m)
    with pytest.raises(ValueError):
        m.gemm_fp8_blockscale(layer.a8, layer.a_scale, g["w2"][0], g["w2_scale"][0],
                              c=torch.empty((cfg.T, 8), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        m.fp8_quant_1x128(g["hidden"], scale=torch.empty((cfg.T, 1), device=DEV))
    torch.cuda.synchronize()


def test_dense_split_deterministic(m):
    from fp8_block_scaled_grouped_amd import inputs
    M, N, K = 3, 2048, 7168
    assert m.gemm_fp8_blockscale_workspace(M, N, K) > 0
    d = inputs.make_dense_inputs(M, N, K, DEV, seed=5)
    a8, sa = m.fp8_quant_1x128(d["a"])
    c1 = m.gemm_fp8_blockscale(a8, sa, d["b"], d["b_scale"]).clone()
    c2 = m.gemm_fp8_blockscale(a8, sa, d["b"], d["b_scale"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


def test_invalid_expert_id_marks_num_valid_and_gemms_skip(m, tiny):
    # an id outside [0, E) sets num_valid = -1; the grouped GEMMs then write nothing
    cfg, x = tiny
    for BM, T in [(16, cfg.T), (128, 3000)]:
        ids = np.random.default_rng(BM).integers(0, cfg.E, (T, cfg.topk)).astype(np.int32)
        ids[T // 2, 1] = cfg.E + 3
        w = np.ones((T, cfg.topk), np.float32)
        sid, sw, seid, nv = m.moe_sort(torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), cfg.E, BM)
        torch.cuda.synchronize()
        assert int(nv.item()) == -1
    g = {k: v.to(DEV) for k, v in x.items()}
    a8, sa = m.fp8_quant_1x128(g["hidden"])
    ids = np.zeros((cfg.T, cfg.topk), np.int32)
    ids[:, :] = np.arange(cfg.topk)
    ids[0, 0] = -1
    sid, sw, seid, nv = m.moe_sort(torch.from_numpy(ids).to(DEV), torch.ones((cfg.T, cfg.topk), device=DEV), cfg.E, 16)
    h8 = torch.full((sid.numel(), cfg.I), 0x5A, dtype=torch.uint8, device=DEV)
    hs = torch.full((sid.numel(), cfg.I // 128), 7.0, device=DEV)
    m.moe_fp8_blockscale_g1u1(a8, sa, g["w1"], g["w1_scale"], sid, seid, nv, cfg.topk, 16, h8, hs)
    out = torch.full((cfg.T, cfg.H), 3.0, dtype=torch.bfloat16, device=DEV)
    m.moe_down_combine(h8, hs, g["w2"], g["w2_scale"], sid, sw, seid, nv, cfg.T, cfg.topk, 16, out)
    torch.cuda.synchronize()
    assert int(nv.item()) == -1
    assert bool((h8 == 0x5A).all()) and bool((hs == 7.0).all())
    assert bool((out == 3.0).all())


@pytest.mark.parametrize("T,E,G,tg,k", [(64, 256, 8, 4, 8), (9, 96, 4, 2, 6), (4096, 256, 8, 4, 8)])
def test_topk_bf16_logits_bitexact(m, T, E, G, tg, k):
    # bf16 router logits: the oracle routes their exact fp32 values (bf16 makes ties common)
    g = torch.Generator().manual_seed(T + E)
    logits = torch.randn((T, E), generator=g).to(torch.bfloat16)
    bias = torch.randn((E,), generator=g) * 0.1
    w, ids = m.grouped_topk(logits.to(DEV), bias.to(DEV), G, tg, k, True, 2.5)
    torch.cuda.synchronize()
    wr, ir = oracle.routing.grouped_topk(logits.float().numpy(), bias.numpy(), G, tg, k, True, 2.5)
    assert np.array_equal(ids.cpu().numpy(), ir)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), wr.view(np.uint32))


@pytest.mark.parametrize("M,N,K", [(1, 2048, 7168), (37, 384, 512), (300, 256, 1024)])
def test_dense_fp16_output(m, M, N, K):
    from fp8_block_scaled_grouped_amd import inputs
    d = inputs.make_dense_inputs(M, N, K, "cpu", seed=M + 3 * N)
    a8, sa = oracle.quant.quant_1x128(f32_of_bf16(d["a"]))
    c = m.gemm_fp8_blockscale(torch.from_numpy(a8).to(DEV), torch.from_numpy(sa).to(DEV), d["b"].to(DEV),
                              d["b_scale"].to(DEV), out_dtype=torch.float16)
    cb = m.gemm_fp8_blockscale(torch.from_numpy(a8).to(DEV), torch.from_numpy(sa).to(DEV), d["b"].to(DEV),
                               d["b_scale"].to(DEV))
    torch.cuda.synchronize()
    assert c.dtype == torch.float16
    ref = oracle.gemm.gemm_blockscale(a8, sa, d["b"].numpy(), d["b_scale"].numpy())
    assert_rel_max(c.float().cpu().numpy().astype(np.float64), ref, what="dense fp16 %dx%dx%d" % (M, N, K))
    # same fp32 result rounded two ways: fp16 and bf16 agree to bf16 precision
    assert torch.allclose(c.float(), cb.float(), rtol=2 ** -7, atol=1e-3)


@pytest.mark.parametrize("seed", range(1, 9))
def test_layer_seeds_all_stages(m, seed):
    # the whole layer on fresh draws: routing, sort and quantised bytes bit-exact, h within the
    # requantisation bar, output within 1e-2 max|ref|; a mid-sized shape (E 64 in 8 groups,
    # top-6 of 3 groups, H 512, I 384) and an M tile drawn per seed
    from fp8_block_scaled_grouped_amd import inputs
    BM = [16, 32, 64, 128][seed % 4]
    T = [7, 100, 333, 1024][seed % 4]
    cfg = inputs.MoEConfig("seeds", T=T, H=512, I=384, E=64, n_group=8, topk_group=3, topk=6, block_m=BM)
    print("seed", seed, "T", T, "BM", BM, flush=True)
    x = inputs.make_moe_inputs(cfg, DEV, seed=seed)
    layer = m.MoELayer(cfg, x["bias"], x["w1"], x["w1_scale"], x["w2"], x["w2_scale"])
    out = layer.forward(x["hidden"], x["logits"])
    torch.cuda.synchronize()
    w, ids = oracle_routing(x, cfg)
    assert np.array_equal(layer.topk_ids.cpu().numpy(), ids)
    assert np.array_equal(layer.topk_w.cpu().numpy().view(np.uint32), w.view(np.uint32))
    rsid, rsw, rseid, P = oracle.sort.moe_sort(ids, w, cfg.E, BM)
    sid, sw, seid, nv = layer.sort_out
    assert int(nv.item()) == P and np.array_equal(sid[:P].cpu().numpy(), rsid)
    assert np.array_equal(seid[:P // BM].cpu().numpy(), rseid)
    a8, sa = oracle.quant.quant_1x128(f32_of_bf16(x["hidden"]))
    assert np.array_equal(np_u8(layer.a8), a8)
    assert np.array_equal(layer.a_scale.cpu().numpy().view(np.uint32), sa.view(np.uint32))
    ref, h_ref, _, _ = oracle.moe.layer_tokens(a8, sa, x["w1"].cpu().numpy(), x["w1_scale"].cpu().numpy(),
                                               x["w2"].cpu().numpy(), x["w2_scale"].cpu().numpy(), ids, w)
    assert_rel_max(f32_of_bf16(out), ref, what="seed %d layer" % seed)
    pos = {int(p): r for r, p in enumerate(rsid) if p < T * cfg.topk}
    rows = [pos[t * cfg.topk + j] for t in range(T) for j in range(cfg.topk)]
    check_requant(np_u8(layer.h8)[rows], layer.h_scale.cpu().numpy()[rows], h_ref.reshape(-1, cfg.I))


# caller-chosen tilings: every tile_m x tile_n with the same K split gives the same bits
# (each output element sums the same K blocks in the same order, whichever workgroup holds
# it), the plan gemm_fp8_blockscale picks among them; all within the oracle's tolerance.
# Shapes: ragged M and N (N off a multiple of 256 and of 128), partial K, long K
@pytest.mark.parametrize("M,N,K", [(70, 1040, 1536), (5, 2048, 7168), (130, 520, 1040), (3, 576, 16512)])
def test_dense_tiled_plans(m, M, N, K):
    from fp8_block_scaled_grouped_amd import inputs
    print("dense tiled", M, N, K, flush=True)
    d = inputs.make_dense_inputs(M, N, K, "cpu", seed=M + 11 * N + K)
    a8, sa = oracle.quant.quant_1x128(f32_of_bf16(d["a"]))
    ref = oracle.gemm.gemm_blockscale(a8, sa, d["b"].numpy(), d["b_scale"].numpy())
    args = (torch.from_numpy(a8).to(DEV), torch.from_numpy(sa).to(DEV), d["b"].to(DEV), d["b_scale"].to(DEV))
    KB = -(-K // 128)
    least = -(-KB // 128)
    outs = {}
    for sp in sorted({max(least, s) for s in (1, 3, 8)}):
        for bm in (16, 32, 64, 128):
            for bn in (128, 256):
                ws = torch.full((max(m.gemm_fp8_blockscale_tiled_workspace(M, N, K, sp), 16),), 0x7F,
                                dtype=torch.uint8, device=DEV)
                c = m.gemm_fp8_blockscale_tiled(*args, bm, bn, sp, workspace=ws)
                torch.cuda.synchronize()
                outs[(bm, bn, sp)] = c.view(torch.int16).cpu()
        first = outs[(16, 128, sp)]
        for key, v in outs.items():
            if key[2] == sp:
                assert torch.equal(v, first), key
        assert_rel_max(f32_of_bf16(first.view(torch.bfloat16)), ref, what="tiled splits %d" % sp)
    # the default plan's K split (read back from its workspace size), run as a tiling, gives
    # the default call's bits
    nws = m.gemm_fp8_blockscale_workspace(M, N, K)
    sp = (nws - 256) // (M * N * 4) if nws else 1
    c = m.gemm_fp8_blockscale(*args)
    t = m.gemm_fp8_blockscale_tiled(*args, 64, 256, sp)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), t.view(torch.int16)), sp


# The 64- and 128-row tiles run the K loop that reads the next K block's fragments during the
# current block's MFMAs; K from one block (fewer than its 3 stages) to 11 blocks covers the
# unrolled rounds and tails of every length.  Every tiling gives the same bits (the block sums
# are added in the same K order) and matches the oracle.
@pytest.mark.parametrize("K", [128, 256, 384, 512, 640, 768, 896, 1152, 1408])
def test_dense_k_steps_all_tilings(m, K):
    from fp8_block_scaled_grouped_amd import inputs
    M, N = 200, 384
    print("dense K steps", M, N, K, flush=True)
    d = inputs.make_dense_inputs(M, N, K, "cpu", seed=K)
    a8, sa = oracle.quant.quant_1x128(f32_of_bf16(d["a"]))
    ref = oracle.gemm.gemm_blockscale(a8, sa, d["b"].numpy(), d["b_scale"].numpy())
    args = (torch.from_numpy(a8).to(DEV), torch.from_numpy(sa).to(DEV), d["b"].to(DEV), d["b_scale"].to(DEV))
    outs = {}
    for bm in (16, 64, 128):
        for bn in (128, 256):
            outs[(bm, bn)] = m.gemm_fp8_blockscale_tiled(*args, bm, bn, 1).view(torch.int16).cpu()
    first = outs[(16, 128)]
    for key, v in outs.items():
        assert torch.equal(v, first), key
    assert_rel_max(f32_of_bf16(first.view(torch.bfloat16)), ref, what="dense K %d" % K)


# The grouped GEMMs over K sweeps: g1u1's K is H, down's K is I.  The layer output is the same
# bits at block_m 16 (the plain K loop) and 64 / 128 (fragments one block ahead) and matches
# the oracle.
@pytest.mark.parametrize("H,I", [(512, 128), (768, 384), (1280, 640)])
def test_layer_k_steps_all_block_m(m, H, I):
    from fp8_block_scaled_grouped_amd import inputs
    cfg = inputs.MoEConfig("ksteps", T=300, H=H, I=I, E=8, n_group=4, topk_group=2, topk=2, block_m=64)
    print("layer K steps", H, I, flush=True)
    x = inputs.make_moe_inputs(cfg, "cpu", seed=H + I)
    g = {k: v.to(DEV) for k, v in x.items()}
    outs = {}
    for BM in (16, 64, 128):
        layer = m.MoELayer(cfg, g["bias"], g["w1"], g["w1_scale"], g["w2"], g["w2_scale"], block_m=BM)
        outs[BM] = layer.forward(g["hidden"], g["logits"]).clone()
    torch.cuda.synchronize()
    for BM in (64, 128):
        assert torch.equal(outs[BM].view(torch.int16), outs[16].view(torch.int16)), BM
    w, ids = oracle_routing(x, cfg)
    a8, sa = oracle.quant.quant_1x128(f32_of_bf16(x["hidden"]))
    ref, _, _, _ = oracle.moe.layer_tokens(a8, sa, x["w1"].numpy(), x["w1_scale"].numpy(), x["w2"].numpy(),
                                           x["w2_scale"].numpy(), ids, w)
    assert_rel_max(f32_of_bf16(outs[64]), ref, what="layer H %d I %d" % (H, I))


def test_dense_tiled_rejects(m):
    from fp8_block_scaled_grouped_amd import inputs
    d = inputs.make_dense_inputs(8, 256, 16512, DEV, seed=1)
    a8, sa = m.fp8_quant_1x128(d["a"])
    with pytest.raises(RuntimeError):  # K of 129 blocks in one run: beyond the scales a workgroup holds
        m.gemm_fp8_blockscale_tiled(a8, sa, d["b"], d["b_scale"], 16, 128, 1)
    with pytest.raises(RuntimeError):  # tile shape outside the compiled set
        m.gemm_fp8_blockscale_tiled(a8, sa, d["b"], d["b_scale"], 48, 128, 2)
    with pytest.raises(RuntimeError):  # a split without workspace
        m.gemm_fp8_blockscale_tiled(a8, sa, d["b"], d["b_scale"], 16, 128, 2,
                                    workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    with pytest.raises(RuntimeError):  # 16-column tiles split K inside the workgroup only
        m.gemm_fp8_blockscale_tiled(a8, sa, d["b"], d["b_scale"], 16, 16, 2)
    with pytest.raises(RuntimeError):  # ... and take at most tile_m (<= 64) rows
        m.gemm_fp8_blockscale_tiled(a8[:8], sa[:8], d["b"], d["b_scale"], 128, 16, 1)
    torch.cuda.synchronize()


# the small-M kernel (16-column tiles, K split over the waves of a workgroup and summed
# in LDS in wave order): against the oracle, deterministic, on ragged M (1, 2 and 4
# tiles of 16 rows), N off a multiple of 16, partial and short K, K above 16,384
@pytest.mark.parametrize("M,N,K", [(1, 2048, 7168), (5, 576, 1040), (8, 1000, 4112), (37, 136, 64),
                                   (64, 4104, 7184), (17, 256, 18432), (50, 384, 512)])
@pytest.mark.parametrize("layout", ["row", "kblock"])
def test_dense_small_m_kernel(m, M, N, K, layout):
    from fp8_block_scaled_grouped_amd import inputs
    print("dense small-M", M, N, K, layout, flush=True)
    d = inputs.make_dense_inputs(M, N, K, "cpu", seed=M + 5 * N + K)
    a8, sa = oracle.quant.quant_1x128(f32_of_bf16(d["a"]))
    sa_dev = torch.from_numpy(sa if layout == "row" else np.ascontiguousarray(sa.T)).to(DEV)
    args = (torch.from_numpy(a8).to(DEV), sa_dev, d["b"].to(DEV), d["b_scale"].to(DEV))
    tm = 16 * -(-M // 16)
    tm = 64 if tm > 32 else tm
    c1 = m.gemm_fp8_blockscale_tiled(*args, tm, 16, 1, scale_layout=layout).clone()
    c2 = m.gemm_fp8_blockscale_tiled(*args, tm, 16, 1, scale_layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))
    ref = oracle.gemm.gemm_blockscale(a8, sa, d["b"].numpy(), d["b_scale"].numpy())
    assert_rel_max(f32_of_bf16(c1), ref, what="dense small-M %dx%dx%d" % (M, N, K))


# Row-major activation scales (with K blocks in whole groups of 4) go through the scale ring
# of the 64- and 128-row tiles; K-block-major scales, K splits off groups of 4 and the 16-row
# tiles keep a scale DMA per stage.  Both carry the same values, so every variant gives the
# same bits.  K of 8 to 28 blocks puts the ring's groups at every phase of the 3-step rounds.
@pytest.mark.parametrize("K", [1024, 2048, 2560, 3072, 3584])
def test_scale_ring_dense_bit_identical(m, K):
    from fp8_block_scaled_grouped_amd import inputs
    M, N = 300, 512
    print("scale ring dense", M, N, K, flush=True)
    d = inputs.make_dense_inputs(M, N, K, "cpu", seed=K + 5)
    a8, sa = oracle.quant.quant_1x128(f32_of_bf16(d["a"]))
    ref = oracle.gemm.gemm_blockscale(a8, sa, d["b"].numpy(), d["b_scale"].numpy())
    b8, bs = d["b"].to(DEV), d["b_scale"].to(DEV)
    a8d = torch.from_numpy(a8).to(DEV)
    outs = {}
    for layout in ("row", "kblock"):
        sad = torch.from_numpy(sa).to(DEV) if layout == "row" else torch.from_numpy(np.ascontiguousarray(sa.T)).to(DEV)
        for bm in (16, 64, 128):
            c = m.gemm_fp8_blockscale_tiled(a8d, sad, b8, bs, bm, 256, 1, scale_layout=layout)
            torch.cuda.synchronize()
            outs[(layout, bm)] = c.view(torch.int16).cpu()
    first = outs[("kblock", 16)]
    for key, v in outs.items():
        assert torch.equal(v, first), key
    assert_rel_max(f32_of_bf16(first.view(torch.bfloat16)), ref, what="scale ring dense K %d" % K)


# The grouped GEMMs with H and I multiples of 512 take the scale ring for row-major scales
# (gate/up: the activations' scales; down: h's scales, always row-major); with K-block-major
# activation scales gate/up keeps the per-stage scale DMA.  h and the output must agree bit for
# bit between the two, and with the oracle.
@pytest.mark.parametrize("BM", [64, 128])
def test_scale_ring_grouped_bit_identical(m, BM):
    from fp8_block_scaled_grouped_amd import inputs
    cfg = inputs.MoEConfig("ring", T=300, H=1536, I=1024, E=16, n_group=4, topk_group=2, topk=4, block_m=BM)
    print("scale ring grouped", BM, flush=True)
    x = inputs.make_moe_inputs(cfg, "cpu", seed=BM)
    g = {k: v.to(DEV) for k, v in x.items()}
    res = {}
    for layout in ("row", "kblock"):
        layer = m.MoELayer(cfg, g["bias"], g["w1"], g["w1_scale"], g["w2"], g["w2_scale"], block_m=BM,
                           scale_layout=layout)
        out = layer.forward(g["hidden"], g["logits"])
        torch.cuda.synchronize()
        # h rows of routed pairs (padding rows of a block are never written)
        nv = int(layer.sort_out[3].item())
        live = np.zeros(layer.max_sorted, bool)
        live[:nv] = layer.sort_out[0].cpu().numpy()[:nv] < cfg.T * cfg.topk
        res[layout] = (out.view(torch.int16).cpu(), np_u8(layer.h8)[live], layer.h_scale.cpu().numpy()[live])
    assert res["row"][1].shape[0] == cfg.T * cfg.topk
    assert torch.equal(res["row"][0], res["kblock"][0])
    assert np.array_equal(res["row"][1], res["kblock"][1])
    assert np.array_equal(res["row"][2], res["kblock"][2])
    w, ids = oracle_routing(x, cfg)
    a8, sa = oracle.quant.quant_1x128(f32_of_bf16(x["hidden"]))
    ref, _, _, _ = oracle.moe.layer_tokens(a8, sa, x["w1"].numpy(), x["w1_scale"].numpy(), x["w2"].numpy(),
                                           x["w2_scale"].numpy(), ids, w)
    assert_rel_max(f32_of_bf16(res["row"][0].view(torch.bfloat16)), ref, what="scale ring layer")


# The e4m3 encoder the kernels use (the hardware conversion after a clamp) equals the
# integer-op nearest-even encoder on every finite fp32 bit pattern, at every byte position of
# its packed result: the check program built with the library runs the comparison on the GPU.
def test_e4m3_encoder_exhaustive():
    import json
    import os
    import subprocess
    exe = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "fp8_block_scaled_grouped_amd",
                       "e4m3_cvt_check")
    assert os.path.exists(exe), "build the library first (python -m fp8_block_scaled_grouped_amd.build)"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    line = [x for x in r.stdout.splitlines() if x.startswith("{")][-1]
    res = json.loads(line)
    assert r.returncode == 0 and res["mismatches"] == 0, res
