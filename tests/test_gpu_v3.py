"""GPU parity at the full DeepSeek-V3 layer sizes (hidden 7168, intermediate 2048, 256 experts
in 8 groups, topk_group 4, top-8) and the dense GEMM shapes.

Routing, sort and quantisation are compared bit for bit (all tokens, all pairs, sampled rows
of the quantised activations).  Layer outputs are compared on sampled tokens that the
oracle evaluates one expert at a time: max|gpu - ref| <= 1e-2 * max|ref|.  Sampled tokens
always include tokens routed to the most loaded expert (the longest sorted segment).
"""
import numpy as np
import pytest
import torch

import oracle
from tests.helpers import assert_rel_max, check_requant, f32_of_bf16, np_u8

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def m():
    import fp8_block_scaled_grouped_amd as mod
    mod.lib()
    return mod


@pytest.fixture(scope="module")
def weights():
    """V3 expert weights, generated once on the GPU (shared by decode, prefill and skew)."""
    from fp8_block_scaled_grouped_amd import inputs
    cfg = inputs.MOE_CONFIGS["decode"]
    x = inputs.make_moe_inputs(cfg, DEV, seed=0)
    torch.cuda.synchronize()
    return {k: x[k] for k in ("w1", "w1_scale", "w2", "w2_scale")}


class _Rows:
    """Host copies of single experts of a device weight tensor, fetched on use."""

    def __init__(self, t):
        self.t, self.d, self.shape = t, {}, tuple(t.shape)

    def __getitem__(self, e):
        e = int(e)
        if e not in self.d:
            self.d[e] = self.t[e].cpu().numpy()
        return self.d[e]


def _inputs(name, T=None):
    from fp8_block_scaled_grouped_amd import inputs
    cfg = inputs.MOE_CONFIGS[name]
    if T is not None:
        cfg = inputs.with_tokens(cfg, T)
    x = inputs.make_moe_inputs(cfg, DEV, seed=0, weights=False)
    return cfg, x


def _sample_tokens(ids, n, seed):
    rng = np.random.default_rng(seed)
    load = np.bincount(ids.reshape(-1), minlength=ids.max() + 1)
    hot = int(load.argmax())
    hot_tok = np.nonzero((ids == hot).any(1))[0]
    pick = {int(hot_tok[0]), int(hot_tok[-1]), 0, ids.shape[0] - 1}
    while len(pick) < min(n, ids.shape[0]):
        pick.add(int(rng.integers(ids.shape[0])))
    return np.array(sorted(pick))


@pytest.mark.parametrize("name", ["decode", "prefill", "skew"])
def test_routing_and_sort_bitexact(m, name):
    cfg, x = _inputs(name)
    print("routing/sort", name, flush=True)
    k = cfg.topk
    wbuf = torch.zeros((cfg.T, k + 10), device=DEV)
    ibuf = torch.zeros((cfg.T, k + 10), dtype=torch.int32, device=DEV)
    m.grouped_topk(x["logits"], x["bias"], cfg.n_group, cfg.topk_group, k, cfg.renorm, cfg.routed_scaling_factor,
                   wbuf[:, :k], ibuf[:, :k])
    torch.cuda.synchronize()
    w, ids = oracle.routing.grouped_topk(x["logits"].cpu().numpy(), x["bias"].cpu().numpy(), cfg.n_group,
                                         cfg.topk_group, k, cfg.renorm, cfg.routed_scaling_factor)
    gi = ibuf[:, :k].cpu().numpy()
    gw = wbuf[:, :k].cpu().numpy()
    assert np.array_equal(gi, ids)
    n_diff = int((gw.view(np.uint32) != w.view(np.uint32)).sum())
    if n_diff:  # allowed only as single-ulp differences, reported
        ulp = np.abs(gw.view(np.int32).astype(np.int64) - w.view(np.int32).astype(np.int64)).max()
        print("topk_weights: %d entries differ, max %d ulp" % (n_diff, ulp))
        assert ulp <= 1
    for bm in sorted({cfg.block_m, 64, 16}):
        sid, sw, seid, nv = m.moe_sort(torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), cfg.E, bm)
        torch.cuda.synchronize()
        rsid, rsw, rseid, P = oracle.sort.moe_sort(ids, w, cfg.E, bm)
        assert int(nv.item()) == P
        assert np.array_equal(sid.cpu().numpy()[:P], rsid)
        assert np.array_equal(sw.cpu().numpy()[:P].view(np.uint32), rsw.view(np.uint32))
        assert np.array_equal(seid.cpu().numpy()[:P // bm], rseid)


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_quant_full_shape_bitexact(m, name):
    cfg, x = _inputs(name)
    q, s = m.fp8_quant_1x128(x["hidden"])
    torch.cuda.synchronize()
    rows = np.unique(np.linspace(0, cfg.T - 1, min(cfg.T, 512)).astype(int))
    qr, sr = oracle.quant.quant_1x128(f32_of_bf16(x["hidden"][torch.from_numpy(rows).to(DEV)]))
    assert np.array_equal(np_u8(q)[rows], qr)
    assert np.array_equal(s.cpu().numpy()[rows].view(np.uint32), sr.view(np.uint32))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,block_m,n_tok", [("decode", 16, 6), ("decode", 32, 3), ("prefill", 128, 4),
                                                ("prefill", 64, 3), ("skew", 128, 4)])
def test_layer_sampled_tokens(m, weights, name, block_m, n_tok):
    cfg, x = _inputs(name)
    print("layer", name, block_m, flush=True)
    layer = m.MoELayer(cfg, x["bias"], weights["w1"], weights["w1_scale"], weights["w2"], weights["w2_scale"],
                       block_m=block_m)
    out = layer.forward(x["hidden"], x["logits"])
    torch.cuda.synchronize()
    gids = layer.topk_ids.cpu().numpy()
    w, ids = oracle.routing.grouped_topk(x["logits"].cpu().numpy(), x["bias"].cpu().numpy(), cfg.n_group,
                                         cfg.topk_group, cfg.topk, cfg.renorm, cfg.routed_scaling_factor)
    assert np.array_equal(gids, ids)
    tok = _sample_tokens(ids, n_tok, seed=block_m)
    a8, sa = oracle.quant.quant_1x128(f32_of_bf16(x["hidden"][torch.from_numpy(tok).to(DEV)]))
    W1, W2 = _Rows(weights["w1"]), _Rows(weights["w2"])
    s1, s2 = weights["w1_scale"].cpu().numpy(), weights["w2_scale"].cpu().numpy()
    ref, h_ref, _, _ = oracle.moe.layer_tokens(a8, sa, W1, s1, W2, s2, ids[tok], w[tok])
    gout = f32_of_bf16(out[torch.from_numpy(tok).to(DEV)])
    assert_rel_max(gout, ref, what="%s layer (BM %d)" % (name, block_m))
    # the requantised intermediate of the sampled pairs, found through the sorted buffer
    sid = layer.sort_out[0].cpu().numpy()
    P = int(layer.sort_out[3].item())
    pos = {int(p): r for r, p in enumerate(sid[:P]) if p < cfg.T * cfg.topk}
    rows = [pos[int(t) * cfg.topk + j] for t in tok for j in range(cfg.topk)]
    h8g = np_u8(layer.h8)[rows]
    hsg = layer.h_scale.cpu().numpy()[rows]
    check_requant(h8g, hsg, h_ref.reshape(-1, cfg.I))


@pytest.mark.parametrize("name,block_m", [("decode", 16), ("prefill", 128)])
def test_layer_preshuffled_bitwise(m, weights, name, block_m):
    # the whole layer on load-time shuffled V3 weights equals the plain layer bit for bit
    cfg, x = _inputs(name)
    print("layer preshuffled", name, block_m, flush=True)
    args = (cfg, x["bias"], weights["w1"], weights["w1_scale"], weights["w2"], weights["w2_scale"])
    plain = m.MoELayer(*args, block_m=block_m)
    a = plain.forward(x["hidden"], x["logits"]).clone()
    shuf = m.MoELayer(*args, block_m=block_m, preshuffle=True)
    b = shuf.forward(x["hidden"], x["logits"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    del shuf
    torch.cuda.empty_cache()


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,block_m", [("decode", 16), ("prefill", 128)])
def test_down_combine_stage(m, weights, name, block_m):
    """moe_down_combine alone on seeded random h8 / scales (inputs from the generator)."""
    cfg, x = _inputs(name)
    w, ids = oracle.routing.grouped_topk(x["logits"].cpu().numpy(), x["bias"].cpu().numpy(), cfg.n_group,
                                         cfg.topk_group, cfg.topk, cfg.renorm, cfg.routed_scaling_factor)
    sid, sw, seid, P = oracle.sort.moe_sort(ids, w, cfg.E, block_m)
    ms, mbk, _ = m.moe_sort_sizes(cfg.T, cfg.topk, cfg.E, block_m)
    g = torch.Generator(device=DEV).manual_seed(7)
    h8 = torch.randint(0, 0x7F, (ms, cfg.I), generator=g, device=DEV, dtype=torch.uint8)
    h8 = h8 | (torch.randint(0, 2, (ms, cfg.I), generator=g, device=DEV, dtype=torch.uint8) << 7)
    hs = torch.rand((ms, cfg.I // 128), generator=g, device=DEV) * 1e-2 + 1e-3
    pad = lambda a, fill, n: torch.from_numpy(np.concatenate([a, np.full(n - len(a), fill, a.dtype)])).to(DEV)
    out = m.moe_down_combine(h8, hs, weights["w2"], weights["w2_scale"], pad(sid, cfg.T * cfg.topk, ms),
                             pad(sw, np.float32(0), ms), pad(seid, 0, mbk), torch.tensor([P], dtype=torch.int32,
                                                                                       device=DEV),
                             cfg.T, cfg.topk, block_m)
    torch.cuda.synchronize()
    tok = _sample_tokens(ids, 4, seed=1)
    pos = {int(p): r for r, p in enumerate(sid) if p < cfg.T * cfg.topk}
    h8n, hsn = np_u8(h8), hs.cpu().numpy()
    W2 = _Rows(weights["w2"])
    s2 = weights["w2_scale"].cpu().numpy()
    ref = np.zeros((len(tok), cfg.H))
    for i, t in enumerate(tok):
        for j in range(cfg.topk):
            r = pos[int(t) * cfg.topk + j]
            y = oracle.gemm.gemm_blockscale(h8n[r:r + 1], hsn[r:r + 1], W2[ids[t, j]], s2[ids[t, j]])[0]
            ref[i] += np.float64(w[t, j]) * y
    assert_rel_max(f32_of_bf16(out[torch.from_numpy(tok).to(DEV)]), ref, what="down_combine %s" % name)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("M,N", [(1, 2048), (1, 18432), (64, 2048), (64, 18432), (4096, 2048), (4096, 18432)])
def test_dense_full_shapes(m, M, N):
    from fp8_block_scaled_grouped_amd import inputs
    K = inputs.DENSE_K
    d = inputs.make_dense_inputs(M, N, K, DEV, seed=1)
    a8, sa = m.fp8_quant_1x128(d["a"])
    c = m.gemm_fp8_blockscale(a8, sa, d["b"], d["b_scale"])
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(min(M, 24)), np.linspace(0, M - 1, 8).astype(int)]))
    ar, sr = oracle.quant.quant_1x128(f32_of_bf16(d["a"][torch.from_numpy(rows).to(DEV)]))
    assert np.array_equal(np_u8(a8)[rows], ar)
    ref = oracle.gemm.gemm_blockscale(ar, sr, np_u8(d["b"]), d["b_scale"].cpu().numpy())
    assert_rel_max(f32_of_bf16(c[torch.from_numpy(rows).to(DEV)]), ref, what="dense %dx%d" % (M, N))


@pytest.mark.timeout(300)
def test_dense_largest_operand(m):
    # M*K just under 2^32: the 32-bit per-lane DMA offsets into A and the quantisation's
    # group indexing at their limit (A is 8.6 GB of bf16, 4.3 GB of e4m3)
    from fp8_block_scaled_grouped_amd import inputs
    K, N = 16384, 256
    M = (1 << 32) // K - 1
    print("dense largest", M, N, K, flush=True)
    d = inputs.make_dense_inputs(M, N, K, DEV, seed=3)
    a8, sa = m.fp8_quant_1x128(d["a"])
    c = m.gemm_fp8_blockscale(a8, sa, d["b"], d["b_scale"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 1, M // 2, M - 2, M - 1], rng.integers(0, M, 11)]))
    rt = torch.from_numpy(rows).to(DEV)
    ar, sr = oracle.quant.quant_1x128(f32_of_bf16(d["a"][rt]))
    assert np.array_equal(np_u8(a8[rt]), ar)
    assert np.array_equal(sa[rt].cpu().numpy().view(np.uint32), sr.view(np.uint32))
    ref = oracle.gemm.gemm_blockscale(ar, sr, np_u8(d["b"]), d["b_scale"].cpu().numpy())
    assert_rel_max(f32_of_bf16(c[rt]), ref, what="dense %dx%dx%d" % (M, N, K))
    del d, a8, sa, c
    torch.cuda.empty_cache()


@pytest.mark.timeout(300)
def test_grouped_gemms_largest_operand(m):
    # T*H just under 2^32 (hidden 16384, the largest the grouped calls take): the gathered A
    # rows' 32-bit DMA offsets at their limit, 17 GB of per-pair down staging
    from fp8_block_scaled_grouped_amd import inputs
    H, I = 16384, 128
    T = (1 << 32) // H - 144
    cfg = inputs.MoEConfig("largest", T=T, H=H, I=I, E=4, n_group=2, topk_group=1, topk=1, block_m=128)
    print("moe largest", T, H, I, flush=True)
    x = inputs.make_moe_inputs(cfg, DEV, seed=4)
    layer = m.MoELayer(cfg, x["bias"], x["w1"], x["w1_scale"], x["w2"], x["w2_scale"])
    out = layer.forward(x["hidden"], x["logits"])
    torch.cuda.synchronize()
    w, ids = oracle.routing.grouped_topk(x["logits"].cpu().numpy(), x["bias"].cpu().numpy(), cfg.n_group,
                                         cfg.topk_group, cfg.topk, cfg.renorm, cfg.routed_scaling_factor)
    assert np.array_equal(layer.topk_ids.cpu().numpy(), ids)
    rng = np.random.default_rng(4)
    tok = np.unique(np.concatenate([[0, T // 2, T - 2, T - 1], rng.integers(0, T, 8)]))
    tt = torch.from_numpy(tok).to(DEV)
    a8, sa = oracle.quant.quant_1x128(f32_of_bf16(x["hidden"][tt]))
    ref, _, _, _ = oracle.moe.layer_tokens(a8, sa, x["w1"].cpu().numpy(), x["w1_scale"].cpu().numpy(),
                                           x["w2"].cpu().numpy(), x["w2_scale"].cpu().numpy(), ids[tok], w[tok])
    assert_rel_max(f32_of_bf16(out[tt]), ref, what="largest grouped layer")
    del layer, x, out
    torch.cuda.empty_cache()
