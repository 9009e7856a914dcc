"""GPU parity at the full DeepSeek-V3 layer sizes (hidden 7168, intermediate 2048, 256 experts
in 8 groups, topk_group 4, top-8) and the dense GEMM shapes.

Routing, sort and quantisation are compared bit for bit (all tokens, all pairs, sampled rows
of the quantised activations).  Layer outputs are compared on every token against the
oracle's token-major evaluation of the whole layer (max|gpu - ref| <= 1e-2 * max|ref|), and the
requantised intermediate h of every routed pair against the oracle's h.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.pool import default_workers
from tests.helpers import assert_rel_max, check_requant, dense_ref, f32_of_bf16, np_u8

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
WORKERS = default_workers()  # host threads for the oracle (at most 16)


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


def _inputs(name, T=None):
    from fp8_block_scaled_grouped_amd import inputs
    cfg = {**inputs.MOE_CONFIGS, **inputs.CONTROL_CONFIGS}[name]
    if T is not None:
        cfg = inputs.with_tokens(cfg, T)
    x = inputs.make_moe_inputs(cfg, DEV, seed=0, weights=False)
    return cfg, x


@pytest.mark.parametrize("name", ["decode", "prefill", "skew", "skew_zipf", "prefill_bias0"])
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


@pytest.mark.parametrize("name", ["decode", "prefill", "skew"])
def test_quant_full_shape_bitexact(m, name):
    # every row of the hidden states, codes and scales bit for bit
    cfg, x = _inputs(name)
    q, s = m.fp8_quant_1x128(x["hidden"])
    torch.cuda.synchronize()
    qr, sr = oracle.quant.quant_1x128(f32_of_bf16(x["hidden"]), workers=WORKERS)
    assert np.array_equal(np_u8(q), qr)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), sr.view(np.uint32))


# The oracle's evaluation of a whole layer (every token, every pair), computed once per
# workload on the host's cores and shared by the tests of that workload.
_ORACLE = {}


def _oracle_layer(name, host_w):
    if name not in _ORACLE:
        _ORACLE.clear()  # one workload's results at a time (prefill: ~1.3 GB)
        cfg, x = _inputs(name)
        w, ids = oracle.routing.grouped_topk(x["logits"].cpu().numpy(), x["bias"].cpu().numpy(), cfg.n_group,
                                             cfg.topk_group, cfg.topk, cfg.renorm, cfg.routed_scaling_factor)
        a8, sa = oracle.quant.quant_1x128(f32_of_bf16(x["hidden"]), workers=WORKERS)
        ref, h_ref, h8_ref, _ = oracle.moe.layer_tokens(a8, sa, host_w["w1"], host_w["w1_scale"], host_w["w2"],
                                                        host_w["w2_scale"], ids, w, workers=WORKERS)
        _ORACLE[name] = (cfg, x, w, ids, a8, sa, ref, h_ref, h8_ref)
    return _ORACLE[name]


@pytest.fixture(scope="module")
def host_w(weights):
    return {k: v.cpu().numpy() for k, v in weights.items()}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,block_m", [("decode", 16), ("decode", 32), ("decode", 128), ("prefill", 128),
                                          ("prefill", 64), ("prefill", 256), ("skew", 128), ("skew", 64),
                                          ("skew", 256),
                                          # the routing controls: Zipf popularity without the hot bias
                                          # (255 experts, a long tail of small loads), and zero bias
                                          ("skew_zipf", 128), ("skew_zipf", 32), ("prefill_bias0", 128)])
def test_layer_all_tokens(m, weights, host_w, name, block_m):
    """The whole layer against the oracle on every token: the bf16 output of all T tokens
    (max|gpu - ref| <= 1e-2 max|ref|) and the requantised h of every routed pair."""
    print("layer", name, block_m, flush=True)
    cfg, x, w, ids, _, _, ref, h_ref, h8_ref = _oracle_layer(name, host_w)
    layer = m.MoELayer(cfg, x["bias"], weights["w1"], weights["w1_scale"], weights["w2"], weights["w2_scale"],
                       block_m=block_m)
    out = layer.forward(x["hidden"], x["logits"])
    torch.cuda.synchronize()
    assert np.array_equal(layer.topk_ids.cpu().numpy(), ids)
    err, bound = assert_rel_max(f32_of_bf16(out), ref, what="%s layer (BM %d)" % (name, block_m))
    # h of every pair, found through the sorted buffer
    sid = layer.sort_out[0].cpu().numpy()
    P = int(layer.sort_out[3].item())
    rows = np.nonzero(sid[:P] < cfg.T * cfg.topk)[0]
    pid = sid[rows]
    assert len(rows) == cfg.T * cfg.topk
    t, j = pid // cfg.topk, pid % cfg.topk
    mism = check_requant(np_u8(layer.h8)[rows], layer.h_scale.cpu().numpy()[rows], h_ref[t, j],
                         q_ref=h8_ref[t, j])
    print("%s BM %d: %d of %d tokens, %d pairs compared; max err %.3g (bound %.3g); h8 codes off %.2g" %
          (name, block_m, cfg.T, cfg.T, len(rows), err, bound, mism), flush=True)
    del layer


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,block_m", [("decode", 16), ("prefill", 128)])
def test_layer_fused_all_tokens(m, weights, host_w, name, block_m):
    """The single-launch expert computation at the V3 sizes: equal bit for bit to the
    two-call layer, and every token within the layer bar of the oracle."""
    print("layer fused", name, block_m, flush=True)
    cfg, x, w, ids, _, _, ref, _, _ = _oracle_layer(name, host_w)
    args = (cfg, x["bias"], weights["w1"], weights["w1_scale"], weights["w2"], weights["w2_scale"])
    two = m.MoELayer(*args, block_m=block_m)
    a = two.forward(x["hidden"], x["logits"]).clone()
    del two
    one = m.MoELayer(*args, block_m=block_m, fused=True)
    b = one.forward(x["hidden"], x["logits"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert_rel_max(f32_of_bf16(b), ref, what="%s fused layer (all %d tokens)" % (name, cfg.T))
    del one
    torch.cuda.empty_cache()


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


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,block_m", [("decode", 16), ("prefill", 128)])
def test_down_combine_stage(m, weights, host_w, name, block_m):
    """moe_down_combine alone on seeded random h8 / scales (inputs from the generator); every
    token compared with the oracle's down projection + combine over the sorted buffer."""
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
    ref = oracle.moe.down_combine(np_u8(h8)[:P], hs.cpu().numpy()[:P], host_w["w2"], host_w["w2_scale"], sid, sw,
                                  seid, P, cfg.T, cfg.topk, block_m, workers=WORKERS)
    assert_rel_max(f32_of_bf16(out), ref, what="down_combine %s (all %d tokens)" % (name, cfg.T))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("M,N", [(1, 2048), (1, 18432), (64, 2048), (64, 18432), (4096, 2048), (4096, 18432)])
def test_dense_full_shapes(m, M, N):
    # every row: quantised A bit for bit, C against the oracle
    from fp8_block_scaled_grouped_amd import inputs
    K = inputs.DENSE_K
    d = inputs.make_dense_inputs(M, N, K, DEV, seed=1)
    a8, sa = m.fp8_quant_1x128(d["a"])
    c = m.gemm_fp8_blockscale(a8, sa, d["b"], d["b_scale"])
    torch.cuda.synchronize()
    ar, sr = oracle.quant.quant_1x128(f32_of_bf16(d["a"]), workers=WORKERS)
    assert np.array_equal(np_u8(a8), ar)
    ref = dense_ref(ar, sr, np_u8(d["b"]), d["b_scale"].cpu().numpy(), workers=WORKERS)
    assert_rel_max(f32_of_bf16(c), ref, what="dense %dx%d (all rows)" % (M, N))


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
