"""Guard bands: every call writes only inside the buffers it is given.

Each output and workspace buffer sits inside a larger allocation filled with a
canary byte; after the call the bytes before and after it (and the padding
columns of row-strided outputs) must still hold the canary.  Shapes cover
every M tile, ragged last tiles, strided top-k outputs and partial dense blocks.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
G = 4096          # guard bytes on each side
CANARY = 0xA5


@pytest.fixture(scope="module")
def m():
    import fp8_block_scaled_grouped_amd as mod
    mod.lib()
    return mod


class Guarded:
    """A tensor view inside a canary-filled allocation."""

    def __init__(self, shape, dtype):
        self.n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.base = torch.full((self.n + 2 * G,), CANARY, dtype=torch.uint8, device=DEV)
        self.t = self.base[G:G + self.n].view(dtype).view(shape)

    def intact(self):
        return bool((self.base[:G] == CANARY).all()) and bool((self.base[G + self.n:] == CANARY).all())


def _bytes_canary(t):
    return bool((t.contiguous().view(torch.uint8) == CANARY).all())


def _medium_cfg(T):
    from fp8_block_scaled_grouped_amd import inputs
    return inputs.MoEConfig("guard", T=T, H=512, I=256, E=32, n_group=4, topk_group=2, topk=6)


@pytest.mark.parametrize("T,BM", [(16, 16), (300, 16), (300, 32), (300, 64), (1000, 128), (1, 128)])
def test_layer_calls_stay_inside_their_buffers(m, T, BM):
    from fp8_block_scaled_grouped_amd import inputs
    cfg = _medium_cfg(T)
    print("guard layer", T, BM, flush=True)
    x = inputs.make_moe_inputs(cfg, DEV, seed=T + BM)
    k, H, I, E = cfg.topk, cfg.H, cfg.I, cfg.E
    # top-k into row-strided outputs (3 padding columns per row)
    tw, ti = Guarded((T, k + 3), torch.float32), Guarded((T, k + 3), torch.int32)
    m.grouped_topk(x["logits"], x["bias"], cfg.n_group, cfg.topk_group, k, True, 2.5, tw.t[:, :k], ti.t[:, :k])
    ms, mb, wsb = m.moe_sort_sizes(T, k, E, BM)
    sid, sw = Guarded((ms,), torch.int32), Guarded((ms,), torch.float32)
    seid, nv = Guarded((mb,), torch.int32), Guarded((1,), torch.int32)
    sws = Guarded((max(wsb, 1),), torch.uint8)
    ids_c, w_c = ti.t[:, :k].contiguous(), tw.t[:, :k].contiguous()
    m.moe_sort(ids_c, w_c, E, BM, (sid.t, sw.t, seid.t, nv.t), sws.t[:wsb] if wsb else sws.t[:1])
    a8, sa = Guarded((T, H), torch.uint8), Guarded((T, H // 128), torch.float32)
    m.fp8_quant_1x128(x["hidden"], a8.t, sa.t)
    h8, hs = Guarded((ms, I), torch.uint8), Guarded((ms, I // 128), torch.float32)
    m.moe_fp8_blockscale_g1u1(a8.t, sa.t, x["w1"], x["w1_scale"], sid.t, seid.t, nv.t, k, BM, h8.t, hs.t)
    out = Guarded((T, H), torch.bfloat16)
    dws = Guarded((m.moe_down_combine_workspace(T, H, k),), torch.uint8)
    m.moe_down_combine(h8.t, hs.t, x["w2"], x["w2_scale"], sid.t, sw.t, seid.t, nv.t, T, k, BM, out.t, dws.t)
    torch.cuda.synchronize()
    for name, gbuf in [("topk_weights", tw), ("topk_ids", ti), ("sorted_ids", sid), ("sorted_weights", sw),
                       ("sorted_expert_ids", seid), ("num_valid", nv), ("sort workspace", sws), ("a8", a8),
                       ("a_scale", sa), ("h8", h8), ("h_scale", hs), ("out", out), ("down workspace", dws)]:
        assert gbuf.intact(), name
    assert _bytes_canary(tw.t[:, k:]) and _bytes_canary(ti.t[:, k:]), "top-k padding columns"
    assert int(nv.t.item()) > 0


@pytest.mark.parametrize("M,N,K", [(1, 2048, 7168), (37, 200, 208), (130, 520, 400), (64, 4104, 7184),
                                   (300, 256, 1024)])
@pytest.mark.parametrize("split", [True, False], ids=["ws", "nows"])
def test_dense_stays_inside_its_buffers(m, M, N, K, split):
    from fp8_block_scaled_grouped_amd import inputs
    print("guard dense", M, N, K, split, flush=True)
    d = inputs.make_dense_inputs(M, N, K, DEV, seed=M + N)
    a8, sa = Guarded((M, K), torch.uint8), Guarded((M, -(-K // 128)), torch.float32)
    m.fp8_quant_1x128(d["a"], a8.t, sa.t)
    c = Guarded((M, N + 8), torch.bfloat16)          # 8 padding columns per row
    nws = m.gemm_fp8_blockscale_workspace(M, N, K)
    ws = Guarded((max(nws, 16),), torch.uint8)
    m.gemm_fp8_blockscale(a8.t, sa.t, d["b"], d["b_scale"], c=c.t[:, :N], workspace=ws.t[:nws] if (split and nws)
                          else False)
    torch.cuda.synchronize()
    for name, gbuf in [("a8", a8), ("a_scale", sa), ("c", c), ("workspace", ws)]:
        assert gbuf.intact(), name
    assert _bytes_canary(c.t[:, N:]), "c padding columns"
    if not (split and nws):
        assert _bytes_canary(ws.t), "workspace untouched without split-K"


def test_shuffle_stays_inside_its_buffer(m):
    w = torch.randint(0, 256, (2, 256, 384), dtype=torch.uint8, device=DEV)
    out = Guarded((2, 256, 384), torch.uint8)
    m.shuffle_weight_128x128(w, out=out.t)
    torch.cuda.synchronize()
    assert out.intact()
