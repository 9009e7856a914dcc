"""Seeded synthetic inputs for the FP8 block-scale MoE layer and the dense GEMM.

This module only draws random numbers and lays them out; it holds none of
the layer's arithmetic and is shared, as data, by the tests, the benchmark
and the CPU oracle.  Expert weights are prepared the way a checkpoint would
ship them -- fp32 draws quantised per 128x128 block with torch's own
float32 -> float8_e4m3fn cast (scale = block amax / 448, a dequantisation
multiplier) -- which is weight preparation, not part of the layer.

Workloads (sizes of DeepSeek-V3 style MoE layers):
  tiny     16 tokens, hidden 256, intermediate 128, 16 experts / 4 groups,
           topk_group 2, top-4
  decode   64 tokens, hidden 7168, intermediate 2048, 256 experts / 8 groups,
           topk_group 4, top-8
  prefill  8192 tokens, same layer
  skew     4096 tokens, same layer; logits Zipf(1.1) over experts via
           log-probability plus Gumbel noise, +3.0 correction bias on the 16
           most popular experts
  dense    A [M, 7168] bf16, B [N, 7168] e4m3 with 128x128 scales
All MoE workloads: renormalise on, routed scaling factor 2.5, hidden
~N(0,1) in bf16, logits ~N(0,1) fp32, bias ~N(0,0.1), weights ~N(0,0.02).
"""
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    H: int
    I: int
    E: int
    n_group: int
    topk_group: int
    topk: int
    renorm: bool = True
    routed_scaling_factor: float = 2.5
    block_m: int = 16
    skew: bool = False
    bias_std: float = 0.1
    hot_experts: int = 16
    hot_bias: float = 3.0
    zipf_s: float = 1.1


MOE_CONFIGS = {
    "tiny": MoEConfig("tiny", T=16, H=256, I=128, E=16, n_group=4, topk_group=2, topk=4, block_m=16),
    "decode": MoEConfig("decode", T=64, H=7168, I=2048, E=256, n_group=8, topk_group=4, topk=8, block_m=16),
    "prefill": MoEConfig("prefill", T=8192, H=7168, I=2048, E=256, n_group=8, topk_group=4, topk=8, block_m=128),
    "skew": MoEConfig("skew", T=4096, H=7168, I=2048, E=256, n_group=8, topk_group=4, topk=8, block_m=128,
                      skew=True),
}

# Labelled controls beside the workloads above: prefill with a zero correction bias
# (near-uniform routing) and the skewed workload's Zipf(1.1) popularity without the
# +3.0 bias on its 16 most popular experts.
CONTROL_CONFIGS = {
    "prefill_bias0": replace(MOE_CONFIGS["prefill"], name="prefill_bias0", bias_std=0.0),
    "skew_zipf": replace(MOE_CONFIGS["skew"], name="skew_zipf", hot_bias=0.0),
}

DENSE_K = 7168
DENSE_SHAPES = [(m, n) for m in (1, 64, 4096) for n in (2048, 18432)]

# sub-stream ids of the master seed
_S_HIDDEN, _S_LOGITS, _S_BIAS, _S_W1, _S_W2, _S_PERM, _S_GUMBEL, _S_DA, _S_DB = range(1, 10)


def with_tokens(cfg, T):
    return replace(cfg, T=T)


def _gen(device, seed, stream):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + stream)
    return g


def bf16_bits(x):
    """bf16 tensor -> its uint16 bit patterns (as int16 storage viewed)."""
    return x.contiguous().view(torch.int16)


def quantize_weight_blocks(w):
    """fp32 [..., R, C] -> (e4m3 bytes uint8 [..., R, C], fp32 scales [..., ceil(R/128), ceil(C/128)]).

    Checkpoint-style weight preparation with torch's cast (saturated to +-448);
    a last, shorter block takes the amax of the values it holds.
    """
    *lead, R, C = w.shape
    Rp, Cp = -(-R // 128) * 128, -(-C // 128) * 128
    if (Rp, Cp) != (R, C):
        w = torch.nn.functional.pad(w, (0, Cp - C, 0, Rp - R))       # zeros leave each amax as it is
    blk = w.reshape(*lead, Rp // 128, 128, Cp // 128, 128)
    amax = blk.abs().amax(dim=(-3, -1))
    scale = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
    q = (blk / scale[..., :, None, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    q = q.reshape(*lead, Rp, Cp)[..., :R, :C].contiguous()
    return q.view(torch.uint8), scale.float().contiguous()


def _expert_weights(E, R, C, device, seed, stream, std=0.02):
    g = _gen(device, seed, stream)
    q = torch.empty((E, R, C), dtype=torch.uint8, device=device)
    s = torch.empty((E, R // 128, C // 128), dtype=torch.float32, device=device)
    for e in range(E):
        w = torch.randn((R, C), generator=g, device=device, dtype=torch.float32) * std
        q[e], s[e] = quantize_weight_blocks(w)
    return q, s


def make_routing_inputs(cfg, device="cpu", seed=0):
    """(logits fp32 [T, E], bias fp32 [E])."""
    T, E = cfg.T, cfg.E
    if not cfg.skew:
        logits = torch.randn((T, E), generator=_gen(device, seed, _S_LOGITS), device=device)
        bias = torch.randn((E,), generator=_gen(device, seed, _S_BIAS), device=device) * cfg.bias_std
        return logits.float().contiguous(), bias.float().contiguous()
    # Zipf(s) popularity over a seeded ranking of the experts; Gumbel-max sampling
    # makes each token's top-1 expert Zipf-distributed.
    perm = torch.randperm(E, generator=_gen(device, seed, _S_PERM), device=device)
    rank = torch.empty(E, dtype=torch.int64, device=device)
    rank[perm] = torch.arange(1, E + 1, device=device)
    logp = -cfg.zipf_s * torch.log(rank.double())
    logp = logp - torch.logsumexp(logp, 0)
    u = torch.rand((T, E), generator=_gen(device, seed, _S_GUMBEL), device=device, dtype=torch.float64)
    u = u.clamp_min(1e-300)
    gumbel = -torch.log(-torch.log(u))
    logits = (logp[None, :] + gumbel).float().contiguous()
    bias = torch.randn((E,), generator=_gen(device, seed, _S_BIAS), device=device) * cfg.bias_std
    bias = bias + torch.where(rank <= cfg.hot_experts, cfg.hot_bias, 0.0).to(device)
    return logits, bias.float().contiguous()


def hot_expert_mask(cfg, device="cpu", seed=0):
    """Bool [E]: the experts given the extra bias in the skewed workload."""
    perm = torch.randperm(cfg.E, generator=_gen(device, seed, _S_PERM), device=device)
    rank = torch.empty(cfg.E, dtype=torch.int64, device=device)
    rank[perm] = torch.arange(1, cfg.E + 1, device=device)
    return rank <= cfg.hot_experts


def make_moe_inputs(cfg, device="cpu", seed=0, weights=True):
    """Dict of the layer's inputs on `device`.

    hidden bf16 [T, H]; logits fp32 [T, E]; bias fp32 [E];
    w1 uint8 [E, 2I, H] + w1_scale fp32 [E, 2I/128, H/128];
    w2 uint8 [E, H, I]  + w2_scale fp32 [E, H/128, I/128].
    """
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E
    hidden = torch.randn((T, H), generator=_gen(device, seed, _S_HIDDEN), device=device).to(torch.bfloat16)
    logits, bias = make_routing_inputs(cfg, device, seed)
    out = {"hidden": hidden.contiguous(), "logits": logits, "bias": bias}
    if weights:
        out["w1"], out["w1_scale"] = _expert_weights(E, 2 * I, H, device, seed, _S_W1)
        out["w2"], out["w2_scale"] = _expert_weights(E, H, I, device, seed, _S_W2)
    return out


def make_dense_inputs(M, N, K=DENSE_K, device="cpu", seed=0):
    """A bf16 [M, K] ~N(0,1); B e4m3 [N, K] with fp32 [ceil(N/128), ceil(K/128)] scales, from N(0,0.02)."""
    a = torch.randn((M, K), generator=_gen(device, seed, _S_DA), device=device).to(torch.bfloat16)
    g = _gen(device, seed, _S_DB)
    b = torch.empty((N, K), dtype=torch.uint8, device=device)
    bs = torch.empty((ceil_div(N, 128), ceil_div(K, 128)), dtype=torch.float32, device=device)
    step = 2048
    for n0 in range(0, N, step):
        w = torch.randn((min(step, N - n0), K), generator=g, device=device) * 0.02
        b[n0:n0 + w.shape[0]], bs[n0 // 128:ceil_div(n0 + w.shape[0], 128)] = quantize_weight_blocks(w)
    return {"a": a.contiguous(), "b": b, "b_scale": bs}


def moe_flops(cfg):
    """Algorithmic flops of the layer: 2 * T * k * 3 * H * I."""
    return 2.0 * cfg.T * cfg.topk * 3 * cfg.H * cfg.I


def moe_bytes(cfg, n_active):
    """Algorithmic HBM bytes: routed experts' weights and scales, hidden in, output, logits, bias."""
    H, I = cfg.H, cfg.I
    per_expert = 3 * H * I + 4 * ((2 * I // 128) * (H // 128) + (H // 128) * (I // 128))
    return n_active * per_expert + cfg.T * H * 2 * 2 + cfg.T * cfg.E * 4 + cfg.E * 4


def ceil_div(a, b):
    return -(-a // b)


__all__ = ["MoEConfig", "MOE_CONFIGS", "DENSE_SHAPES", "DENSE_K", "make_moe_inputs", "make_dense_inputs",
           "make_routing_inputs", "with_tokens", "quantize_weight_blocks", "moe_flops", "moe_bytes",
           "hot_expert_mask", "bf16_bits", "ceil_div"]
