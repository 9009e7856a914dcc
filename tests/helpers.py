"""Shared helpers for the parity tests: oracle runs on CPU copies of the inputs and comparisons."""
import numpy as np
import torch

import oracle
from oracle import fp8 as ofp8


def f32_of_bf16(t):
    """bf16 torch tensor (any device) -> float32 numpy, exact."""
    return ofp8.bf16_bits_to_f32(t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def np_u8(t):
    return t.detach().cpu().contiguous().numpy().view(np.uint8)


def assert_rel_max(gpu, ref, tol=1e-2, what=""):
    """max|gpu - ref| <= tol * max|ref| (the layer-output bar)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = float(np.abs(gpu - ref).max()) if ref.size else 0.0
    bound = tol * float(np.abs(ref).max()) if ref.size else 0.0
    assert err <= bound, "%s max|gpu-ref| = %.4g > %.4g (= %g * max|ref|)" % (what, err, bound, tol)
    return err, bound


def check_requant(h8_gpu, hs_gpu, h_ref, rtol_scale=5e-3, acc_rel=1e-3, max_code_mismatch=0.05):
    """Compare a GPU 1x128 requantisation of h with the oracle's unquantised h.

    The GPU accumulates h in fp32 (different order from the binary64 oracle), so a
    code may land on the neighbouring e4m3 value.  Bound per element:
      |dec(q)*s - h| <= 2^-4 (|h| + d) + 2^-10 s + d,   d = acc_rel * amax(group)
    (half an e4m3 step at |h| plus the accumulation difference d).
    """
    R, I = h_ref.shape
    g = h_ref.reshape(R, I // 128, 128).astype(np.float64)
    amax = np.abs(g).max(-1)
    s_ref = np.where(amax == 0, 1.0, (amax.astype(np.float32) / np.float32(448.0)).astype(np.float64))
    s_gpu = np.asarray(hs_gpu, np.float64).reshape(R, I // 128)
    assert np.all(np.abs(s_gpu - s_ref) <= rtol_scale * s_ref), "h scales differ"
    deq = ofp8.decode(h8_gpu).reshape(R, I // 128, 128) * s_gpu[..., None]
    d = acc_rel * amax[..., None]
    bound = 2.0 ** -4 * (np.abs(g) + d) + 2.0 ** -10 * s_gpu[..., None] + d
    bad = np.abs(deq - g) > bound
    assert not bad.any(), "requantised h outside bound at %d elements" % int(bad.sum())
    q_ref, _ = oracle.quant.quant_1x128(h_ref.astype(np.float32))
    mism = float(np.mean(q_ref != np.asarray(h8_gpu).reshape(R, I)))
    assert mism <= max_code_mismatch, "h8 code mismatch fraction %.4f" % mism
    return mism


def oracle_routing(x, cfg):
    return oracle.routing.grouped_topk(x["logits"].cpu().numpy(), x["bias"].cpu().numpy(), cfg.n_group,
                                       cfg.topk_group, cfg.topk, cfg.renorm, cfg.routed_scaling_factor)
