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


def check_requant(h8_gpu, hs_gpu, h_ref, rtol_scale=1e-4, acc_rel=1e-4, max_code_mismatch=1e-2, q_ref=None,
                  chunk=4096, rtol_scale_all=1e-3, max_scale_outliers=1e-5):
    """Compare a GPU 1x128 requantisation of h with the oracle's unquantised h.

    The GPU accumulates h in fp32 (different order from the binary64 oracle) and
    evaluates SiLU with the hardware exponential, so h differs from the oracle's
    by about 1e-6 of the group's amax; a code may then land on the neighbouring e4m3
    value when h sits next to a rounding midpoint.  Bounds:
      scale:   |s_gpu - s_ref| <= rtol_scale * s_ref for all but a fraction
               max_scale_outliers of the groups (a group whose amax comes out of a
               cancelling sum carries a larger relative error), rtol_scale_all for all
      element: |dec(q)*s - h| <= 2^-4 (|h| + d) + 2^-10 s + d,  d = acc_rel * amax(group)
               (half an e4m3 step at |h|, the subnormal step, and the h difference d)
      codes:   at most max_code_mismatch of them differ from the oracle's own codes
               (random differences of 1e-6 amax in h move ~0.2% of the codes, 5e-6 amax ~0.8%;
               an error proportional to |h| of 1e-3 moves ~1.1%; an error of the scale moves
               none and is caught by the scale bound)
    q_ref: the oracle's codes of h_ref if already computed.  Rows are checked in chunks.
    Returns the fraction of codes that differ.
    """
    R, I = h_ref.shape
    h8_gpu = np.asarray(h8_gpu).reshape(R, I)
    s_all = np.asarray(hs_gpu, np.float64).reshape(R, I // 128)
    n_mism = n_out = 0
    for r0 in range(0, R, chunk):
        r1 = min(R, r0 + chunk)
        g = h_ref[r0:r1].reshape(r1 - r0, I // 128, 128).astype(np.float64)
        amax = np.abs(g).max(-1)
        s_ref = np.where(amax == 0, 1.0, (amax.astype(np.float32) / np.float32(448.0)).astype(np.float64))
        s_gpu = s_all[r0:r1]
        rel = np.abs(s_gpu - s_ref) / s_ref
        assert not (rel > rtol_scale_all).any(), "h scales differ at %d groups (max rel %.3g)" % (
            int((rel > rtol_scale_all).sum()), float(rel.max()))
        n_out += int(np.count_nonzero(rel > rtol_scale))
        deq = ofp8.decode(h8_gpu[r0:r1]).reshape(r1 - r0, I // 128, 128) * s_gpu[..., None]
        d = acc_rel * amax[..., None]
        bound = 2.0 ** -4 * (np.abs(g) + d) + 2.0 ** -10 * s_gpu[..., None] + d
        bad = np.abs(deq - g) > bound
        assert not bad.any(), "requantised h outside bound at %d elements" % int(bad.sum())
        qr = oracle.quant.quant_1x128(h_ref[r0:r1].astype(np.float32))[0] if q_ref is None else q_ref[r0:r1]
        n_mism += int(np.count_nonzero(np.asarray(qr).reshape(r1 - r0, I) != h8_gpu[r0:r1]))
    assert n_out <= max_scale_outliers * R * (I // 128), "h scales beyond %g relative at %d of %d groups" % (
        rtol_scale, n_out, R * (I // 128))
    mism = n_mism / float(max(1, R * I))
    assert mism <= max_code_mismatch, "h8 code mismatch fraction %.5f" % mism
    return mism


def dense_ref(a8, a_scale, b8, b_scale, workers=1, cols=1152):
    """oracle.gemm.gemm_blockscale over column blocks of `cols` (a multiple of 128) on a
    thread pool: each piece takes its own weight rows and their scale rows, so every
    output element is computed exactly as in one call."""
    from oracle import pool
    M, N = a8.shape[0], b8.shape[0]
    out = np.zeros((M, N), np.float64)

    def piece(n0, n1):
        out[:, n0:n1] = oracle.gemm.gemm_blockscale(a8, a_scale, b8[n0:n1], b_scale[n0 // 128:-(-n1 // 128)])

    pool.run([lambda a=a, b=b: piece(a, b) for a, b in pool.row_chunks(N, cols)], workers)
    return out


def oracle_routing(x, cfg):
    return oracle.routing.grouped_topk(x["logits"].cpu().numpy(), x["bias"].cpu().numpy(), cfg.n_group,
                                       cfg.topk_group, cfg.topk, cfg.renorm, cfg.routed_scaling_factor)
