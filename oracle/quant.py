"""Dynamic 1x128 FP8 quantisation (CPU oracle; test infrastructure only).

"Accelerate DeepSeek-R1 Inference: Integrate AITER into SGLang", section
"General Linear Layer": every 1x128 run of an activation row carries one
scale; section "Blockscale FP8 MoE Computation" (asm_moe) quantises the
bf16 hidden states viewed as rows of 128 with one scale per row.

Reading taken for the steps the page leaves open, per group x[0..127]:
  amax  = max |x_i|                           (exact)
  scale = 1.0 if amax == 0 else fl32(amax / 448)   (IEEE fp32 division)
  q_i   = encode(fl32(x_i / scale))           (IEEE fp32 division, RNE,
                                               saturating, sign kept)
The scale is a dequantisation multiplier: value = decode(q) * scale.
When K is not a multiple of 128 the last group of a row holds the remaining
K mod 128 values (ceil(K/128) scales per row, as the pages size them).
"""
import numpy as np

from . import fp8, pool

GROUP = 128


def quant_1x128(x, workers=1):
    """x: float32 [M, K] -> (q uint8 [M, K], scale float32 [M, ceil(K/128)]).

    workers > 1 quantises blocks of rows on a thread pool (rows are independent)."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    if workers > 1 and M > 256:
        q = np.zeros((M, K), dtype=np.uint8)
        scale = np.ones((M, -(-K // GROUP)), dtype=np.float32)

        def rows(r0, r1):
            q[r0:r1], scale[r0:r1] = quant_1x128(x[r0:r1])

        pool.run([lambda a=a, b=b: rows(a, b) for a, b in pool.row_chunks(M, 256)], workers)
        return q, scale
    KB = -(-K // GROUP)
    q = np.zeros((M, K), dtype=np.uint8)
    scale = np.ones((M, KB), dtype=np.float32)
    for kb in range(KB):
        g = x[:, kb * GROUP:(kb + 1) * GROUP]                               # the last may be shorter
        amax = np.max(np.abs(g), axis=1)                                     # float32, exact
        s = np.divide(amax, np.float32(fp8.E4M3_MAX), dtype=np.float32)    # fl32(amax/448)
        s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
        q[:, kb * GROUP:(kb + 1) * GROUP] = fp8.encode(np.divide(g, s[:, None], dtype=np.float32))
        scale[:, kb] = s
    return q, scale


def dequant_1x128(q, scale):
    """decode(q) * scale per 1x128 group, binary64."""
    q = np.asarray(q, dtype=np.uint8)
    M, K = q.shape
    s = np.repeat(np.asarray(scale, dtype=np.float64), GROUP, axis=1)[:, :K]
    return fp8.decode(q) * s
