"""Block-scaled FP8 GEMM (CPU oracle; test infrastructure only).

"Accelerate DeepSeek-R1 Inference: Integrate AITER into SGLang", section
"General Linear Layer": Y[m, n] from XQ [M, K] (e4m3, one scale per 1x128
of a row) and WQ [N, K] (e4m3, one scale per 128x128 block), with
scale_n = ceil(N/128) and scale_k = ceil(K/128).

  ref[m, n] = sum_kb  sa[m, kb] * sb[n // 128, kb] * sum_{k in kb} dec(a[m, k]) * dec(b[n, k])

in binary64.  Each 128-term block sum is exact in binary64 in any order:
an e4m3 value is a multiple of 2^-9 of magnitude <= 448, so a product is
a multiple of 2^-18 below 2^18 and a 128-term sum stays below 2^25, which
needs at most 43 significant bits.  The block sums are therefore taken with
a library matrix product (numpy), the scaled sum over kb in ascending kb.
Scales are dequantisation multipliers (the pages call the weight scales
scale_inv).  K and N are multiples of 128 here.
"""
import numpy as np

from . import fp8

BLK = 128


def block_sums(a8, b8):
    """Exact per-128-K block sums: float64 [KB, M, N]."""
    A = fp8.decode(a8)
    B = fp8.decode(b8)
    M, K = A.shape
    N = B.shape[0]
    KB = K // BLK
    out = np.empty((KB, M, N), dtype=np.float64)
    for kb in range(KB):
        out[kb] = A[:, kb * BLK:(kb + 1) * BLK] @ B[:, kb * BLK:(kb + 1) * BLK].T
    return out


def gemm_blockscale(a8, a_scale, b8, b_scale):
    """a8 uint8 [M, K], a_scale float32 [M, K/128], b8 uint8 [N, K], b_scale float32 [N/128, K/128] -> float64 [M, N]."""
    a8 = np.asarray(a8, dtype=np.uint8)
    b8 = np.asarray(b8, dtype=np.uint8)
    M, K = a8.shape
    N = b8.shape[0]
    assert K % BLK == 0 and N % BLK == 0 and b8.shape[1] == K
    sa = np.asarray(a_scale, dtype=np.float64).reshape(M, K // BLK)
    sb = np.asarray(b_scale, dtype=np.float64).reshape(N // BLK, K // BLK)
    sbn = np.repeat(sb, BLK, axis=0)                    # [N, KB]: scale of column n
    A = fp8.decode(a8)
    B = fp8.decode(b8)
    out = np.zeros((M, N), dtype=np.float64)
    for kb in range(K // BLK):
        part = A[:, kb * BLK:(kb + 1) * BLK] @ B[:, kb * BLK:(kb + 1) * BLK].T
        out += (sa[:, kb:kb + 1] * sbn[None, :, kb]) * part
    return out
