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
scale_inv).  K and N need not be multiples of 128: block kb covers
k in [128 kb, min(K, 128 kb + 128)) and scale row n // 128 serves the last,
shorter column block, as the ceil-sized scale arrays imply.
"""
import numpy as np

from . import fp8

BLK = 128


def nblocks(n):
    """ceil(n / 128): scale entries along a dimension of n."""
    return -(-n // BLK)


def block_sums(a8, b8):
    """Exact per-128-K block sums: float64 [ceil(K/128), M, N]."""
    A = fp8.decode(a8)
    B = fp8.decode(b8)
    M, K = A.shape
    N = B.shape[0]
    KB = nblocks(K)
    out = np.empty((KB, M, N), dtype=np.float64)
    for kb in range(KB):
        ks = slice(kb * BLK, min(K, (kb + 1) * BLK))
        out[kb] = A[:, ks] @ B[:, ks].T
    return out


def gemm_blockscale(a8, a_scale, b8, b_scale):
    """a8 uint8 [M, K], a_scale float32 [M, ceil(K/128)], b8 uint8 [N, K],
    b_scale float32 [ceil(N/128), ceil(K/128)] -> float64 [M, N]."""
    a8 = np.asarray(a8, dtype=np.uint8)
    b8 = np.asarray(b8, dtype=np.uint8)
    M, K = a8.shape
    N = b8.shape[0]
    assert b8.shape[1] == K
    KB, NB = nblocks(K), nblocks(N)
    sa = np.asarray(a_scale, dtype=np.float64).reshape(M, KB)
    sb = np.asarray(b_scale, dtype=np.float64).reshape(NB, KB)
    sbn = np.repeat(sb, BLK, axis=0)[:N]                 # [N, KB]: scale of column n
    A = fp8.decode(a8)
    B = fp8.decode(b8)
    out = np.zeros((M, N), dtype=np.float64)
    for kb in range(KB):
        ks = slice(kb * BLK, min(K, (kb + 1) * BLK))
        part = A[:, ks] @ B[:, ks].T
        out += (sa[:, kb:kb + 1] * sbn[None, :, kb]) * part
    return out
