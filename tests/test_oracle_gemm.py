"""Pins of the oracle's block-scaled FP8 GEMM."""
import numpy as np
import torch

from oracle import fp8, gemm


def _codes(rng, shape):
    c = rng.integers(0, 0x7F, size=shape).astype(np.uint8)       # finite magnitudes
    return c | (rng.integers(0, 2, size=shape).astype(np.uint8) << 7)


def test_block_sums_exact_against_integers(rng):
    a = _codes(rng, (9, 384))
    b = _codes(rng, (128, 384))
    bs = gemm.block_sums(a, b)
    ai = np.rint(fp8.decode(a) * 512).astype(np.int64)               # e4m3 * 2^9 is an integer
    bi = np.rint(fp8.decode(b) * 512).astype(np.int64)
    for kb in range(3):
        exact = ai[:, kb * 128:(kb + 1) * 128] @ bi[:, kb * 128:(kb + 1) * 128].T
        assert np.array_equal(bs[kb], exact.astype(np.float64) / 2.0 ** 18)


def test_identity_weight_reproduces_input(rng):
    K = 256
    a = _codes(rng, (5, K))
    b = np.zeros((K, K), np.uint8)
    b[np.arange(K), np.arange(K)] = 0x38                             # 1.0 on the diagonal
    out = gemm.gemm_blockscale(a, np.ones((5, 2), np.float32), b, np.ones((2, 2), np.float32))
    assert np.array_equal(out, fp8.decode(a))


def test_against_dequantised_torch_matmul(rng):
    M, N, K = 7, 256, 512
    a = _codes(rng, (M, K)) & 0xF7
    b = _codes(rng, (N, K)) & 0xF7
    sa = rng.random((M, K // 128)).astype(np.float32) + 0.1
    sb = rng.random((N // 128, K // 128)).astype(np.float32) + 0.1
    out = gemm.gemm_blockscale(a, sa, b, sb)
    A = torch.from_numpy(fp8.decode(a) * np.repeat(sa.astype(np.float64), 128, axis=1))
    B = torch.from_numpy(fp8.decode(b) * np.repeat(np.repeat(sb.astype(np.float64), 128, 0), 128, 1))
    ref = (A @ B.T).numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_partial_blocks_brute_force(rng):
    # K and N not multiples of 128: element-by-element sum with the scale of each k's block
    M, N, K = 3, 136, 144
    a = _codes(rng, (M, K)) & 0xF7
    b = _codes(rng, (N, K)) & 0xF7
    sa = (rng.random((M, 2)) + 0.5).astype(np.float32)
    sb = (rng.random((2, 2)) + 0.5).astype(np.float32)
    out = gemm.gemm_blockscale(a, sa, b, sb)
    A, B = fp8.decode(a).tolist(), fp8.decode(b).tolist()
    sal, sbl = sa.astype(np.float64).tolist(), sb.astype(np.float64).tolist()
    for m in range(M):
        for n in range(N):
            ref = sum(sal[m][k // 128] * sbl[n // 128][k // 128] * A[m][k] * B[n][k] for k in range(K))
            assert abs(out[m, n] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_partial_blocks_equal_zero_padded_problem(rng):
    # zero codes appended along K (and rows along N) change no block sum: the padded
    # problem's leading N columns reproduce the partial one bit for bit
    M, N, K = 5, 200, 328
    a = _codes(rng, (M, K)) & 0xF7
    b = _codes(rng, (N, K)) & 0xF7
    sa = (rng.random((M, 3)) + 0.5).astype(np.float32)
    sb = (rng.random((2, 3)) + 0.5).astype(np.float32)
    out = gemm.gemm_blockscale(a, sa, b, sb)
    ap = np.zeros((M, 384), np.uint8)
    ap[:, :K] = a
    bp = np.zeros((256, 384), np.uint8)
    bp[:N, :K] = b
    full = gemm.gemm_blockscale(ap, sa, bp, sb)
    assert np.array_equal(out, full[:, :N])
    assert np.array_equal(gemm.block_sums(a, b), gemm.block_sums(ap, bp)[:, :, :N])


def test_column_blocked_reference_equals_one_call():
    # the parity tests evaluate large dense products in column blocks on a thread pool;
    # every element must equal the single oracle call bit for bit
    from tests.helpers import dense_ref
    rng = np.random.default_rng(5)
    a8 = rng.integers(0, 0x7E, (7, 400), dtype=np.uint8)
    sa = rng.random((7, 4), dtype=np.float32)
    b8 = rng.integers(0, 0x7E, (600, 400), dtype=np.uint8)
    sb = rng.random((5, 4), dtype=np.float32)
    one = gemm.gemm_blockscale(a8, sa, b8, sb)
    assert np.array_equal(dense_ref(a8, sa, b8, sb, workers=3, cols=256), one)
