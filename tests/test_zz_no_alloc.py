"""The allocation-free dense GEMM (gemm_fp8_blockscale_noalloc) against the call with
a workspace, through the C ABI: two calls in a row on one GPU, the second with a
smaller problem, each equal bit for bit to gemm_fp8_blockscale (same tiles, same
split of K, same fixed-order reduction) and within the layer bar of the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import assert_rel_max, f32_of_bf16, np_u8

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _noalloc(m, a8, sa, b8, bs, c):
    M, K = a8.shape
    N = b8.shape[0]
    st = m.lib().gemm_fp8_blockscale_noalloc(
        ctypes.c_void_p(a8.data_ptr()), ctypes.c_void_p(sa.data_ptr()), sa.shape[1], 1,
        ctypes.c_void_p(b8.data_ptr()), ctypes.c_void_p(bs.data_ptr()), M, N, K,
        ctypes.c_void_p(c.data_ptr()), c.stride(0), 0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def test_noalloc_matches_workspace_call_twice():
    import fp8_block_scaled_grouped_amd as m
    from fp8_block_scaled_grouped_amd import inputs
    # split-K shapes: 64 x 18432 (3 splits, 14 MB of partials), then 5 x 2048 (fewer bytes)
    for M, N, K, seed in [(64, 18432, 7168, 11), (5, 2048, 7168, 12)]:
        print("noalloc", M, N, K, flush=True)
        assert m.gemm_fp8_blockscale_workspace(M, N, K) > 0
        d = inputs.make_dense_inputs(M, N, K, DEV, seed=seed)
        a8, sa = m.fp8_quant_1x128(d["a"])
        ref_dev = m.gemm_fp8_blockscale(a8, sa, d["b"], d["b_scale"])  # with a workspace
        c = torch.full((M, N), -7.0, dtype=torch.bfloat16, device=DEV)
        assert _noalloc(m, a8, sa, d["b"], d["b_scale"], c) == 0
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), ref_dev.view(torch.int16))
        ref = oracle.gemm.gemm_blockscale(np_u8(a8), sa.cpu().numpy(), np_u8(d["b"]), d["b_scale"].cpu().numpy())
        assert_rel_max(f32_of_bf16(c), ref, what="noalloc dense %dx%dx%d" % (M, N, K))


def test_noalloc_rejects_beyond_its_scratch():
    import fp8_block_scaled_grouped_amd as m
    # 4096 x 7168 x 18432 always splits K: 2 x 4096 x 7168 fp32 partials (235 MB) exceed the
    # static array; nothing is launched (the pointers are never read)
    M, N, K = 4096, 7168, 18432
    assert m.gemm_fp8_blockscale_workspace(M, N, K) > (32 << 20)
    p = ctypes.c_void_p(256)
    st = m.lib().gemm_fp8_blockscale_noalloc(p, p, K // 128, 1, p, p, M, N, K, p, N, 0, None)
    assert st == -5
    assert "static scratch" in m.lib().moe355_strerror(st).decode()
