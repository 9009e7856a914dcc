"""libmoe355: FP8 block-scale Mixture-of-Experts layer for MI355X (gfx950).

The compute lives in libmoe355.so (HIP kernels behind the C ABI declared in
include/moe355.h); `moe355` is its ctypes binding and `inputs` the seeded
synthetic workload generator.
"""
from . import inputs  # noqa: F401
from .moe355 import (  # noqa: F401
    MoELayer,
    Moe355Error,
    fp8_quant_1x128,
    gemm_fp8_blockscale,
    gemm_fp8_blockscale_plan,
    gemm_fp8_blockscale_tiled,
    gemm_fp8_blockscale_tiled_workspace,
    gemm_fp8_blockscale_workspace,
    grouped_topk,
    lib,
    moe_block_m,
    moe_down_combine,
    moe_down_combine_workspace,
    moe_fp8_blockscale_fused,
    moe_fp8_blockscale_fused_workspace,
    moe_fp8_blockscale_g1u1,
    moe_sort,
    moe_sort_sizes,
    shuffle_weight_128x128,
)
