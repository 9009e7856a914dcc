"""Plain CPU oracle for the FP8 block-scale Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant with the HIP library; the two meet only through the seeded input
generator, which holds none of the method's arithmetic.

What it computes follows "Accelerate DeepSeek-R1 Inference: Integrate AITER
into SGLang" (rocm.blogs.amd.com), section "Complete MoE Implementation"
(Top-K routing, MoE Sorting, Blockscale FP8 MoE Computation) and section
"General Linear Layer", with the FP8 format fixed to OCP E4M3 (e4m3fn,
largest finite 448).  Floating point is accumulated in binary64 with exact
FP8 decode; every place where the pages leave a step open takes the reading
written in the docstring of the function concerned.

Modules
-------
fp8      exact e4m3fn decode / nearest-even saturating encode
quant    dynamic 1x128 activation quantisation
routing  biased grouped top-k
sort     per-expert bucketing padded to the M tile
gemm     block-scaled FP8 GEMM (exact 128-term block sums, binary64)
moe      gate/up + SiLU*up + requantisation, down projection + combine,
         and a token-major evaluation of the whole layer
layout   the pre-shuffled 128x128-tile weight layout (a byte permutation)
pool     runs independent pieces (experts, blocks of rows) on host threads
"""
from . import fp8, pool, quant, routing, sort, gemm, moe, layout  # noqa: F401
