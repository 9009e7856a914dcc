"""Host-side checks of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments with the documented codes before touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe355.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", txt, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    from fp8_block_scaled_grouped_amd import moe355
    if not os.path.exists(moe355.LIB_PATH):
        pytest.skip("libmoe355.so not built")
    return moe355.lib()


def test_header_declares_the_six_calls():
    d = _declared()
    for name in ["grouped_topk", "moe_sort", "fp8_quant_1x128", "moe_fp8_blockscale_g1u1", "moe_down_combine",
                 "gemm_fp8_blockscale", "gemm_fp8_blockscale_workspace", "moe_sort_sizes", "moe_down_combine_workspace", "moe355_strerror"]:
        assert name in d, name


def test_every_declared_symbol_exported(lib):
    from fp8_block_scaled_grouped_amd import moe355
    for name in _declared():
        assert hasattr(lib, name), name
        assert name in moe355.EXPORTED, name


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4, -5, -99):
        assert lib.moe355_strerror(code).decode().startswith("moe355:")


def test_sort_sizes(lib):
    from fp8_block_scaled_grouped_amd import moe355
    import oracle
    for T, k, E, BM in [(16, 4, 16, 16), (64, 8, 256, 16), (8192, 8, 256, 128), (4096, 8, 256, 64), (0, 8, 256, 32),
                        (8192, 8, 256, 256)]:
        ms, mb, ws = moe355.moe_sort_sizes(T, k, E, BM)
        assert (ms, mb) == oracle.sort.max_sizes(T, k, E, BM)
        assert ws > 0
    with pytest.raises(moe355.Moe355Error) as e:
        moe355.moe_sort_sizes(16, 4, 16, 48)
    assert e.value.code == -2


def _p(v=16):
    return ctypes.c_void_p(v)


def test_invalid_arguments_return_codes(lib):
    L = lib
    # grouped_topk: E % n_group != 0 -> EUNSUPPORTED; ld_topk < topk -> EINVAL; null -> EINVAL
    assert L.grouped_topk(_p(), 0, 16, _p(), 4, 16, 3, 2, 4, 1, 1.0, _p(), _p(), 4, None) == -2
    assert L.grouped_topk(_p(), 0, 16, _p(), 4, 16, 4, 2, 4, 1, 1.0, _p(), _p(), 3, None) == -1
    assert L.grouped_topk(None, 0, 16, _p(), 4, 16, 4, 2, 4, 1, 1.0, _p(), _p(), 4, None) == -1
    assert L.grouped_topk(_p(), 0, 16, _p(), 4, 16, 4, 2, 9, 1, 1.0, _p(), _p(), 9, None) == -2   # topk > tg*E/G
    assert L.grouped_topk(_p(), 0, 16, _p(), 0, 16, 4, 2, 4, 1, 1.0, None, None, 4, None) == 0    # T = 0 no-op
    # quant: K % 8 -> EUNSUPPORTED; misaligned -> EMISALIGNED; ld < K -> EINVAL
    assert L.fp8_quant_1x128(_p(), 204, 4, 204, _p(), 208, _p(), 2, 1, None) == -2
    assert L.fp8_quant_1x128(_p(8), 256, 4, 256, _p(), 256, _p(), 2, 1, None) == -3
    assert L.fp8_quant_1x128(_p(), 256, 4, 256, _p(), 260, _p(), 2, 1, None) == -3
    assert L.fp8_quant_1x128(_p(), 128, 4, 256, _p(), 256, _p(), 2, 1, None) == -1
    # dense GEMM: N % 8 or K % 16 -> EUNSUPPORTED; ldc < N -> EINVAL
    assert L.gemm_fp8_blockscale(_p(), _p(), 2, 1, _p(), _p(), 4, 100, 256, _p(), 104, 0, None, 0, None) == -2
    assert L.gemm_fp8_blockscale(_p(), _p(), 2, 1, _p(), _p(), 4, 128, 200, _p(), 128, 0, None, 0, None) == -2
    assert L.gemm_fp8_blockscale(_p(), _p(), 2, 1, _p(), _p(), 4, 128, 256, _p(), 120, 0, None, 0, None) == -1
    # K above 16384 needs the split-K workspace: none -> EUNSUPPORTED, too little -> EINVAL
    assert L.gemm_fp8_blockscale(_p(), _p(), 2, 1, _p(), _p(), 300, 256, 18432, _p(), 256, 0, None, 0, None) == -2
    assert L.gemm_fp8_blockscale(_p(), _p(), 2, 1, _p(), _p(), 300, 256, 18432, _p(), 256, 0, _p(), 64, None) == -1
    assert L.gemm_fp8_blockscale(_p(), _p(), 2, 1, _p(), _p(), 4, 128, 256, _p(), 64, 0, None, 0, None) == -1
    # output type flag must be 0 or 1; logits type flag likewise
    assert L.gemm_fp8_blockscale(_p(), _p(), 2, 1, _p(), _p(), 4, 128, 256, _p(), 128, 2, None, 0, None) == -1
    assert L.grouped_topk(_p(), 2, 16, _p(), 4, 16, 4, 2, 4, 1, 1.0, _p(), _p(), 4, None) == -1
    # sort: workspace too small -> EINVAL; bad block_m -> EUNSUPPORTED
    assert L.moe_sort(_p(), _p(), 4, 16, 4, 16, 16, _p(), _p(), _p(), _p(), _p(), 1, None) == -1
    assert L.moe_sort(_p(), _p(), 4, 16, 4, 16, 24, _p(), _p(), _p(), _p(), _p(), 1 << 20, None) == -2
    # g1u1: capacity below the worst case -> EINVAL; I % 128 -> EUNSUPPORTED
    assert L.moe_fp8_blockscale_g1u1(_p(), _p(), 2, 1, _p(), _p(), _p(), _p(), _p(), 16, 256, 128, 16, 4, 16, 100,
                                     _p(), _p(), None, None) == -1
    assert L.moe_fp8_blockscale_g1u1(_p(), _p(), 2, 1, _p(), _p(), _p(), _p(), _p(), 16, 256, 100, 16, 4, 16, 304,
                                     _p(), _p(), None, None) == -2
    # weight shuffle: rows or K off multiples of 128 -> EUNSUPPORTED; out overlapping w -> EINVAL
    assert L.shuffle_weight_128x128(_p(), 100, 128, _p(1 << 20), None) == -2
    assert L.shuffle_weight_128x128(_p(), 128, 200, _p(1 << 20), None) == -2
    assert L.shuffle_weight_128x128(_p(1 << 20), 128, 128, _p((1 << 20) + 4096), None) == -1
    assert L.shuffle_weight_128x128(None, 0, 128, None, None) == 0
    # pre-shuffled dense weights need whole 128x128 tiles
    assert L.gemm_fp8_blockscale_wpreshuffle(_p(), _p(), 2, 1, _p(), _p(), 4, 136, 256, _p(), 136, 0, None, 0,
                                             None) == -2
    # A-scale row strides whose byte offset of the last row reaches 2^32 -> EUNSUPPORTED
    # (the scale DMA takes a 32-bit offset per row): dense M 4096 with sstride_m 2^18,
    # g1u1 T 16 with sstride_m 2^26; one element less is accepted as far as the checks go
    assert L.gemm_fp8_blockscale(_p(), _p(), 1 << 18, 1, _p(), _p(), 4096, 128, 256, _p(), 128, 0, None, 0,
                                 None) == -2
    assert L.moe_fp8_blockscale_g1u1(_p(), _p(), 1 << 26, 1, _p(), _p(), _p(), _p(), _p(), 16, 256, 128, 16, 4, 16,
                                     304, _p(), _p(), None, None) == -2
    assert L.moe_fp8_blockscale_g1u1(_p(), _p(), 1 << 26, 1, _p(), _p(), _p(), _p(), _p(), 16, 256, 128, 16, 4, 16,
                                     304, _p(8), _p(), None, None) == -2
    # the allocation-free dense GEMM: split-K partials beyond its static array -> ESCRATCH
    # (4096 x 7168 x 18432 always splits K: 235 MB of partials); shape rules as the plain call
    assert L.gemm_fp8_blockscale_noalloc(_p(), _p(), 144, 1, _p(), _p(), 4096, 7168, 18432, _p(), 7168, 0,
                                         None) == -5
    assert L.gemm_fp8_blockscale_noalloc(_p(), _p(), 2, 1, _p(), _p(), 4, 100, 256, _p(), 104, 0, None) == -2
    assert L.gemm_fp8_blockscale_noalloc(None, None, 2, 1, None, None, 0, 256, 256, None, 256, 0, None) == 0
    # down: workspace too small
    assert L.moe_down_combine(_p(), _p(), _p(), _p(), _p(), _p(), _p(), _p(), 16, 256, 128, 16, 4, 16, 304, _p(),
                              256, _p(), 8, None) == -1


def test_dense_workspace_query(lib):
    from fp8_block_scaled_grouped_amd import moe355
    # the rule: small M splits K (needs fp32 partials), large M does not; the workspace
    # follows the plan the call runs (the measured table's where it has an entry)
    for M, N in [(1, 2048), (1, 18432), (64, 2048), (16, 7168)]:
        tm, tn, sp = moe355.gemm_fp8_blockscale_plan(M, N, 7168, measured=False)
        assert sp >= 2 and tn in (128, 256) and tm == (16 if M <= 16 else 64), (M, N, tm, tn, sp)
        tm, tn, sp = moe355.gemm_fp8_blockscale_plan(M, N, 7168)
        n = moe355.gemm_fp8_blockscale_workspace(M, N, 7168)
        assert n == (sp * M * N * 4 + 256 if sp > 1 else 0), (M, N, n, sp)
        assert n <= M * N * 4 * 56 + 256
    assert moe355.gemm_fp8_blockscale_workspace(4096, 18432, 7168) == 0
    assert moe355.gemm_fp8_blockscale_workspace(0, 2048, 7168) == 0
    assert moe355.gemm_fp8_blockscale_workspace(1, 2048, 256) == 0  # two K blocks: nothing to split
    # partial blocks: K and N in ceil(./128) blocks
    assert moe355.gemm_fp8_blockscale_workspace(1, 1000, 4112) > 0
    # more than 128 K blocks always splits, whatever M
    assert moe355.gemm_fp8_blockscale_workspace(4096, 7168, 18432) >= 2 * 4096 * 7168 * 4
    assert moe355.gemm_fp8_blockscale_workspace(4096, 7168, 16384) == 0
    with pytest.raises(moe355.Moe355Error):
        moe355.gemm_fp8_blockscale_workspace(1, 100, 256)
    with pytest.raises(moe355.Moe355Error):
        moe355.gemm_fp8_blockscale_workspace(1, 128, 200)


def test_zero_rows_are_noops_without_touching_memory(lib):
    # zero tokens / rows: OK before any pointer is looked at (all NULL here, no GPU needed)
    L = lib
    N = None
    assert L.grouped_topk(N, 0, 16, N, 0, 16, 4, 2, 4, 1, 2.5, N, N, 4, N) == 0
    assert L.moe_sort(N, N, 4, 0, 4, 16, 16, N, N, N, N, N, 0, N) == 0
    assert L.fp8_quant_1x128(N, 256, 0, 256, N, 256, N, 2, 1, N) == 0
    assert L.moe_fp8_blockscale_g1u1(N, N, 2, 1, N, N, N, N, N, 0, 256, 128, 16, 4, 16, 256, N, N, N, N) == 0
    assert L.moe_down_combine(N, N, N, N, N, N, N, N, 0, 256, 128, 16, 4, 16, 256, N, 256, N, 0, N) == 0
    assert L.gemm_fp8_blockscale(N, N, 2, 1, N, N, 0, 256, 256, N, 256, 0, N, 0, N) == 0
    # ...but shape rules still apply
    assert L.moe_sort(N, N, 4, 0, 4, 16, 24, N, N, N, N, N, 0, N) == -2


def test_block_m_table(lib):
    import json
    import os

    from fp8_block_scaled_grouped_amd import moe355
    # the compiled table returns, at every swept token count of the V3 layer (E 256,
    # top-8), the M tile whose whole-layer time was smallest in the committed sweep, and
    # between two swept counts the choice of the larger one
    path = os.path.join(os.path.dirname(moe355.__file__), "tuning", "block_m_sweep.jsonl")
    best = {}
    for line in open(path):
        r = json.loads(line)
        if r.get("sweep") == "block_m" and (r["tokens"] not in best or r["ms"] < best[r["tokens"]][1]):
            best[r["tokens"]] = (r["block_m"], r["ms"])
    Ts = sorted(best)
    assert len(Ts) >= 8
    for i, T in enumerate(Ts):
        assert moe355.moe_block_m(T, 8, 256) == best[T][0], T
        if i > 0 and T - Ts[i - 1] > 1:
            assert moe355.moe_block_m(Ts[i - 1] + 1, 8, 256) == best[T][0], T
    # beyond the sweep: the largest count's tile; no tokens: the smallest count's tile
    assert moe355.moe_block_m(4 * Ts[-1], 8, 256) == best[Ts[-1]][0]
    assert moe355.moe_block_m(0, 8, 256) == best[Ts[0]][0]
    with pytest.raises(moe355.Moe355Error):
        moe355.moe_block_m(1, 0, 256)


def test_binding_checks_run_on_the_host():
    # the binding's tensor checks raise ValueError without touching a GPU: a host tensor
    # where a device tensor is needed, an unknown scale layout
    import torch
    from fp8_block_scaled_grouped_amd import moe355
    with pytest.raises(ValueError):
        moe355._need(torch.zeros(4), (4,), torch.float32, "x")       # not a GPU tensor
    with pytest.raises(ValueError):
        moe355._scale_strides(torch.zeros((2, 2)), 2, 256, "columns")


def test_trace_library_exports():
    # the diagnostic build carries the whole ABI plus the phase-trace readback
    path = os.path.join(ROOT, "fp8_block_scaled_grouped_amd", "libmoe355_trace.so")
    if not os.path.exists(path):
        pytest.skip("libmoe355_trace.so not built")
    lib = ctypes.CDLL(path)
    for name in _declared() + ["moe355_phase_trace_read"]:
        assert hasattr(lib, name), name
    fn = lib.moe355_phase_trace_read
    fn.argtypes, fn.restype = [ctypes.c_void_p, ctypes.c_size_t], ctypes.c_int
    assert fn(None, 1) == -1  # host-side check, no GPU touched


@pytest.mark.parametrize("name", ["lds_fill_probe", "kstep_probe", "e4m3_cvt_check"])
def test_probes_built_for_gfx950(name):
    # the probe programs are built with the library; their device code must be gfx950 code
    # objects (checked from the bundle's target names)
    path = os.path.join(ROOT, "fp8_block_scaled_grouped_amd", name)
    if not os.path.exists(path):
        pytest.skip(name + " not built")
    assert os.access(path, os.X_OK)
    with open(path, "rb") as f:
        blob = f.read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob
