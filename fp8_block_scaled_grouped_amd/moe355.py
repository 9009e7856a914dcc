"""Python binding of libmoe355 (ctypes).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoe355.so.  Tensors are torch CUDA (HIP) tensors; outputs are allocated
here when not passed in, and every call is queued on torch's current stream.
A missing library raises at the first call -- there is no fallback.

Function names and argument order follow include/moe355.h.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe355.so")
_lib = None

_i32, _i64, _f32, _vp, _sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_P64, _PSZ = ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_size_t)

_SIGNATURES = {
    "moe355_strerror": ([_i32], ctypes.c_char_p),
    "grouped_topk": ([_vp, _i32, _i64, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _vp, _i64, _vp], _i32),
    "moe_sort_sizes": ([_i32, _i32, _i32, _i32, _P64, _P64, _PSZ], _i32),
    "moe_block_m": ([_i32, _i32, _i32, ctypes.POINTER(ctypes.c_int)], _i32),
    "moe_sort": ([_vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "fp8_quant_1x128": ([_vp, _i64, _i32, _i32, _vp, _i64, _vp, _i64, _i64, _vp], _i32),
    "moe_fp8_blockscale_g1u1": ([_vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                 _i64, _vp, _vp, _vp, _vp], _i32),
    "moe_down_combine_workspace": ([_i32, _i32, _i32, _PSZ], _i32),
    "moe_down_combine": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _vp,
                          _i64, _vp, _sz, _vp], _i32),
    "gemm_fp8_blockscale_workspace": ([_i32, _i32, _i32, _PSZ], _i32),
    "gemm_fp8_blockscale": ([_vp, _vp, _i64, _i64, _vp, _vp, _i32, _i32, _i32, _vp, _i64, _i32, _vp, _sz, _vp],
                            _i32),
    "shuffle_weight_128x128": ([_vp, _i64, _i32, _vp, _vp], _i32),
    "gemm_fp8_blockscale_noalloc": ([_vp, _vp, _i64, _i64, _vp, _vp, _i32, _i32, _i32, _vp, _i64, _i32, _vp], _i32),
    "moe_fp8_blockscale_fused_workspace": ([_i32, _i32, _i32, _i32, _i32, _i32, _PSZ], _i32),
    "gemm_fp8_blockscale_tiled": ([_vp, _vp, _i64, _i64, _vp, _vp, _i32, _i32, _i32, _vp, _i64, _i32, _i32, _i32, _i32,
                                   _vp, _sz, _vp], _i32),
    "gemm_fp8_blockscale_tiled_workspace": ([_i32, _i32, _i32, _i32, _PSZ], _i32),
    "gemm_fp8_blockscale_plan": ([_i32, _i32, _i32, _i32, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                  ctypes.POINTER(ctypes.c_int)], _i32),
    "moe_fp8_blockscale_fused": ([_vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                  _i32, _i32, _i64, _vp, _vp, _i64, _vp, _sz, _vp], _i32),
}
# the pre-shuffled-weight variants take the same arguments as their plain calls
for _name in ("gemm_fp8_blockscale", "moe_fp8_blockscale_g1u1", "moe_down_combine"):
    _SIGNATURES[_name + "_wpreshuffle"] = _SIGNATURES[_name]
EXPORTED = tuple(_SIGNATURES)


def lib():
    """Load libmoe355.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe355.so not found at %s; build it with "
                               "`python -m fp8_block_scaled_grouped_amd.build`" % LIB_PATH)
        l = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = res
        _lib = l
    return _lib


class Moe355Error(RuntimeError):
    def __init__(self, code):
        self.code = code
        super().__init__(lib().moe355_strerror(code).decode())


def _check(code):
    if code != 0:
        raise Moe355Error(code)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, dtype, name):
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t


def _need(t, shape, dtype, name):
    """A contiguous device tensor of exactly this shape and dtype (the kernels index it densely)."""
    _dev(t, dtype, name)
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s tensor of shape %s, got %s" % (name, dtype, tuple(shape),
                                                                                 tuple(t.shape)))
    return t


def _rows(t, name):
    """Row stride of a 2-D tensor whose rows are contiguous."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("%s must be 2-D with contiguous rows" % name)
    return t.stride(0)


# ----------------------------------------------------------------- routing
def grouped_topk(logits, bias, n_group, topk_group, topk, renorm, routed_scaling_factor,
                 topk_weights=None, topk_ids=None):
    """Biased grouped top-k.  Returns (topk_weights fp32 [T, k], topk_ids int32 [T, k]).

    logits: fp32 or bf16 [T, E].  Outputs may be passed in as row-strided views (same
    row stride for both).
    """
    if logits.dtype != torch.bfloat16:
        _dev(logits, torch.float32, "logits")
    _dev(logits, logits.dtype, "logits")
    T, E = logits.shape
    _need(bias, (E,), torch.float32, "bias")
    if topk_weights is None:
        topk_weights = torch.empty((T, topk), dtype=torch.float32, device=logits.device)
    if topk_ids is None:
        topk_ids = torch.empty((T, topk), dtype=torch.int32, device=logits.device)
    _dev(topk_weights, torch.float32, "topk_weights")
    _dev(topk_ids, torch.int32, "topk_ids")
    if tuple(topk_weights.shape) != (T, topk) or tuple(topk_ids.shape) != (T, topk):
        raise ValueError("top-k outputs must be [T, topk] = %s" % ((T, topk),))
    ld = _rows(topk_weights, "topk_weights")
    if _rows(topk_ids, "topk_ids") != ld:
        raise ValueError("topk_weights and topk_ids must share a row stride")
    _check(lib().grouped_topk(_ptr(logits), int(logits.dtype == torch.bfloat16), _rows(logits, "logits"),
                              _ptr(bias), T, E, n_group,
                              topk_group, topk, int(bool(renorm)), float(routed_scaling_factor),
                              _ptr(topk_weights), _ptr(topk_ids), ld, _stream()))
    return topk_weights, topk_ids


# ----------------------------------------------------------------- sort
def moe_sort_sizes(T, topk, E, block_m):
    """(max_sorted, max_blocks, workspace_bytes) -- host-only."""
    ms, mb, ws = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t()
    _check(lib().moe_sort_sizes(T, topk, E, block_m, ctypes.byref(ms), ctypes.byref(mb), ctypes.byref(ws)))
    return ms.value, mb.value, ws.value


def moe_block_m(T, topk, E):
    """Tuned M tile of the grouped GEMMs for this size (host-only)."""
    b = ctypes.c_int()
    _check(lib().moe_block_m(T, topk, E, ctypes.byref(b)))
    return b.value


def moe_sort(topk_ids, topk_weights, E, block_m, out=None, workspace=None):
    """Returns (sorted_ids, sorted_weights, sorted_expert_ids, num_valid) device tensors."""
    _dev(topk_ids, torch.int32, "topk_ids")
    _dev(topk_weights, torch.float32, "topk_weights")
    T, k = topk_ids.shape
    if tuple(topk_weights.shape) != (T, k):
        raise ValueError("topk_weights must have the shape of topk_ids")
    ms, mb, wsb = moe_sort_sizes(T, k, E, block_m)
    dev = topk_ids.device
    if out is None:
        out = (torch.empty(ms, dtype=torch.int32, device=dev), torch.empty(ms, dtype=torch.float32, device=dev),
               torch.empty(mb, dtype=torch.int32, device=dev), torch.zeros(1, dtype=torch.int32, device=dev))
    if workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    sid, sw, seid, nv = out
    for t, n, dt, name in ((sid, ms, torch.int32, "sorted_ids"), (sw, ms, torch.float32, "sorted_weights"),
                           (seid, mb, torch.int32, "sorted_expert_ids"), (nv, 1, torch.int32, "num_valid")):
        _dev(t, dt, name)
        if not t.is_contiguous() or t.numel() < n:
            raise ValueError("%s must be contiguous with at least %d entries" % (name, n))
    _dev(workspace, torch.uint8, "workspace")
    ld = _rows(topk_ids, "topk_ids")
    if _rows(topk_weights, "topk_weights") != ld:
        raise ValueError("topk_ids and topk_weights must share a row stride")
    _check(lib().moe_sort(_ptr(topk_ids), _ptr(topk_weights), ld, T, k, E, block_m, _ptr(sid), _ptr(sw), _ptr(seid),
                          _ptr(nv), _ptr(workspace), workspace.numel(), _stream()))
    return sid, sw, seid, nv


# ----------------------------------------------------------------- quant
def fp8_quant_1x128(x, q=None, scale=None, scale_layout="row"):
    """bf16 [M, K] -> (e4m3 uint8 [M, K], fp32 scales).

    scale_layout "row": scales [M, KB]; "kblock": scales [KB, M]; KB = ceil(K/128).
    """
    _dev(x, torch.bfloat16, "x")
    M, K = x.shape
    KB = _nblk(K)
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    shape = (M, KB) if scale_layout == "row" else (KB, M)
    if scale is None:
        scale = torch.empty(shape, dtype=torch.float32, device=x.device)
    _dev(q, torch.uint8, "q")
    if tuple(q.shape) != (M, K):
        raise ValueError("q must be [M, K] = %s, got %s" % ((M, K), tuple(q.shape)))
    _need(scale, shape, torch.float32, "scale")
    ssm, sskb = (KB, 1) if scale_layout == "row" else (1, M)
    _check(lib().fp8_quant_1x128(_ptr(x), _rows(x, "x"), M, K, _ptr(q), _rows(q, "q"), _ptr(scale), ssm, sskb,
                                 _stream()))
    return q, scale


def _nblk(n):
    """ceil(n / 128): scale entries along a dimension of n."""
    return -(-n // 128)


def _scale_strides(a_scale, T, H, scale_layout):
    """Element strides (per row, per K block) of 1x128 activation scales in either layout."""
    KB = _nblk(H)
    if scale_layout == "row":
        _need(a_scale, (T, KB), torch.float32, "a_scale")
        return KB, 1
    if scale_layout != "kblock":
        raise ValueError("scale_layout must be 'row' or 'kblock'")
    _need(a_scale, (KB, T), torch.float32, "a_scale")
    return 1, T


# ----------------------------------------------------------------- grouped GEMMs
def moe_fp8_blockscale_g1u1(a8, a_scale, w1, w1_scale, sorted_ids, sorted_expert_ids, num_valid, topk, block_m,
                            h8=None, h_scale=None, scale_layout="row", fc2_smooth_scale=None, preshuffled=False):
    """Gate/up grouped GEMM + SiLU*up (* fc2_smooth_scale [E, I] if given) + 1x128 requant.

    Returns (h8 [max_sorted, I], h_scale [max_sorted, I/128]).  preshuffled: w1 holds
    shuffle_weight_128x128 output (same shape).
    """
    T, H = a8.shape
    E, twoI, _ = w1.shape
    I = twoI // 2
    _need(a8, (T, H), torch.uint8, "a8")
    _need(w1, (E, 2 * I, H), torch.uint8, "w1")
    _need(w1_scale, (E, _nblk(2 * I), _nblk(H)), torch.float32, "w1_scale")
    ms = sorted_ids.numel()
    _need(sorted_ids, (ms,), torch.int32, "sorted_ids")
    _need(sorted_expert_ids, (sorted_expert_ids.numel(),), torch.int32, "sorted_expert_ids")
    if block_m <= 0 or sorted_expert_ids.numel() < ms // block_m:
        raise ValueError("sorted_expert_ids must hold max_sorted / block_m entries")
    _need(num_valid, (1,), torch.int32, "num_valid")
    if h8 is None:
        h8 = torch.empty((ms, I), dtype=torch.uint8, device=a8.device)
    if h_scale is None:
        h_scale = torch.empty((ms, I // 128), dtype=torch.float32, device=a8.device)
    _need(h8, (ms, I), torch.uint8, "h8")
    _need(h_scale, (ms, _nblk(I)), torch.float32, "h_scale")
    if fc2_smooth_scale is not None:
        _need(fc2_smooth_scale, (E, I), torch.float32, "fc2_smooth_scale")
    ssm, sskb = _scale_strides(a_scale, T, H, scale_layout)
    fn = lib().moe_fp8_blockscale_g1u1_wpreshuffle if preshuffled else lib().moe_fp8_blockscale_g1u1
    _check(fn(_ptr(a8), _ptr(a_scale), ssm, sskb, _ptr(w1), _ptr(w1_scale),
              _ptr(sorted_ids), _ptr(sorted_expert_ids), _ptr(num_valid), T, H, I, E,
              topk, block_m, ms, _ptr(h8), _ptr(h_scale),
              _ptr(fc2_smooth_scale), _stream()))
    return h8, h_scale


def moe_down_combine_workspace(T, H, topk):
    b = ctypes.c_size_t()
    _check(lib().moe_down_combine_workspace(T, H, topk, ctypes.byref(b)))
    return b.value


def moe_down_combine(h8, h_scale, w2, w2_scale, sorted_ids, sorted_weights, sorted_expert_ids, num_valid, T, topk,
                     block_m, out=None, workspace=None, preshuffled=False):
    """Down grouped GEMM + top-k weighted combine.  Returns bf16 [T, H].  preshuffled: w2 holds
    shuffle_weight_128x128 output (same shape)."""
    E, H, I = w2.shape
    _need(w2, (E, H, I), torch.uint8, "w2")
    _need(w2_scale, (E, _nblk(H), _nblk(I)), torch.float32, "w2_scale")
    ms = sorted_ids.numel()
    _need(sorted_ids, (ms,), torch.int32, "sorted_ids")
    _need(sorted_weights, (ms,), torch.float32, "sorted_weights")
    _need(sorted_expert_ids, (sorted_expert_ids.numel(),), torch.int32, "sorted_expert_ids")
    if block_m <= 0 or sorted_expert_ids.numel() < ms // block_m:
        raise ValueError("sorted_expert_ids must hold max_sorted / block_m entries")
    _need(num_valid, (1,), torch.int32, "num_valid")
    _need(h8, (ms, I), torch.uint8, "h8")
    _need(h_scale, (ms, _nblk(I)), torch.float32, "h_scale")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=h8.device)
    if workspace is None:
        workspace = torch.empty(moe_down_combine_workspace(T, H, topk), dtype=torch.uint8, device=h8.device)
    _dev(out, torch.bfloat16, "out")
    if tuple(out.shape) != (T, H):
        raise ValueError("out must be [T, H] = %s, got %s" % ((T, H), tuple(out.shape)))
    _dev(workspace, torch.uint8, "workspace")
    fn = lib().moe_down_combine_wpreshuffle if preshuffled else lib().moe_down_combine
    _check(fn(_ptr(h8), _ptr(h_scale), _ptr(w2), _ptr(w2_scale), _ptr(sorted_ids), _ptr(sorted_weights),
              _ptr(sorted_expert_ids), _ptr(num_valid), T, H, I, E, topk, block_m, ms, _ptr(out), _rows(out, "out"),
              _ptr(workspace), workspace.numel(), _stream()))
    return out


def gemm_fp8_blockscale_plan(M, N, K, measured=True):
    """(tile_m, tile_n, splits) gemm_fp8_blockscale runs for this shape (host-only);
    measured=False: the rule alone, without the table of measured plans."""
    tm, tn, sp = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib().gemm_fp8_blockscale_plan(M, N, K, int(bool(measured)), ctypes.byref(tm), ctypes.byref(tn),
                                          ctypes.byref(sp)))
    return tm.value, tn.value, sp.value


def gemm_fp8_blockscale_tiled_workspace(M, N, K, splits):
    b = ctypes.c_size_t()
    _check(lib().gemm_fp8_blockscale_tiled_workspace(M, N, K, splits, ctypes.byref(b)))
    return b.value


def gemm_fp8_blockscale_tiled(a8, a_scale, b8, b_scale, tile_m, tile_n, splits, c=None, workspace=None,
                              scale_layout="row", out_dtype=torch.bfloat16):
    """gemm_fp8_blockscale with a caller-chosen tiling (tile_m rows x tile_n columns, K in
    `splits` runs); workspace None allocates what the split needs."""
    M, K = a8.shape
    N = b8.shape[0]
    _need(a8, (M, K), torch.uint8, "a8")
    _need(b8, (N, K), torch.uint8, "b8")
    _need(b_scale, (_nblk(N), _nblk(K)), torch.float32, "b_scale")
    if c is None:
        c = torch.empty((M, N), dtype=out_dtype, device=a8.device)
    if c.dtype not in (torch.bfloat16, torch.float16) or tuple(c.shape) != (M, N):
        raise ValueError("c must be bf16 or fp16 [M, N]")
    _dev(c, c.dtype, "c")
    if workspace is None:
        n = gemm_fp8_blockscale_tiled_workspace(M, N, K, splits)
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=a8.device)
    _dev(workspace, torch.uint8, "workspace")
    ssm, sskb = _scale_strides(a_scale, M, K, scale_layout)
    _check(lib().gemm_fp8_blockscale_tiled(_ptr(a8), _ptr(a_scale), ssm, sskb, _ptr(b8), _ptr(b_scale), M, N, K,
                                           _ptr(c), _rows(c, "c"), int(c.dtype == torch.float16), tile_m, tile_n,
                                           splits, _ptr(workspace), workspace.numel(), _stream()))
    return c


def moe_fp8_blockscale_fused_workspace(T, H, I, E, topk, block_m):
    b = ctypes.c_size_t()
    _check(lib().moe_fp8_blockscale_fused_workspace(T, H, I, E, topk, block_m, ctypes.byref(b)))
    return b.value


def moe_fp8_blockscale_fused(a8, a_scale, w1, w1_scale, w2, w2_scale, sorted_ids, sorted_weights, sorted_expert_ids,
                             num_valid, topk, block_m, out=None, workspace=None, scale_layout="row",
                             fc2_smooth_scale=None):
    """Gate/up + SiLU*up + requant, down projection and combine in one launch.  Returns bf16 [T, H]."""
    T, H = a8.shape
    E, twoI, _ = w1.shape
    I = twoI // 2
    _need(a8, (T, H), torch.uint8, "a8")
    _need(w1, (E, 2 * I, H), torch.uint8, "w1")
    _need(w1_scale, (E, _nblk(2 * I), _nblk(H)), torch.float32, "w1_scale")
    _need(w2, (E, H, I), torch.uint8, "w2")
    _need(w2_scale, (E, _nblk(H), _nblk(I)), torch.float32, "w2_scale")
    ms = sorted_ids.numel()
    _need(sorted_ids, (ms,), torch.int32, "sorted_ids")
    _need(sorted_weights, (ms,), torch.float32, "sorted_weights")
    _need(sorted_expert_ids, (sorted_expert_ids.numel(),), torch.int32, "sorted_expert_ids")
    if block_m <= 0 or sorted_expert_ids.numel() < ms // block_m:
        raise ValueError("sorted_expert_ids must hold max_sorted / block_m entries")
    _need(num_valid, (1,), torch.int32, "num_valid")
    if fc2_smooth_scale is not None:
        _need(fc2_smooth_scale, (E, I), torch.float32, "fc2_smooth_scale")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=a8.device)
    _dev(out, torch.bfloat16, "out")
    if tuple(out.shape) != (T, H):
        raise ValueError("out must be [T, H] = %s, got %s" % ((T, H), tuple(out.shape)))
    if workspace is None:
        workspace = torch.empty(moe_fp8_blockscale_fused_workspace(T, H, I, E, topk, block_m), dtype=torch.uint8,
                                device=a8.device)
    _dev(workspace, torch.uint8, "workspace")
    ssm, sskb = _scale_strides(a_scale, T, H, scale_layout)
    _check(lib().moe_fp8_blockscale_fused(_ptr(a8), _ptr(a_scale), ssm, sskb, _ptr(w1), _ptr(w1_scale), _ptr(w2),
                                          _ptr(w2_scale), _ptr(sorted_ids), _ptr(sorted_weights),
                                          _ptr(sorted_expert_ids), _ptr(num_valid), T, H, I, E, topk, block_m, ms,
                                          _ptr(fc2_smooth_scale), _ptr(out), _rows(out, "out"), _ptr(workspace),
                                          workspace.numel(), _stream()))
    return out


# ----------------------------------------------------------------- weight layout
def shuffle_weight_128x128(w, out=None):
    """e4m3 weights [..., R, K] (R, K multiples of 128) -> the same bytes in the
    pre-shuffled 128x128-tile layout the *_wpreshuffle calls read (new tensor, same shape)."""
    _dev(w, torch.uint8, "w")
    if not w.is_contiguous():
        raise ValueError("w must be contiguous")
    K = w.shape[-1]
    rows = w.numel() // K if K else 0
    if out is None:
        out = torch.empty_like(w)
    _check(lib().shuffle_weight_128x128(_ptr(w), rows, K, _ptr(out), _stream()))
    return out


# ----------------------------------------------------------------- dense
def gemm_fp8_blockscale_workspace(M, N, K):
    b = ctypes.c_size_t()
    _check(lib().gemm_fp8_blockscale_workspace(M, N, K, ctypes.byref(b)))
    return b.value


def gemm_fp8_blockscale(a8, a_scale, b8, b_scale, c=None, scale_layout="row", workspace=None,
                        out_dtype=torch.bfloat16, preshuffled=False):
    """a8 e4m3 [M, K] (1x128 scales), b8 e4m3 [N, K] (128x128 scales) -> [M, N] in out_dtype
    (bf16 or fp16; taken from c when c is given).  K and N need not be multiples of
    128: a_scale [M, ceil(K/128)], b_scale [ceil(N/128), ceil(K/128)].  preshuffled: b8 holds
    shuffle_weight_128x128 output (same shape; N, K multiples of 128).

    workspace: None allocates what gemm_fp8_blockscale_workspace asks for; False runs
    without workspace (no split-K); or a device uint8 tensor.
    """
    M, K = a8.shape
    N = b8.shape[0]
    _need(a8, (M, K), torch.uint8, "a8")
    _need(b8, (N, K), torch.uint8, "b8")
    _need(b_scale, (_nblk(N), _nblk(K)), torch.float32, "b_scale")
    if c is None:
        c = torch.empty((M, N), dtype=out_dtype, device=a8.device)
    if c.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("c must be bf16 or fp16, got %s" % c.dtype)
    _dev(c, c.dtype, "c")
    if tuple(c.shape) != (M, N):
        raise ValueError("c must be [M, N] = %s, got %s" % ((M, N), tuple(c.shape)))
    if workspace is None:
        n = gemm_fp8_blockscale_workspace(M, N, K)
        workspace = torch.empty(n, dtype=torch.uint8, device=a8.device) if n else False
    ws_ptr, ws_n = (None, 0) if workspace is False else (_ptr(workspace), workspace.numel())
    ssm, sskb = _scale_strides(a_scale, M, K, scale_layout)
    fn = lib().gemm_fp8_blockscale_wpreshuffle if preshuffled else lib().gemm_fp8_blockscale
    _check(fn(_ptr(a8), _ptr(a_scale), ssm, sskb, _ptr(b8), _ptr(b_scale), M, N, K, _ptr(c), _rows(c, "c"),
              int(c.dtype == torch.float16), ws_ptr, ws_n, _stream()))
    return c


# ----------------------------------------------------------------- the layer
class MoELayer:
    """The five calls of one MoE layer on preallocated buffers (no allocation per call).

    forward(hidden bf16 [T, H], logits fp32 [T, E]) -> bf16 [T, H], running
    grouped_topk -> moe_sort -> fp8_quant_1x128 -> moe_fp8_blockscale_g1u1 ->
    moe_down_combine on the current stream.  With overlap_quant the quantisation, which
    does not depend on the routing, runs on a second stream (default priority) beside
    grouped_topk and moe_sort: it starts after everything already queued on the current
    stream (so also after the previous forward's GEMMs, which read a8) and the GEMMs wait
    for it.  Off by default: it measured within noise on the prefill layer (5.10 against
    5.11 ms of serial calls) and 14 us slower on the 64-token decode layer, where the
    cross-stream join costs more than the 6 us quantisation.
    """

    def __init__(self, cfg, bias, w1, w1_scale, w2, w2_scale, T=None, block_m=None, scale_layout="row",
                 fc2_smooth_scale=None, preshuffle=False, fused=False, overlap_quant=False):
        self.cfg = cfg
        self.T = cfg.T if T is None else T
        if block_m is None:
            block_m = cfg.block_m if cfg.block_m else moe_block_m(self.T, cfg.topk, cfg.E)
        self.block_m = block_m
        # preshuffle: the weights are permuted once, here, into the 128x128-tile layout
        self.preshuffle = preshuffle
        if preshuffle:
            w1, w2 = shuffle_weight_128x128(w1), shuffle_weight_128x128(w2)
        self.bias, self.w1, self.w1_scale, self.w2, self.w2_scale = bias, w1, w1_scale, w2, w2_scale
        self.scale_layout = scale_layout
        self.fc2_smooth_scale = fc2_smooth_scale
        dev = w1.device
        T, H, I, E, k = self.T, cfg.H, cfg.I, cfg.E, cfg.topk
        ms, mb, wsb = moe_sort_sizes(T, k, E, self.block_m)
        self.max_sorted = ms
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.sort_out = (torch.empty(ms, dtype=torch.int32, device=dev), torch.empty(ms, dtype=torch.float32,
                                                                                      device=dev),
                         torch.empty(mb, dtype=torch.int32, device=dev), torch.zeros(1, dtype=torch.int32,
                                                                                      device=dev))
        self.sort_ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
        self.a8 = torch.empty((T, H), dtype=torch.uint8, device=dev)
        self.a_scale = torch.empty((T, H // 128) if scale_layout == "row" else (H // 128, T), dtype=torch.float32,
                                   device=dev)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        self.side = torch.cuda.Stream(device=dev) if overlap_quant else None
        # fused: the expert computation as one launch (moe_fp8_blockscale_fused), its
        # intermediates in one workspace; else the two calls on h8 / h_scale / down_ws
        self.fused = fused
        if fused:
            if preshuffle:
                raise ValueError("the fused call takes weights as loaded (no pre-shuffled variant)")
            self.fused_ws = torch.empty(moe_fp8_blockscale_fused_workspace(T, H, I, E, k, self.block_m),
                                        dtype=torch.uint8, device=dev)
        else:
            self.h8 = torch.empty((ms, I), dtype=torch.uint8, device=dev)
            self.h_scale = torch.empty((ms, I // 128), dtype=torch.float32, device=dev)
            self.down_ws = torch.empty(moe_down_combine_workspace(T, H, k), dtype=torch.uint8, device=dev)

    def route_and_quantise(self, hidden, logits):
        """grouped_topk, moe_sort and fp8_quant_1x128 (on the side stream with overlap_quant);
        returns the sort outputs.  On return the current stream is ordered after all three."""
        c = self.cfg
        main = torch.cuda.current_stream()
        if self.side is not None:
            self.side.wait_stream(main)
            with torch.cuda.stream(self.side):
                fp8_quant_1x128(hidden, self.a8, self.a_scale, self.scale_layout)
        grouped_topk(logits, self.bias, c.n_group, c.topk_group, c.topk, c.renorm, c.routed_scaling_factor,
                     self.topk_w, self.topk_ids)
        srt = moe_sort(self.topk_ids, self.topk_w, c.E, self.block_m, self.sort_out, self.sort_ws)
        if self.side is not None:
            main.wait_stream(self.side)
        else:
            fp8_quant_1x128(hidden, self.a8, self.a_scale, self.scale_layout)
        return srt

    def forward(self, hidden, logits):
        c = self.cfg
        sid, sw, seid, nv = self.route_and_quantise(hidden, logits)
        if self.fused:
            return moe_fp8_blockscale_fused(self.a8, self.a_scale, self.w1, self.w1_scale, self.w2, self.w2_scale, sid,
                                            sw, seid, nv, c.topk, self.block_m, self.out, self.fused_ws,
                                            self.scale_layout, self.fc2_smooth_scale)
        moe_fp8_blockscale_g1u1(self.a8, self.a_scale, self.w1, self.w1_scale, sid, seid, nv, c.topk, self.block_m,
                                self.h8, self.h_scale, self.scale_layout, self.fc2_smooth_scale, self.preshuffle)
        moe_down_combine(self.h8, self.h_scale, self.w2, self.w2_scale, sid, sw, seid, nv, self.T, c.topk,
                         self.block_m, self.out, self.down_ws, self.preshuffle)
        return self.out
