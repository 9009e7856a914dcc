"""Pre-shuffled weight layout (CPU oracle; test infrastructure only).

"Accelerate DeepSeek-R1 Inference: Integrate AITER into SGLang", section
"General Linear Layer": the linear path runs on weights permuted once at load
time into an order suited to the matrix cores.  The pages name the step but
not the permutation; the one here is the library's own (its header states
it) and is written out by its definition:

  W [rows, K] (rows, K multiples of 128) -> 128-row x 128-byte tiles; tile
  (t, kb) holds rows [128t, 128t+128) and bytes [128kb, 128kb+128) of each
  and starts at byte (t * K/128 + kb) * 16384; inside it row rr occupies
  bytes [128rr, 128rr+128), its 16-byte chunk c stored in slot c ^ (rr & 7).

Only bytes move: a GEMM on shuffled weights computes exactly what it
computes on the original ones.
"""
import numpy as np


def shuffle_128x128(w):
    """uint8 [..., R, K] -> uint8 [..., R, K] in the tile layout (leading dims flattened into rows)."""
    w = np.asarray(w, dtype=np.uint8)
    K = w.shape[-1]
    rows = w.size // K
    assert rows % 128 == 0 and K % 128 == 0
    src = w.reshape(rows, K)
    out = np.empty(rows * K, dtype=np.uint8)
    for t in range(rows // 128):
        for kb in range(K // 128):
            tile = src[128 * t:128 * t + 128, 128 * kb:128 * kb + 128].reshape(128, 8, 16)   # [rr, chunk, byte]
            slotted = np.empty_like(tile)
            for rr in range(128):
                for c in range(8):
                    slotted[rr, c ^ (rr & 7)] = tile[rr, c]
            base = (t * (K // 128) + kb) * 16384
            out[base:base + 16384] = slotted.reshape(-1)
    return out.reshape(w.shape)
