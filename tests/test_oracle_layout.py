"""Pins of the oracle's pre-shuffled weight layout (a byte permutation)."""
import numpy as np

from oracle import layout


def _distinct(rows, K):
    # position-coded bytes are not unique in uint8; track positions with an int array instead
    return np.arange(rows * K, dtype=np.int64).reshape(rows, K)


def _shuffle_positions(rows, K):
    """Apply the oracle's permutation to position labels by shuffling each byte lane of them."""
    pos = _distinct(rows, K)
    out = np.zeros(rows * K, dtype=np.int64)
    for shift in range(0, 32, 8):          # positions < 2^32: four byte lanes
        lane = ((pos >> shift) & 0xFF).astype(np.uint8)
        out |= layout.shuffle_128x128(lane).reshape(-1).astype(np.int64) << shift
    return out


def test_is_a_bijection_and_keeps_every_byte():
    rows, K = 256, 384
    out = _shuffle_positions(rows, K)
    assert np.array_equal(np.sort(out), np.arange(rows * K))


def test_each_16k_tile_is_one_128x128_block_in_row_order():
    rows, K = 256, 384
    out = _shuffle_positions(rows, K).reshape(-1, 16384)
    KB = K // 128
    for i, tile in enumerate(out):
        t, kb = divmod(i, KB)
        r = tile // K
        k = tile % K
        # rows of the block, 128 bytes each, in order; the block's columns only
        assert np.array_equal(r.reshape(128, 128), np.repeat(np.arange(128 * t, 128 * t + 128), 128).reshape(128, 128))
        assert k.min() == 128 * kb and k.max() == 128 * kb + 127


def test_rows_keep_whole_chunks_and_the_chunk_map_is_an_involution():
    rows, K = 128, 256
    out = _shuffle_positions(rows, K).reshape(rows // 128, K // 128, 128, 8, 16)
    for rr in range(128):
        for s in range(8):
            seg = out[0, 1, rr, s]
            # a stored 16-byte slot is one whole source chunk, bytes in order
            assert np.array_equal(seg - seg[0], np.arange(16)) and seg[0] % 16 == 0
            c = (seg[0] % K - 128) // 16
            assert c == (s ^ (rr & 7)) and (c ^ (rr & 7)) == s
    # rows 8 apart use the same slot order: each run of 8 rows is 1 KB that a lane-ordered copy fills
    assert np.array_equal(out[0, 0, 0] % 128, out[0, 0, 8] % 128)


def test_expert_tensors_shuffle_as_stacked_rows(rng):
    w = rng.integers(0, 256, size=(3, 256, 128), dtype=np.uint8)
    a = layout.shuffle_128x128(w)
    b = np.stack([layout.shuffle_128x128(w[e]) for e in range(3)])
    assert np.array_equal(a, b)
