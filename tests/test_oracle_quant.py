"""Pins of the oracle's dynamic 1x128 quantisation."""
import numpy as np
import torch

from oracle import fp8, quant


def test_identity_group_scale_one():
    # a group of e4m3-exact values whose amax is 448 quantises with scale 1 to its own codes
    codes = np.arange(0, 127, dtype=np.uint8)
    codes = np.concatenate([codes, [0x7E]])[:128].copy()
    codes[5] |= 0x80
    x = fp8.decode(codes).astype(np.float32)[None, :]
    q, s = quant.quant_1x128(x)
    assert s[0, 0] == np.float32(1.0)
    assert np.array_equal(q[0], codes)


def test_zero_group_scale_one_and_signed_zeros():
    x = np.zeros((2, 256), dtype=np.float32)
    x[1, :128] = -0.0
    x[1, 128:] = np.linspace(-1, 1, 128)
    q, s = quant.quant_1x128(x)
    assert s[0, 0] == 1.0 and s[0, 1] == 1.0 and s[1, 0] == 1.0
    assert np.all(q[0] == 0) and np.all(q[1, :128] == 0x80)
    assert s[1, 1] == np.float32(np.float32(1.0) / np.float32(448.0))


def test_matches_torch_division_and_cast(rng):
    # independent path: torch fp32 division and torch's e4m3fn cast (RNE; values just above
    # 448 from the rounded scale still round to 448)
    x = (rng.standard_normal((64, 1024)) * np.exp2(rng.integers(-20, 20, (64, 1)))).astype(np.float32)
    q, s = quant.quant_1x128(x)
    xt = torch.from_numpy(x).view(64, 8, 128)
    amax = xt.abs().amax(-1)
    st = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
    qt = (xt / st[..., None]).to(torch.float8_e4m3fn).view(torch.uint8).reshape(64, 1024)
    assert np.array_equal(s, st.numpy())
    assert np.array_equal(q, qt.numpy())


def test_amax_maps_to_448_and_error_bound(rng):
    x = (rng.standard_normal((32, 512)) * 3).astype(np.float32)
    q, s = quant.quant_1x128(x)
    g = x.reshape(32, 4, 128)
    qa = fp8.decode(q).reshape(32, 4, 128)
    # the element of largest magnitude lands on +-448 (or saturates there)
    i = np.abs(g).argmax(-1)
    assert np.all(np.abs(np.take_along_axis(qa, i[..., None], -1)) == 448.0)
    # half-ulp bound of e4m3 (relative 2^-4) plus half the subnormal step
    deq = quant.dequant_1x128(q, s).reshape(32, 4, 128)
    bound = np.abs(g) * 2.0 ** -4 + s[..., None].astype(np.float64) * 2.0 ** -10 + 1e-12
    assert np.all(np.abs(deq - g) <= bound * (1 + 1e-6))


def test_partial_last_group_matches_torch(rng):
    # K = 200: groups of 128 and 72 values, each with its own amax
    x = (rng.standard_normal((16, 200)) * np.exp2(rng.integers(-8, 8, (16, 1)))).astype(np.float32)
    x[3, 128:] = 0.0                                   # an all-zero tail group keeps scale 1
    q, s = quant.quant_1x128(x)
    assert q.shape == (16, 200) and s.shape == (16, 2)
    xt = torch.from_numpy(x)
    for kb, (lo, hi) in enumerate(((0, 128), (128, 200))):
        g = xt[:, lo:hi]
        amax = g.abs().amax(-1)
        st = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
        qt = (g / st[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)
        assert np.array_equal(s[:, kb], st.numpy())
        assert np.array_equal(q[:, lo:hi], qt.numpy())
    assert s[3, 1] == 1.0 and np.all(q[3, 128:] == 0)
    deq = quant.dequant_1x128(q, s)
    assert np.all(np.abs(deq - x) <= np.abs(x) * 2.0 ** -4 + np.repeat(s, 128, 1)[:, :200] * 2.0 ** -10 + 1e-12)
