"""Pins of the oracle's e4m3fn codec against the format specification and torch's cast."""
import os

import numpy as np
import torch

from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_codes.txt")


def _all_codes():
    return np.arange(256, dtype=np.uint8)


def test_decode_matches_spec_table():
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code, val = line.split()
        got = fp8.decode(np.array([int(code, 16)], dtype=np.uint8))[0]
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val), (code, got, val)
            assert np.signbit(got) == val.startswith("-")


def test_decode_matches_torch_cast_all_codes():
    c = _all_codes()
    t = torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    d = fp8.decode(c)
    assert np.array_equal(np.isnan(t), np.isnan(d))
    fin = ~np.isnan(d)
    assert np.array_equal(t[fin], d[fin])
    assert np.array_equal(np.signbit(t[fin]), np.signbit(d[fin]))


def _brute_encode(y):
    """Nearest finite code by exhaustive search; ties to even mantissa LSB; saturate; keep sign."""
    c = _all_codes()
    vals = fp8.decode(c)
    fin = ~np.isnan(vals)
    out = []
    for v in np.asarray(y, dtype=np.float32):
        a = abs(float(v))
        if a >= 448.0:
            code = 0x7E
        else:
            best = None
            for cc, vv in zip(c[fin], vals[fin]):
                if cc & 0x80:
                    continue
                d = abs(vv - a)
                if best is None or d < best[0] or (d == best[0] and (cc & 1) == 0):
                    best = (d, int(cc))
            code = best[1]
        if np.signbit(v):
            code |= 0x80
        out.append(code)
    return np.array(out, dtype=np.uint8)


def test_encode_brute_force_random_and_edges(rng):
    vals = fp8.decode(np.arange(127, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2                       # exact midpoints between neighbours
    edges = np.concatenate([vals, mids, -mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                            np.nextafter(mids.astype(np.float32), np.float32(1e9)),
                            [0.0, -0.0, 447.9, 448.0, 448.01, 464.0, 500.0, 1e30, -1e30, 1e-30, -1e-30,
                             2.0 ** -10, 3 * 2.0 ** -11, -(2.0 ** -10)]]).astype(np.float32)
    rnd = (rng.standard_normal(3000) * np.exp2(rng.integers(-12, 9, 3000))).astype(np.float32)
    y = np.concatenate([edges, rnd])
    assert np.array_equal(fp8.encode(y), _brute_encode(y))


def test_encode_ties_go_to_even_mantissa():
    # 1.0 (0x38) and 1.125 (0x39): the midpoint 1.0625 rounds to 0x38 (even)
    assert fp8.encode(np.float32([1.0625]))[0] == 0x38
    # 1.125 (0x39) and 1.25 (0x3A): midpoint 1.1875 -> 0x3A (even)
    assert fp8.encode(np.float32([1.1875]))[0] == 0x3A
    # subnormal midpoint 2^-10 between 0 and 2^-9 -> 0 ; 3*2^-10 -> 2*2^-9 (code 2)
    assert fp8.encode(np.float32([2.0 ** -10]))[0] == 0x00
    assert fp8.encode(np.float32([3 * 2.0 ** -10]))[0] == 0x02
    # saturation and sign
    assert fp8.encode(np.float32([1e6]))[0] == 0x7E
    assert fp8.encode(np.float32([-1e6]))[0] == 0xFE
    assert fp8.encode(np.float32([-0.0]))[0] == 0x80
    assert fp8.encode(np.float32([-1e-20]))[0] == 0x80


def test_encode_matches_torch_cast_in_range(rng):
    y = (rng.standard_normal(200000) * 100).astype(np.float32)
    y = y[np.abs(y) < 448]
    t = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.encode(y), t)


def test_encode_decode_roundtrip_all_finite_codes():
    c = _all_codes()
    d = fp8.decode(c)
    fin = ~np.isnan(d)
    assert np.array_equal(fp8.encode(d[fin].astype(np.float32)), c[fin])


def test_bf16_widening_matches_torch_cast_all_patterns():
    # every bf16 bit pattern widened by the oracle equals torch's bfloat16 -> float32 cast
    # (a library routine): same value, same sign of zero, NaN exactly where torch has NaN
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = fp8.bf16_bits_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    assert got.dtype == np.float32
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    # a few values fixed by the format: 0x3F80 = 1, 0xC000 = -2, 0x7F80 = +inf, 0x0001 = 2^-133
    spot = fp8.bf16_bits_to_f32(np.array([0x3F80, 0xC000, 0x7F80, 0x0001, 0x8000], np.uint16))
    assert spot[0] == 1.0 and spot[1] == -2.0 and np.isposinf(spot[2]) and spot[3] == 2.0 ** -133
    assert spot[4] == 0.0 and np.signbit(spot[4])
