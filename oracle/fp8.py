"""OCP E4M3 (e4m3fn) codec, written out from the format's definition.

Part of the CPU oracle (test infrastructure only).

Format: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no
infinities, the two codes S.1111.111 are NaN, largest finite magnitude 448
(OCP 8-bit Floating Point Specification; the zaynews item on running "V4
Flash" on one MI300X contrasts it with the fnuz variant MI300X uses, whose
scale differs by a factor of two).

decode: exact binary64 value of every code.
encode: nearest finite code to a finite fp32 value, ties to the code whose
        mantissa LSB is even, saturating at +-448, sign always kept (so -0
        and negative underflow give 0x80).  The search is done over the
        sorted table of the 127 non-negative finite magnitudes.
"""
import numpy as np

E4M3_MAX = 448.0


def _decode_closed_form(codes):
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = b >> 7
    e = (b >> 3) & 15
    m = b & 7
    sub = m.astype(np.float64) * 2.0 ** -9                    # e == 0: m * 2^-9
    nor = (8 + m).astype(np.float64) * np.exp2((e - 10).astype(np.float64))  # (1+m/8) * 2^(e-7)
    mag = np.where(e == 0, sub, nor)
    mag = np.where((b & 0x7F) == 0x7F, np.nan, mag)
    return np.where(s == 1, -mag, mag)


# value of every code, from the closed form above
_TABLE = _decode_closed_form(np.arange(256, dtype=np.uint8))


def decode(codes):
    """Exact value of e4m3fn codes as float64 (NaN for 0x7F / 0xFF)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


# magnitudes of codes 0x00..0x7E; increasing with the code
_MAGS = decode(np.arange(0, 127, dtype=np.uint8))


def encode(y):
    """Nearest-even, saturating e4m3fn encode of finite float32 values."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)                         # exact
    neg = np.signbit(y)
    sat = a >= E4M3_MAX
    ac = np.minimum(a, E4M3_MAX)
    lo = np.searchsorted(_MAGS, ac, side="right") - 1        # _MAGS[lo] <= a
    lo = np.clip(lo, 0, 126)
    hi = np.minimum(lo + 1, 126)
    dlo = ac - _MAGS[lo]                                      # exact in binary64
    dhi = _MAGS[hi] - ac
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi != lo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(sat, 0x7E, code)
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)


def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32 values (exact widening)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)
