"""Element and scale formats, written from their definitions (oracle; test infrastructure).

Formats (OCP Microscaling v1.0 and the NVFP4 convention; the vLLM write-ups
name the dtypes ``float4_e2m1fn_x2`` and ``e4m3`` scales but do not print
their tables):

* E2M1 (FP4): sign, 2 exponent bits (bias 1), 1 mantissa bit, no Inf/NaN.
  Magnitude codes 0..7 decode to {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* E4M3 "fn" (FP8): sign, 4 exponent bits (bias 7), 3 mantissa bits, no Inf,
  0x7F/0xFF are NaN, largest finite 448, subnormals m * 2^-9.
* E8M0: unsigned exponent byte, value 2^(e-127), 0xFF is NaN.
* bfloat16 output: the upper 16 bits of an IEEE binary32.

Rounding everywhere is round-to-nearest, ties to even, and encoders saturate
to the largest finite value instead of producing NaN ("satfinite").

Pins (tests/test_oracle_formats.py): E2M1 against an independent
nearest-of-eight brute force and the tie table; E4M3 against an independent
nearest-of-table brute force and against torch.float8_e4m3fn on [0, 464];
bfloat16 rounding against torch's float32 -> bfloat16 cast.
"""

import numpy as np

# The eight E2M1 magnitudes, indexed by the 3-bit magnitude code.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


# ---------------------------------------------------------------------------
# E2M1
# ---------------------------------------------------------------------------

def e2m1_encode(u):
    """Encode float32 values to E2M1 codes (uint8 in 0..15), RNE, satfinite.

    The magnitude code comes from the round-to-nearest-even decision points
    between neighbouring E2M1 magnitudes: 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.
    At a tie the even magnitude code wins, so a value exactly at 0.25, 1.25,
    2.5 or 5 rounds down and one exactly at 0.75, 1.75 or 3.5 rounds up.
    Anything above 5 saturates to 6 (code 7). The sign bit (bit 3) is copied
    from the input, so negative values that round to zero give code 0x8.
    """
    u = np.asarray(u, dtype=np.float32)
    a = np.abs(u)
    mag = np.zeros(a.shape, dtype=np.uint8)
    mag += (a > np.float32(0.25))
    mag += (a >= np.float32(0.75))
    mag += (a > np.float32(1.25))
    mag += (a >= np.float32(1.75))
    mag += (a > np.float32(2.5))
    mag += (a >= np.float32(3.5))
    mag += (a > np.float32(5.0))
    sign = (u.view(np.uint32) >> np.uint32(31)).astype(np.uint8)
    return (mag | (sign << np.uint8(3))).astype(np.uint8)


def e2m1_decode(codes):
    """Decode E2M1 codes (0..15) to float64 values (exact)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


# ---------------------------------------------------------------------------
# E4M3 (fn variant)
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Decode E4M3 bytes to float64. 0x7F and 0xFF decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    sub = m * 2.0 ** -9
    nor = (8 + m) * np.ldexp(1.0, (e - 10).astype(np.int64))
    v = np.where(e == 0, sub, nor)
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return np.where(s == 1, -v, v)


def e4m3_encode(x):
    """Encode float32 values to E4M3 bytes: RNE, subnormals kept, satfinite.

    Written arithmetically: find the binade of |x| (never below the smallest
    normal binade 2^-6, which also covers the subnormals), divide by the
    quantum 2^(E-3) of that binade (exact in float64), round the quotient to
    an integer with ties to even, and rebuild the exponent/mantissa fields.
    Magnitudes above 448 saturate to 448 (0x7E).
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    sign = ((x.view(np.uint32) >> np.uint32(31)) & 1).astype(np.uint8)
    sat = a >= E4M3_MAX
    a = np.where(sat, 1.0, a)                   # saturated lanes are overwritten below
    _, e2 = np.frexp(np.where(a > 0, a, 1.0))  # a = f * 2^e2, f in [0.5, 1)
    E = np.maximum(e2 - 1, -6)                  # binade exponent, floored at 2^-6
    quantum = np.ldexp(1.0, (E - 3).astype(np.int64))
    n = np.rint(a / quantum)                    # RNE; a/quantum is exact
    # rounding up into the next binade
    up = n >= 16
    E = np.where(up, E + 1, E)
    n = np.where(up, n / 2, n)
    is_sub = (E == -6) & (n < 8)
    ebits = np.where(is_sub, 0, E + 7)
    mbits = np.where(is_sub, n, n - 8)
    code = (ebits.astype(np.int64) << 3) | mbits.astype(np.int64)
    code = np.where(sat | (code > 0x7E), 0x7E, code)
    code = np.where(a == 0, 0, code)
    return (code.astype(np.uint8) | (sign << np.uint8(7))).astype(np.uint8)


# ---------------------------------------------------------------------------
# E8M0
# ---------------------------------------------------------------------------

def e8m0_decode(codes):
    """Decode E8M0 bytes to float64 powers of two; 0xFF decodes to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    v = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, v)


# ---------------------------------------------------------------------------
# bfloat16
# ---------------------------------------------------------------------------

def bf16_round_bits(y):
    """Round float64 values to bfloat16 (RNE, single rounding), return uint16 bits.

    bfloat16 keeps 8 significant bits. For normal results the significand is
    scaled to an 8-bit integer range and rounded with ties to even; below the
    smallest normal (2^-126) the quantum is fixed at 2^-133. Results beyond
    the largest finite bfloat16 become infinity, as in IEEE rounding.
    """
    y = np.asarray(y, dtype=np.float64)
    f, e = np.frexp(y)                              # y = f * 2^e, |f| in [0.5, 1)
    normal = (e - 1) >= -126
    r_norm = np.ldexp(np.rint(np.ldexp(f, 8)), (e - 8).astype(np.int64))
    r_sub = np.rint(np.ldexp(y, 133)) * 2.0 ** -133
    r = np.where(normal, r_norm, r_sub)
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > bf16_max, np.copysign(np.inf, y), r)
    r = np.where(np.isnan(y), np.nan, r)
    bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return bits


def bf16_bits_to_f64(bits):
    """Decode bfloat16 bit patterns (uint16) to float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(bits):
    """Decode bfloat16 bit patterns (uint16) to float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)
