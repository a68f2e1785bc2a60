"""Pins for the oracle's element formats (CPU).

Each encoder is checked against something other than itself: an independent
nearest-value brute force over the format's decode table, a library cast
(torch.float8_e4m3fn, torch.bfloat16) where one exists, the hand-listed tie
table, and exact round trips.
"""

import numpy as np
import pytest
import torch

from oracle import formats as F

# E2M1 magnitudes as the OCP MX v1.0 FP4 definition gives them
# (also quoted in the method statement: {0, 0.5, 1, 1.5, 2, 3, 4, 6}).
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _all_bf16_as_f32():
    bits = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    v = bits.view(np.float32)
    return v[np.isfinite(v)]


def _around(points, n_ulps, dtype=np.float32):
    pts = np.asarray(points, dtype=dtype)
    out = [pts]
    lo = pts.copy()
    hi = pts.copy()
    for _ in range(n_ulps):
        lo = np.nextafter(lo, dtype(-np.inf))
        hi = np.nextafter(hi, dtype(np.inf))
        out += [lo, hi]
    return np.concatenate(out)


def _brute_e2m1(u):
    """Nearest E2M1 magnitude by exhaustive distance, ties to the even code."""
    u = np.asarray(u, dtype=np.float32)
    a = np.abs(u.astype(np.float64))
    mags = np.array(E2M1_TABLE)
    d = np.abs(a[:, None] - mags[None, :])
    best = np.min(d, axis=1)
    cand = d == best[:, None]
    # among tied candidates pick the even code; a tie always has exactly one
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    code = np.where(cand.sum(1) > 1, np.argmax(even, axis=1), np.argmax(cand, axis=1))
    code = np.where(a > 6.0, 7, code)  # saturate
    sign = (u.view(np.uint32) >> 31).astype(np.int64)
    return (code | (sign << 3)).astype(np.uint8)


def test_e2m1_decode_table():
    for c in range(8):
        assert F.e2m1_decode(np.uint8(c)) == E2M1_TABLE[c]
        assert F.e2m1_decode(np.uint8(c | 8)) == -E2M1_TABLE[c]


def test_e2m1_round_trip_all_codes():
    codes = np.arange(16, dtype=np.uint8)
    vals = F.e2m1_decode(codes).astype(np.float32)
    vals[8] = np.float32(-0.0)  # code 0x8 is negative zero
    assert np.array_equal(F.e2m1_encode(vals), codes)


def test_e2m1_ties_by_hand():
    # (value, expected magnitude code): ties go to the even code
    table = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
             (0.2500001, 1), (0.7499999, 1), (5.0000005, 7), (6.0, 7), (7.0, 7), (1e30, 7),
             (np.inf, 7)]
    for v, c in table:
        assert F.e2m1_encode(np.float32(v)) == c, v
        assert F.e2m1_encode(np.float32(-v)) == (c | 8), -v


def test_e2m1_negative_zero_keeps_sign():
    assert F.e2m1_encode(np.float32(-0.0)) == 0x8
    assert F.e2m1_encode(np.float32(-0.1)) == 0x8
    assert F.e2m1_encode(np.float32(0.0)) == 0x0


def test_e2m1_vs_brute_force():
    thresholds = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]
    near = _around(thresholds, 300)
    r = np.random.default_rng(123)
    rand = r.uniform(-8, 8, size=400_000).astype(np.float32)
    allbf = _all_bf16_as_f32()
    allbf = allbf[np.abs(allbf) < 1e6]
    u = np.concatenate([near, -near, rand, allbf])
    assert np.array_equal(F.e2m1_encode(u), _brute_e2m1(u))


# ---------------------------------------------------------------------------
# E4M3
# ---------------------------------------------------------------------------

def _e4m3_table():
    """All 127 non-negative finite E4M3 values by field decomposition."""
    vals = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            if e == 0:
                vals.append((e << 3 | m, m * 2.0 ** -9))
            else:
                vals.append((e << 3 | m, (1 + m / 8.0) * 2.0 ** (e - 7)))
    return vals


def _brute_e4m3(x):
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x.astype(np.float64))
    tab = _e4m3_table()
    codes = np.array([c for c, _ in tab])
    vals = np.array([v for _, v in tab])
    out = np.empty(a.shape, dtype=np.int64)
    for i in range(0, a.size, 20000):
        blk = a[i:i + 20000]
        d = np.abs(blk[:, None] - vals[None, :])
        best = d.min(1)
        cand = d == best[:, None]
        even = cand & (codes[None, :] % 2 == 0)
        pick = np.where(cand.sum(1) > 1, np.argmax(even, 1), np.argmax(cand, 1))
        out[i:i + 20000] = codes[pick]
    out = np.where(a > 448.0, 0x7E, out)
    sign = (x.view(np.uint32) >> 31).astype(np.int64)
    return (out | (sign << 7)).astype(np.uint8)


def test_e4m3_decode_known_points():
    assert F.e4m3_decode(np.uint8(0x7E)) == 448.0
    assert F.e4m3_decode(np.uint8(0x01)) == 2.0 ** -9
    assert F.e4m3_decode(np.uint8(0x08)) == 2.0 ** -6
    assert F.e4m3_decode(np.uint8(0x38)) == 1.0
    assert np.isnan(F.e4m3_decode(np.uint8(0x7F)))
    assert np.isnan(F.e4m3_decode(np.uint8(0xFF)))
    assert F.e4m3_decode(np.uint8(0xFE)) == -448.0


def test_e4m3_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = F.e4m3_decode(codes).astype(np.float32)
    vals[codes == 0x80] = np.float32(-0.0)
    assert np.array_equal(F.e4m3_encode(vals), codes)


def test_e4m3_vs_torch_cast_in_range():
    tab = np.array([v for _, v in _e4m3_table()])
    mids = (tab[1:] + tab[:-1]) / 2
    near = _around(np.concatenate([mids, tab]).astype(np.float32), 40)
    r = np.random.default_rng(7)
    rand = np.concatenate([r.uniform(0, 464, 300_000), np.exp(r.uniform(-12, 6.1, 300_000))])
    allbf = _all_bf16_as_f32()
    x = np.concatenate([near, rand.astype(np.float32), allbf]).astype(np.float32)
    x = x[(np.abs(x) <= 464.0)]
    x = np.concatenate([x, -x])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_encode(x), ref)


def test_e4m3_vs_brute_force():
    r = np.random.default_rng(11)
    x = np.concatenate([np.exp(r.uniform(-14, 7, 100_000)), r.uniform(0, 600, 20_000)])
    x = x.astype(np.float32)
    assert np.array_equal(F.e4m3_encode(x), _brute_e4m3(x))


def test_e4m3_saturates():
    for v in (448.0, 464.0, 464.0001, 500.0, 1e6, 3e38, np.inf):
        assert F.e4m3_encode(np.float32(v)) == 0x7E
        assert F.e4m3_encode(np.float32(-v)) == 0xFE


def test_e4m3_subnormal_boundaries():
    assert F.e4m3_encode(np.float32(2.0 ** -10)) == 0x00       # tie -> even (0)
    assert F.e4m3_encode(np.float32(1.5 * 2.0 ** -10)) == 0x01
    assert F.e4m3_encode(np.float32(7.5 * 2.0 ** -9)) == 0x08  # rounds into the normals
    assert F.e4m3_encode(np.float32(6.5 * 2.0 ** -9)) == 0x06  # tie -> even


# ---------------------------------------------------------------------------
# E8M0
# ---------------------------------------------------------------------------

def test_e8m0_decode():
    assert F.e8m0_decode(np.uint8(127)) == 1.0
    assert F.e8m0_decode(np.uint8(0)) == 2.0 ** -127
    assert F.e8m0_decode(np.uint8(254)) == 2.0 ** 127
    assert np.isnan(F.e8m0_decode(np.uint8(255)))


# ---------------------------------------------------------------------------
# bfloat16
# ---------------------------------------------------------------------------

def test_bf16_round_matches_torch_for_float32_inputs():
    r = np.random.default_rng(5)
    x = np.concatenate([
        r.standard_normal(200_000).astype(np.float32) * np.float32(1e3),
        np.exp(r.uniform(-100, 88, 100_000)).astype(np.float32),
        _around(np.array([1.0, 1.0 + 2 ** -8, 3.0, 1e-38, 2e-40]), 5),
    ]).astype(np.float32)
    x = np.concatenate([x, -x])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.bf16_round_bits(x.astype(np.float64)), ref)


def test_bf16_round_is_single_rounding_from_f64():
    # 1 + 2^-8 + 2^-40 lies just above the midpoint of 1 and 1 + 2^-7:
    # one rounding goes up; rounding through float32 first would tie to 1.0.
    y = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert F.bf16_round_bits(y) == 0x3F81
    assert F.bf16_round_bits(1.0 + 2.0 ** -8) == 0x3F80
    assert F.bf16_round_bits(-(1.0 + 2.0 ** -8 + 2.0 ** -40)) == 0xBF81


def test_bf16_round_overflow_and_zero():
    assert F.bf16_round_bits(1e39) == 0x7F80
    assert F.bf16_round_bits(-1e39) == 0xFF80
    assert F.bf16_round_bits(0.0) == 0x0000
    assert F.bf16_round_bits(-0.0) == 0x8000


@pytest.mark.parametrize("bits", [0x0000, 0x3F80, 0xC2F7, 0x0001, 0x7F7F])
def test_bf16_decode(bits):
    ref = torch.tensor([bits], dtype=torch.int32).to(torch.int16).view(torch.bfloat16).double().item()
    assert F.bf16_bits_to_f64(np.uint16(bits)) == ref
