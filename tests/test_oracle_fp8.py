"""Pins for the FP8 oracles (oracle/fp8.py), CPU only.

Each check ties the oracle to something other than itself: closed forms of
the MX shared exponent, exact round trips of representable values, the
round-to-nearest error bound, saturation, group independence, an independent
scalar re-derivation in plain Python (nearest of the E4M3 value table, built
from the format's definition), and the GEMMs against math.fsum.
"""

import math
import struct

import numpy as np
import pytest

from oracle import fp8 as P


def _e4m3_table():
    """All finite non-negative E4M3 values by code, from the definition."""
    vals = []
    for code in range(0x7F):  # 0x7F is NaN
        e, m = code >> 3, code & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return vals


E4M3 = _e4m3_table()


def _f32(v):
    return struct.unpack("f", struct.pack("f", v))[0]


def _e4m3_nearest(u):
    """Independent encoder: nearest table value, ties to the even code, saturating."""
    a = abs(u)
    best = None
    for code, val in enumerate(E4M3):
        d = abs(a - val)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    code = best[1]
    if a > 448.0:
        code = 0x7E
    return code | (0x80 if math.copysign(1.0, u) < 0 else 0)


# ---------------------------------------------------------------------------
# MXFP8
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("amax,expect", [
    (448.0, 0), (256.0, 0), (511.9, 0), (512.0, 1), (255.9, -1), (1.0, -8), (2.0 ** -100, -108),
    (2.0 ** -118, -126), (2.0 ** -119, -127), (2.0 ** -149, -127), (0.0, -127), (3.0e38, 119)])
def test_mx8_shared_exponent_closed_form(amax, expect):
    assert int(P.mx8_shared_exponent(np.float32(amax))) == expect


def test_mx8_block_max_maps_into_256_to_512():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((32, 256)) * np.exp(rng.uniform(-30, 30, (32, 1)))).astype(np.float32)
    _, s = P.quant_mxfp8(x)
    amax = np.abs(x.reshape(32, 8, 32)).max(axis=2).astype(np.float64)
    ratio = amax / np.ldexp(1.0, s.astype(np.int64) - 127)
    assert np.all((ratio >= 256.0) & (ratio < 512.0))


@pytest.mark.parametrize("E", [-30, -4, 0, 3, 60])
def test_mx8_exact_round_trip(E):
    rng = np.random.default_rng(E + 50)
    vals = np.array(E4M3[:0x7F])
    c = rng.choice(vals[vals <= 448], size=(6, 64)) * rng.choice([-1.0, 1.0], size=(6, 64))
    c[:, ::32] = 448.0  # block maximum in [256, 512) -> exponent exactly E
    x = (c * 2.0 ** E).astype(np.float32)
    # subnormal E4M3 values times 2^E may fall below float32's range for very negative E
    assume = np.all(x.astype(np.float64) == c * 2.0 ** E)
    codes, s = P.quant_mxfp8(x)
    assert np.all(s == E + 127)
    if assume:
        assert np.array_equal(P.dequant_mxfp8(codes, s), x.astype(np.float64))


def test_mx8_saturation_and_ties():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 500.0     # in [464, 512): saturates to 448
    x[0, 1] = -470.0
    x[0, 2] = 460.0     # rounds to 448 (nearest)
    x[0, 3] = 17.0      # tie between 16 and 18 -> even mantissa (16)
    x[0, 4] = 19.0      # tie between 18 and 20 -> 20 (mantissa 2 is even)
    codes, s = P.quant_mxfp8(x)
    assert s[0, 0] == 127
    assert list(codes[0, :5]) == [0x7E, 0xFE, 0x7E, 0x58, 0x5A]


def test_mx8_matches_scalar_rederivation():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((3, 64)) * np.exp(rng.uniform(-8, 8, (3, 1)))).astype(np.float32)
    x[1, :32] = 0.0
    codes, s = P.quant_mxfp8(x)
    for r in range(3):
        for b in range(2):
            blk = [float(v) for v in x[r, 32 * b:32 * b + 32]]
            a = max(abs(v) for v in blk)
            E = -127 if a == 0 else max(-127, min(127, math.frexp(a)[1] - 1 - 8))
            assert s[r, b] == E + 127
            for i, v in enumerate(blk):
                assert codes[r, 32 * b + i] == _e4m3_nearest(_f32(v * 2.0 ** -E))


def test_mx8_gemm_matches_fsum():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 96)).astype(np.float32)
    w = (rng.standard_normal((5, 96)) * 0.05).astype(np.float32)
    xc, xs = P.quant_mxfp8(x)
    wc, ws = P.quant_mxfp8(w)
    y = P.linear_mxfp8_f64(xc, xs, wc, ws, alpha=0.5)

    def dec(c, s, k):
        code = int(c[k])
        v = E4M3[code & 0x7F] * (-1 if code & 0x80 else 1)
        return v * 2.0 ** (int(s[k // 32]) - 127)

    for m in range(3):
        for n in range(5):
            ref = 0.5 * math.fsum(dec(xc[m], xs[m], k) * dec(wc[n], ws[n], k) for k in range(96))
            assert y[m, n] == pytest.approx(ref, rel=1e-14, abs=1e-300)


# ---------------------------------------------------------------------------
# block FP8
# ---------------------------------------------------------------------------

def test_block_act_scalar_rederivation_and_group_max():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((3, 256)) * np.exp(rng.uniform(-6, 6, (3, 1)))).astype(np.float32)
    x[2, 128:] = 0.0
    codes, s = P.quant_fp8_block_act(x)
    assert s.dtype == np.float32 and s.shape == (3, 2)
    for m in range(3):
        for g in range(2):
            grp = [float(v) for v in x[m, 128 * g:128 * g + 128]]
            a = max(abs(v) for v in grp)
            sg = _f32(a / 448.0)
            assert s[m, g] == sg
            r = _f32(1.0 / sg) if sg > 0 else 0.0
            for i, v in enumerate(grp):
                assert codes[m, 128 * g + i] == _e4m3_nearest(_f32(v * r))
            if a > 0:
                # the group's largest element maps onto the largest E4M3 magnitude
                k = int(np.argmax(np.abs(x[m, 128 * g:128 * g + 128])))
                assert codes[m, 128 * g + k] & 0x7F == 0x7E


def test_block_groups_are_independent():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 384)).astype(np.float32)
    c0, s0 = P.quant_fp8_block_act(x)
    x2 = x.copy()
    x2[:, 128:256] *= 1000.0
    c1, s1 = P.quant_fp8_block_act(x2)
    assert np.array_equal(c0[:, :128], c1[:, :128]) and np.array_equal(c0[:, 256:], c1[:, 256:])
    assert np.array_equal(s0[:, [0, 2]], s1[:, [0, 2]])


def test_block_weight_tiles_and_error_bound():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    w[128:, 128:256] *= 50.0  # one tile with a much larger range
    codes, s = P.quant_fp8_block_weight(w)
    assert s.shape == (2, 3)
    for i in range(2):
        for j in range(3):
            t = w[128 * i:128 * i + 128, 128 * j:128 * j + 128]
            assert s[i, j] == _f32(float(np.abs(t).max()) / 448.0)
    deq = P.dequant_fp8_block_weight(codes, s)
    # RNE error: at most half a quantum of the value's binade, in units of the tile scale
    sfull = np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)
    u = np.abs(w.astype(np.float64)) / sfull
    quantum = np.ldexp(1.0, np.maximum(np.floor(np.log2(np.maximum(u, 1e-300))), -6).astype(np.int64) - 3)
    assert np.all(np.abs(deq - w) / sfull <= quantum / 2 * (1 + 1e-6) + 1e-12)


def test_block_gemm_is_the_per_group_promotion():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, 256)).astype(np.float32)
    w = (rng.standard_normal((128, 256)) * 0.03).astype(np.float32)
    xc, xs = P.quant_fp8_block_act(x)
    wc, ws = P.quant_fp8_block_weight(w)
    bias = rng.standard_normal(128) * 0.01
    y = P.linear_fp8_block_f64(xc, xs, wc, ws, bias)

    def dec(code):
        code = int(code)
        return E4M3[code & 0x7F] * (-1 if code & 0x80 else 1)

    for m in range(2):
        for n in (0, 5, 127):
            # integer-code partial sums per 128-group, promoted by sx * sw
            parts = []
            for g in range(2):
                p = math.fsum(dec(xc[m, k]) * dec(wc[n, k]) for k in range(128 * g, 128 * g + 128))
                parts.append(p * float(xs[m, g]) * float(ws[n // 128, g]))
            ref = math.fsum(parts) + bias[n]
            assert y[m, n] == pytest.approx(ref, rel=1e-13, abs=1e-15)


def test_block_zero_group():
    x = np.zeros((1, 128), np.float32)
    c, s = P.quant_fp8_block_act(x)
    assert s[0, 0] == 0 and np.all(c & 0x7F == 0)


# ---------------------------------------------------------------------------
# per-tensor FP8
# ---------------------------------------------------------------------------

def test_tensor_quant_scalar_rederivation():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((4, 64)).astype(np.float32) * 3
    s = P.scale_from_amax(np.abs(x).max())
    codes = P.quant_fp8_tensor(x, s)
    r = _f32(1.0 / float(s))
    for m in range(4):
        for k in range(64):
            assert codes[m, k] == _e4m3_nearest(_f32(float(x[m, k]) * r))
    assert np.max(codes & 0x7F) == 0x7E


def test_tensor_linear_matches_fsum_and_alpha():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((3, 128)).astype(np.float32)
    w = (rng.standard_normal((4, 128)) * 0.02).astype(np.float32)
    sx = P.scale_from_amax(np.abs(x).max())
    sw = P.scale_from_amax(np.abs(w).max())
    alpha = P.output_scale(sx, sw)
    assert alpha == _f32(float(sx) * float(sw))
    xc, wc = P.quant_fp8_tensor(x, sx), P.quant_fp8_tensor(w, sw)
    y = P.linear_fp8_tensor_f64(xc, wc, alpha)

    def dec(code):
        code = int(code)
        return E4M3[code & 0x7F] * (-1 if code & 0x80 else 1)

    for m in range(3):
        for n in range(4):
            ref = float(alpha) * math.fsum(dec(xc[m, k]) * dec(wc[n, k]) for k in range(128))
            assert y[m, n] == pytest.approx(ref, rel=1e-14)
    # and the quantized product approximates the float product (FP8 error level)
    yf = x.astype(np.float64) @ w.T.astype(np.float64)
    assert np.linalg.norm(y - yf) / np.linalg.norm(yf) < 0.05


def test_block_subnormal_group_uses_largest_finite_reciprocal():
    # a group of float32 subnormals: 1/s overflows, r is the largest finite float32
    x = np.zeros((1, 128), np.float32)
    x[0, :] = np.float32(1e-39)
    x[0, 7] = np.float32(-3e-39)
    x[0, 9] = 0.0
    c, s = P.quant_fp8_block_act(x)
    assert 0 < float(s[0, 0]) < 2.0 ** -126
    r = float(np.finfo(np.float32).max)
    for k in (0, 7, 9):
        assert c[0, k] == _e4m3_nearest(_f32(float(x[0, k]) * r))
    assert c[0, 9] == 0 and np.all(c & 0x7F != 0x7F)
