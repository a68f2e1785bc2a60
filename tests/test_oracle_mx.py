"""Pins for the MXFP4 oracle (oracle/mx.py), CPU only.

Each check ties the oracle to something other than itself: closed forms of
the shared exponent, exact round trips of representable blocks, the
round-to-nearest error bound, saturation, an independent scalar re-derivation
in plain Python floats, and the GEMM against math.fsum.
"""

import math

import numpy as np
import pytest

from oracle import formats as F
from oracle import mx as X

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


@pytest.mark.parametrize("amax,expect", [
    (6.0, 0), (4.0, 0), (7.99, 0), (8.0, 1), (3.99, -1), (1.0, -2), (0.75, -3),
    (2.0 ** -100, -102), (2.0 ** -124, -126), (2.0 ** -125, -127), (2.0 ** -140, -127),
    (0.0, -127), (3.0e38, 125), (2.0 ** 127, 125)])
def test_shared_exponent_closed_form(amax, expect):
    # floor(log2 amax) - 2, clamped to [-127, 127]
    assert int(X.shared_exponent(np.float32(amax))) == expect


def test_block_max_maps_into_4_to_8():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    codes, scales = X.quant_mxfp4(x)
    amax = np.abs(x.reshape(64, 8, 32)).max(axis=2).astype(np.float64)
    ratio = amax / np.ldexp(1.0, scales.astype(np.int64) - 127)
    assert np.all((ratio >= 4.0) & (ratio < 8.0))


@pytest.mark.parametrize("E", [-20, -3, 0, 5, 40])
def test_exact_round_trip_of_representable_blocks(E):
    rng = np.random.default_rng(E + 100)
    mags = np.array(E2M1)
    c = rng.choice(mags, size=(8, 64)) * rng.choice([-1.0, 1.0], size=(8, 64))
    c[:, ::32] = 6.0  # block maximum 6 (or 4) -> exponent exactly E
    c[::2, ::32] = -4.0
    x = (c * 2.0 ** E).astype(np.float32)
    codes, scales = X.quant_mxfp4(x)
    assert np.all(scales == E + 127)
    back = X.dequant_mxfp4(codes, scales)
    assert np.array_equal(back, x.astype(np.float64))


def test_saturation_above_six():
    # block max in (6, 8) * 2^E rounds/saturates to +-6 * 2^E
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 7.9
    x[0, 1] = -6.5
    x[0, 2] = 5.0  # tie between 4 and 6 -> even code (4)
    x[0, 3] = 5.01
    codes, scales = X.quant_mxfp4(x)
    assert scales[0, 0] == 127
    q = np.empty(32, dtype=np.uint8)
    q[0::2] = codes[0] & 15
    q[1::2] = codes[0] >> 4
    assert list(q[:4]) == [7, 15, 6, 7]


def test_zero_block_and_signed_zero():
    x = np.zeros((2, 32), dtype=np.float32)
    x[1, 5] = -1e-30  # far below the block's quantum: rounds to -0
    x[1, 6] = 1.0
    codes, scales = X.quant_mxfp4(x)
    assert scales[0, 0] == 0 and np.all(codes[0] == 0)
    q5 = (codes[1, 2] >> 4) & 15
    assert q5 == 8


def test_error_bound():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((32, 512)).astype(np.float32)
    codes, scales = X.quant_mxfp4(x)
    deq = X.dequant_mxfp4(codes, scales)
    s = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
    a = np.abs(x.astype(np.float64)) / s
    half_gap = np.where(a <= 2.0, 0.25, np.where(a <= 4.0, 0.5, 1.0))
    err = np.abs(x - deq) / s
    unsat = a <= 6.0
    assert np.all(err[unsat] <= half_gap[unsat] + 1e-12)
    assert np.all(np.abs(deq[~unsat]) / s[~unsat] == 6.0)


def _scalar_quant(row):
    """Independent re-derivation in plain Python floats (no numpy arithmetic)."""
    out_q, out_s = [], []
    for b in range(len(row) // 32):
        blk = [float(v) for v in row[32 * b: 32 * b + 32]]
        a = max(abs(v) for v in blk)
        if a == 0.0:
            E = -127
        else:
            m, e = math.frexp(a)
            E = max(-127, min(127, e - 1 - 2))
        out_s.append(E + 127)
        for v in blk:
            u = float(np.float32(v * 2.0 ** (-E)))
            best = None
            for code, mag in enumerate(E2M1):
                d = abs(abs(u) - mag)
                if best is None or d < best[0] or (d == best[0] and code % 2 == 0 and best[1] % 2 == 1):
                    best = (d, code)
            if abs(u) > 6.0:
                best = (0.0, 7)
            sign = 8 if math.copysign(1.0, u) < 0 else 0
            out_q.append(best[1] | sign)
    return out_q, out_s


def test_matches_scalar_rederivation():
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((4, 96)) * np.exp(rng.uniform(-5, 5, (4, 1)))).astype(np.float32)
    x[0, :32] = 0.0
    codes, scales = X.quant_mxfp4(x)
    for r in range(4):
        q, s = _scalar_quant(x[r])
        got = np.empty(96, dtype=np.uint8)
        got[0::2] = codes[r] & 15
        got[1::2] = codes[r] >> 4
        assert list(got) == q
        assert list(scales[r]) == s


def test_gemm_matches_fsum():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((4, 64)).astype(np.float32)
    w = (rng.standard_normal((6, 64)) * 0.05).astype(np.float32)
    xc, xs = X.quant_mxfp4(x)
    wc, ws = X.quant_mxfp4(w)
    y = X.linear_mxfp4_f64(xc, xs, wc, ws)
    xh, wh = X.dequant_mxfp4(xc, xs), X.dequant_mxfp4(wc, ws)
    for m in range(4):
        for n in range(6):
            ref = math.fsum(float(xh[m, k]) * float(wh[n, k]) for k in range(64))
            assert y[m, n] == pytest.approx(ref, rel=1e-15, abs=1e-300)


def test_identity_weight_closed_form():
    rng = np.random.default_rng(9)
    K = 64
    x = rng.standard_normal((3, K)).astype(np.float32)
    xc, xs = X.quant_mxfp4(x)
    eye = np.eye(K, dtype=np.float32)
    wc, ws = X.quant_mxfp4(eye)
    bias = rng.standard_normal(K) * 0.1
    y = X.linear_mxfp4_f64(xc, xs, wc, ws, alpha=2.0, bias=bias)
    assert np.allclose(y, 2.0 * X.dequant_mxfp4(xc, xs) + bias[None, :], rtol=0, atol=1e-12)
