"""Pins for the oracle's general block-diagonal transform and dynamic global
scale (CPU).

The QUTLASS online-transforms write-up says the fused quantizer takes any
block-diagonal transform (b in {16, 32, 64, 128}) with the normalisation
folded into the matrix, and its dense branch applies the matrix as a linear
layer. The pins tie T1 to matrices whose effect is known exactly (identity,
permutation, power-of-two diagonal, the normalised Sylvester matrix against
the independently pinned Hadamard quantizer), to exact rational arithmetic,
and tie the dynamic scale D1-D3 to its defining invariant and edge cases.
"""

from fractions import Fraction

import numpy as np
import pytest

import synthetic
from oracle.formats import bf16_bits_to_f64, e2m1_decode
from oracle.hadamard import hadamard_scale_fp32, sylvester
from oracle.nvfp4 import global_scale_from_amax, quant_nvfp4, unpack_nibbles
from oracle.transform import (
    TRANSFORM_BLOCKS,
    block_transform,
    dynamic_alpha,
    dynamic_global_scale,
    quant_nvfp4_transform,
    tensor_amax,
    transform_abs_sum,
    transform_f64,
)


def _x(M, K, seed=0, kind="student_t3"):
    return synthetic.bf16_bits_to_f32(synthetic.activations(kind, M, K, config="transform", seed=seed))


def _T(b, kind="orthogonal", seed=0):
    return bf16_bits_to_f64(synthetic.transform_matrix(b, kind, seed))


@pytest.mark.parametrize("b", TRANSFORM_BLOCKS)
def test_identity_reproduces_plain_quantizer(b):
    x = _x(5, 4 * b, seed=b)
    g = global_scale_from_amax(tensor_amax(x))
    c0, s0 = quant_nvfp4(x, g)
    c1, s1 = quant_nvfp4_transform(x, np.eye(b), g)
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
    assert np.array_equal(block_transform(x, np.eye(b)).view(np.uint32), x.view(np.uint32))


def test_zero_sums_are_positive_zero():
    b = 16
    x = np.zeros((2, 32), np.float32)
    x[0, :] = -0.0
    x[1, 3] = 1.5
    x[1, 4] = -1.5
    T = np.zeros((b, b))
    T[0, 3] = 1.0
    T[0, 4] = 1.0  # x3 + x4 = 0 exactly
    T[1, 0] = 1.0  # picks -0 from row 0
    v = block_transform(x, T)
    assert np.all(v == 0) and not np.any(np.signbit(v))
    codes, scales = quant_nvfp4_transform(x, T, 1.0)
    assert not np.any(codes) and not np.any(scales)


@pytest.mark.parametrize("b", (16, 64))
def test_normalised_sylvester_matches_hadamard_quantizer(b):
    # For b = 16, 64 the normalisation 1/sqrt(b) is a power of two, so the
    # matrix is exact in bfloat16; on inputs that are small multiples of 1/4
    # every FWHT partial sum is exact, so both evaluations give the same floats.
    T = sylvester(b).astype(np.float64) * float(hadamard_scale_fp32(b))
    assert np.array_equal(bf16_bits_to_f64(synthetic.f32_to_bf16_bits(T.astype(np.float32))), T)
    g = synthetic.rng(9, b)
    x = (g.integers(-24, 25, size=(6, 4 * b)) * 0.25).astype(np.float32)
    gs = np.float32(37.5)
    c0, s0 = quant_nvfp4(x, gs, hadamard_block=b)
    c1, s1 = quant_nvfp4_transform(x, T, gs)
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)


@pytest.mark.parametrize("b", TRANSFORM_BLOCKS)
def test_permutation_moves_elements(b):
    # v[i] = x[perm[i]] within each chunk; a non-symmetric permutation catches
    # a transposed matrix.
    perm = synthetic.rng(10, b).permutation(b)
    P = np.zeros((b, b))
    P[np.arange(b), perm] = 1.0
    assert not np.array_equal(P, P.T)
    x = _x(3, 3 * b, seed=1)
    v = block_transform(x, P)
    expect = x.reshape(3, 3, b)[:, :, perm].reshape(3, 3 * b)
    assert np.array_equal(v, expect)


@pytest.mark.parametrize("b", TRANSFORM_BLOCKS)
def test_power_of_two_diagonal_scales(b):
    e = synthetic.rng(11, b).integers(-4, 5, size=b)
    D = np.diag(np.ldexp(1.0, e))
    x = _x(2, 2 * b, seed=2)
    v = block_transform(x, D)
    expect = np.ldexp(x.astype(np.float64).reshape(2, 2, b), e[None, None, :]).reshape(2, 2 * b)
    assert np.array_equal(v.astype(np.float64), expect)


def _round_f32_exact(q):
    """Round a Fraction to the nearest float32, ties to even (normal range)."""
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    # a in [2^e, 2^(e+1)): 24 significant bits
    scaled = a / Fraction(2) ** (e - 23)
    n = round(scaled)  # Fraction.__round__ rounds half to even
    return np.float32(sign * float(Fraction(n) * Fraction(2) ** (e - 23)))


@pytest.mark.parametrize("b,kind", [(16, "orthogonal"), (32, "gaussian"), (64, "orthogonal")])
def test_against_exact_rational_sum(b, kind):
    T = _T(b, kind, seed=3)
    x = _x(2, 2 * b, seed=4)
    v = block_transform(x, T)
    for m in range(2):
        for c in range(2):
            for i in range(b):
                s = sum((Fraction(float(T[i, j])) * Fraction(float(x[m, c * b + j])) for j in range(b)),
                        Fraction(0))
                assert v[m, c * b + i] == _round_f32_exact(s), (m, c, i)


def test_abs_sum_bounds_the_sum():
    b = 32
    T = _T(b, "gaussian", seed=5)
    x = _x(4, 4 * b, seed=6)
    assert np.all(np.abs(transform_f64(x, T)) <= transform_abs_sum(x, T))
    xp, Tp = np.abs(x), np.abs(T)
    assert np.allclose(transform_f64(xp, Tp), transform_abs_sum(x, T), rtol=1e-15, atol=0)


def test_chunks_are_independent():
    b = 32
    T = _T(b, seed=7)
    x = _x(3, 4 * b, seed=8)
    v0 = block_transform(x, T)
    x2 = x.copy()
    x2[:, 2 * b:3 * b] *= np.float32(-3.0)
    v1 = block_transform(x2, T)
    same = np.ones(4 * b, bool)
    same[2 * b:3 * b] = False
    assert np.array_equal(v0[:, same], v1[:, same])
    assert not np.array_equal(v0[:, ~same], v1[:, ~same])


def test_orthogonal_transform_preserves_norms():
    b = 128
    T = _T(b, "orthogonal", seed=12)
    x = _x(4, 2 * b, seed=13, kind="normal")
    v = block_transform(x, T).astype(np.float64)
    nx = np.linalg.norm(x.astype(np.float64).reshape(-1, b), axis=1)
    nv = np.linalg.norm(v.reshape(-1, b), axis=1)
    # bfloat16 rounding of an orthogonal matrix: relative error ~ 2^-8 * sqrt(b)-ish
    assert np.allclose(nv, nx, rtol=2e-2)


@pytest.mark.parametrize("b,seed", [(16, 0), (64, 1), (128, 2)])
def test_dynamic_scale_puts_amax_on_the_grid_edge(b, seed):
    # g = 2688 / amax makes the largest element's block scale 448 (E4M3 0x7E)
    # and its code +-6 (magnitude code 7), whatever the rounding of g.
    T = _T(b, seed=seed)
    x = _x(7, 2 * b, seed=seed)
    v = block_transform(x, T)
    a = tensor_amax(v)
    g = dynamic_global_scale(a)
    codes, scales = quant_nvfp4(v, g)
    m, k = np.unravel_index(np.argmax(np.abs(v)), v.shape)
    assert scales[m, k // 16] == 0x7E
    q = unpack_nibbles(codes)[m, k]
    assert q & 7 == 7 and e2m1_decode(np.uint8(q)) == np.copysign(6.0, v[m, k])


def test_dynamic_scale_edge_cases():
    assert dynamic_global_scale(np.float32(2688.0)) == np.float32(1.0)
    assert dynamic_global_scale(np.float32(0.0)) == np.float32(1.0)
    assert dynamic_global_scale(np.float32(1.0)) == np.float32(2688.0)
    cap = np.float32(2.0 ** 118)
    assert dynamic_global_scale(np.float32(2688.0) / cap) == cap
    for tiny in (np.float32(1e-34), np.float32(1e-38)):  # 2688 / tiny exceeds the cap
        g = dynamic_global_scale(tiny)
        assert g == cap
        # the block then quantizes to finite codes and scales, never NaN:
        # r = g / s_d is finite for every nonzero E4M3 scale
        v = np.full((1, 32), tiny, np.float32)
        v[0, 16:] = 0.0
        codes, scales = quant_nvfp4(v, g)
        q = unpack_nibbles(codes)
        assert np.all(q[0, 16:] == 0) and scales[0, 1] == 0
        if tiny == np.float32(1e-34):
            assert scales[0, 0] != 0 and np.all(q[0, :16] == 7)
        else:  # fl32(tiny / 6) * g is below half the smallest E4M3 step
            assert scales[0, 0] == 0 and np.all(q[0, :16] == 0)
    assert tensor_amax(np.zeros((0, 16), np.float32)) == 0


def test_dynamic_alpha_closed_form():
    assert dynamic_alpha(2.0, 4.0) == np.float32(0.125)
    gx, gw = np.float32(3.0), np.float32(7.0)
    assert dynamic_alpha(gx, gw) == np.float32(1.0 / 21.0)
