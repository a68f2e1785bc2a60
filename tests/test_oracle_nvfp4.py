"""Pins for the oracle's NVFP4 quantizer and linear layer (CPU).

Ties the oracle to what the pages and the arithmetic fix, not to itself:
* a scalar, pure-Python re-derivation of the quantizer (nearest-of-table
  encoders, CPython float32 rounding via struct) on small random inputs;
* the global-scale invariant (the block holding the tensor amax is scaled to
  448 and that element encodes to +-6);
* exact round trip of blocks built from representable values;
* the per-element error bound of round-to-nearest;
* special blocks: all zero, underflowing scale, saturating, subnormal scale;
* the GEMM against a math.fsum brute force, the epilogue closed form with an
  identity weight, and the end-to-end quantization error as information.
"""

import math
import struct

import numpy as np
import pytest

import synthetic
from oracle import formats as F
from oracle import nvfp4 as Q
from oracle.hadamard import sylvester

# ---------------------------------------------------------------------------
# independent scalar re-derivation
# ---------------------------------------------------------------------------


def fl32(x):
    return struct.unpack("<f", struct.pack("<f", x))[0]


_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
_E4M3 = []
for _e in range(16):
    for _m in range(8):
        if _e == 15 and _m == 7:
            continue
        _E4M3.append((_e << 3 | _m, _m * 2.0 ** -9 if _e == 0 else (1 + _m / 8) * 2.0 ** (_e - 7)))


def _nearest(a, table):
    """(code, value) nearest to a >= 0; ties -> even code."""
    best = None
    for code, val in table:
        d = abs(a - val)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code, val)
    return best[1], best[2]


def scalar_e2m1(u):
    a = abs(u)
    code = 7 if a > 6.0 else _nearest(a, list(enumerate(_E2M1)))[0]
    neg = math.copysign(1.0, u) < 0
    return code | (8 if neg else 0)


def scalar_e4m3(s):
    if s > 448.0:
        return 0x7E, 448.0
    return _nearest(s, _E4M3)


def scalar_fwht(v, b):
    v = list(v)
    h = 1
    while h < b:
        for i in range(b):
            if i % (2 * h) < h:
                a, c = v[i], v[i + h]
                v[i], v[i + h] = fl32(a + c), fl32(a - c)
        h *= 2
    cb = fl32(1.0 / math.sqrt(b))
    return [fl32(t * cb) for t in v]


def scalar_quant(row, g, b):
    row = [fl32(float(t)) for t in row]
    if b:
        row = [t for i in range(0, len(row), b) for t in scalar_fwht(row[i:i + b], b)]
    codes, scales = [], []
    for i in range(0, len(row), 16):
        blk = row[i:i + 16]
        amax = max(abs(t) for t in blk)
        s_f = fl32(fl32(amax / 6.0) * g)
        s_code, s_d = scalar_e4m3(s_f)
        r = 0.0 if s_d == 0 else fl32(g / s_d)
        scales.append(s_code)
        codes += [scalar_e2m1(fl32(t * r)) for t in blk]
    packed = [codes[2 * j] | (codes[2 * j + 1] << 4) for j in range(len(codes) // 2)]
    return packed, scales


@pytest.mark.parametrize("b", [0, 16, 32, 64])
@pytest.mark.parametrize("gmode", ["calibrated", "small", "large"])
def test_quant_matches_scalar_rederivation(b, gmode):
    r = np.random.default_rng(1000 + b)
    x = r.standard_normal((3, 128)).astype(np.float32)
    x[0, :16] *= np.float32(1e-3)   # a quiet block
    x[1, 16:32] = 0.0               # an all-zero block
    x[1, 33] = np.float32(-0.0)
    x[2, 40] = np.float32(30.0)     # an outlier
    amax = Q.amax_for_calibration(x, b)
    g = {"calibrated": Q.global_scale_from_amax(amax),
         "small": np.float32(0.37), "large": np.float32(9000.0)}[gmode]
    codes, scales = Q.quant_nvfp4(x, g, b)
    for m in range(3):
        pc, sc = scalar_quant(x[m], float(g), b)
        assert list(codes[m]) == pc
        assert list(scales[m]) == sc


def test_quant_bf16_inputs_match_scalar():
    xb = synthetic.activations("student_t3", 4, 256, config="hadamard")
    x = synthetic.bf16_bits_to_f32(xb)
    for b in (0, 128):
        g = Q.global_scale_from_amax(Q.amax_for_calibration(x, b))
        codes, scales = Q.quant_nvfp4(x, g, b)
        for m in range(4):
            pc, sc = scalar_quant(x[m], float(g), b)
            assert list(codes[m]) == pc and list(scales[m]) == sc


# ---------------------------------------------------------------------------
# properties fixed by the format definitions
# ---------------------------------------------------------------------------


def test_nibble_order_even_element_low():
    q = np.array([[1, 2, 0xF, 0x8]], dtype=np.uint8)
    assert list(Q.pack_nibbles(q)[0]) == [0x21, 0x8F]
    assert np.array_equal(Q.unpack_nibbles(Q.pack_nibbles(q)), q)


@pytest.mark.parametrize("seed", range(5))
def test_global_scale_invariant(seed):
    r = np.random.default_rng(seed)
    x = (r.standard_normal((8, 512)) * r.uniform(0.01, 100)).astype(np.float32)
    amax = Q.amax_for_calibration(x)
    g = Q.global_scale_from_amax(amax)
    codes, scales = Q.quant_nvfp4(x, g)
    q = Q.unpack_nibbles(codes)
    m, k = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert scales[m, k // 16] == 0x7E
    assert q[m, k] & 7 == 7
    assert np.all(scales <= 0x7E)


@pytest.mark.parametrize("logg", [-3, 0, 5])
def test_exact_round_trip_of_representable_blocks(logg):
    r = np.random.default_rng(50 + logg)
    g = np.float32(2.0 ** logg)
    n_blocks = 400
    # scales spanning subnormal and normal E4M3 codes
    s_codes = r.integers(1, 0x7F, n_blocks).astype(np.uint8)
    s_d = F.e4m3_decode(s_codes)
    c = r.integers(0, 16, (n_blocks, 16)).astype(np.uint8)
    c[c == 8] = 0                       # no negative zero in the construction
    c[:, 0] = np.where(r.random(n_blocks) < 0.5, 7, 15)  # block max magnitude 6
    v = F.e2m1_decode(c) * s_d[:, None] / float(g)
    x = v.reshape(1, -1).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), v.reshape(1, -1))  # exact in float32
    codes, scales = Q.quant_nvfp4(x, g)
    assert np.array_equal(scales[0], s_codes)
    assert np.array_equal(Q.unpack_nibbles(codes)[0], c.reshape(-1))


def test_error_bound_round_to_nearest():
    r = np.random.default_rng(77)
    x = r.standard_normal((64, 1024)).astype(np.float32)
    g = Q.global_scale_from_amax(Q.amax_for_calibration(x))
    codes, scales = Q.quant_nvfp4(x, g)
    q = Q.unpack_nibbles(codes)
    val = F.e2m1_decode(q)
    s_d = np.repeat(F.e4m3_decode(scales), 16, axis=1)
    half_gap = np.select([np.abs(val) <= 1.5, np.abs(val) <= 3.0], [0.25, 0.5], 1.0)
    err = np.abs(x.astype(np.float64) - val * s_d / float(g))
    normal_scale = s_d >= 2.0 ** -6
    bound = half_gap * s_d / float(g) * (1 + 2.0 ** -20)
    assert np.all(err[normal_scale] <= bound[normal_scale])
    assert normal_scale.mean() > 0.99


def test_all_zero_block():
    x = np.zeros((2, 32), np.float32)
    x[1, :16] = -0.0
    codes, scales = Q.quant_nvfp4(x, np.float32(5.0))
    assert np.all(scales == 0)
    q = Q.unpack_nibbles(codes)
    assert np.all(q[0] == 0) and np.all(q[1, :16] == 8) and np.all(q[1, 16:] == 0)


def test_underflowing_scale_gives_signed_zeros():
    x = np.zeros((1, 16), np.float32)
    x[0, :8] = 1e-4
    x[0, 8:] = -1e-4
    g = np.float32(0.05)   # s_f = 1e-4/6*0.05 < 2^-10 -> scale 0
    codes, scales = Q.quant_nvfp4(x, g)
    assert scales[0, 0] == 0
    q = Q.unpack_nibbles(codes)[0]
    assert np.all(q[:8] == 0) and np.all(q[8:] == 8)


def test_saturating_global_scale():
    r = np.random.default_rng(3)
    x = r.standard_normal((4, 64)).astype(np.float32)
    g = np.float32(50.0) * Q.global_scale_from_amax(Q.amax_for_calibration(x))
    codes, scales = Q.quant_nvfp4(x, g)
    assert np.all(scales == 0x7E)
    q = Q.unpack_nibbles(codes)
    m, k = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert q[m, k] & 7 == 7
    assert (q & 7 == 7).mean() > 0.5


def test_subnormal_scales_forced():
    r = np.random.default_rng(4)
    x = r.standard_normal((4, 64)).astype(np.float32)
    g = np.float32(0.02)   # block amax/6*g ~ 1e-2 .. 1e-3 -> E4M3 subnormals
    codes, scales = Q.quant_nvfp4(x, g)
    assert np.any((scales & 0x78) == 0) and np.any(scales > 0)
    for m in range(4):
        pc, sc = scalar_quant(x[m], float(g), 0)
        assert list(codes[m]) == pc and list(scales[m]) == sc


def test_global_scale_zero_amax():
    assert Q.global_scale_from_amax(0.0) == 1.0
    assert Q.global_scale_from_amax(np.float32(2688.0)) == 1.0


# ---------------------------------------------------------------------------
# GEMM and epilogue
# ---------------------------------------------------------------------------


def _tiny_case():
    xb = synthetic.activations("normal", 16, 256, config="tiny")
    x = synthetic.bf16_bits_to_f32(xb)
    w = synthetic.weight(512, 256, config="tiny")
    gx = Q.global_scale_from_amax(Q.amax_for_calibration(x))
    gw = Q.global_scale_from_amax(Q.amax_for_calibration(w))
    xc, xs = Q.quant_nvfp4(x, gx)
    wc, ws = Q.quant_nvfp4(w, gw)
    alpha = np.float32((1.0 / np.float64(gx)) * (1.0 / np.float64(gw)))
    return x, w, xc, xs, wc, ws, alpha


def test_gemm_matches_fsum_brute_force():
    x, w, xc, xs, wc, ws, alpha = _tiny_case()
    bias = synthetic.bias(512, config="tiny")
    bias64 = F.bf16_bits_to_f64(bias)
    y64 = Q.linear_nvfp4_f64(xc, xs, wc, ws, alpha, bias64)
    xq, wq = Q.unpack_nibbles(xc), Q.unpack_nibbles(wc)
    xsd, wsd = F.e4m3_decode(xs), F.e4m3_decode(ws)
    e2 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]

    def dq(c, s):
        v = e2[c & 7] * s
        return -v if c & 8 else v

    rows = range(0, 16, 3)
    cols = range(0, 512, 37)
    for m in rows:
        xr = [dq(int(xq[m, k]), float(xsd[m, k // 16])) for k in range(256)]
        for n in cols:
            wr = [dq(int(wq[n, k]), float(wsd[n, k // 16])) for k in range(256)]
            acc = math.fsum(a * b for a, b in zip(xr, wr))  # products exact in float64
            ref = float(alpha) * acc + float(bias64[n])
            assert abs(y64[m, n] - ref) <= 1e-13 * max(1.0, abs(ref))


def test_epilogue_closed_form_identity_weight():
    r = np.random.default_rng(21)
    K = 64
    x = r.standard_normal((5, K)).astype(np.float32)
    gx = Q.global_scale_from_amax(Q.amax_for_calibration(x))
    xc, xs = Q.quant_nvfp4(x, gx)
    # identity weight: code 2 (1.0) on the diagonal, E4M3 scale 0x38 (1.0)
    wq = np.zeros((K, K), np.uint8)
    np.fill_diagonal(wq, 2)
    wc = Q.pack_nibbles(wq)
    ws = np.full((K, K // 16), 0x38, np.uint8)
    alpha = np.float32(0.0625)
    bias = r.standard_normal(K)
    y = Q.linear_nvfp4(xc, xs, wc, ws, alpha, bias)
    expect = F.bf16_round_bits(0.0625 * Q.dequant_nvfp4(xc, xs) + bias[None, :])
    # compare values: the sign of a zero output carries no meaning
    assert np.array_equal(F.bf16_bits_to_f64(y), F.bf16_bits_to_f64(expect))
    # and without bias the output is alpha * x_hat, exactly
    y0 = Q.linear_nvfp4(xc, xs, wc, ws, alpha)
    expect0 = F.bf16_round_bits(0.0625 * Q.dequant_nvfp4(xc, xs))
    assert np.array_equal(F.bf16_bits_to_f64(y0), F.bf16_bits_to_f64(expect0))


def test_quantization_error_vs_unquantized_is_modest():
    x, w, xc, xs, wc, ws, alpha = _tiny_case()
    y64 = Q.linear_nvfp4_f64(xc, xs, wc, ws, alpha)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    rel = np.linalg.norm(y64 - ref) / np.linalg.norm(ref)
    # NVFP4 on Gaussian data: information only, a loose sanity window
    assert 0.02 < rel < 0.25


def test_hadamard_layer_invariance_through_quantization():
    # rotating both operands keeps the unquantized product; the quantized
    # layer stays close to it
    r = np.random.default_rng(31)
    b = 32
    K, N, M = 128, 64, 8
    x = r.standard_t(3, (M, K)).astype(np.float32)
    w = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    gx = Q.global_scale_from_amax(Q.amax_for_calibration(x, b))
    from oracle.hadamard import fwht_fp32
    wr = fwht_fp32(w, b)
    gw = Q.global_scale_from_amax(Q.amax_for_calibration(wr))
    xc, xs = Q.quant_nvfp4(x, gx, b)
    wc, ws = Q.quant_nvfp4(wr, gw)
    alpha = np.float32(1.0 / (np.float64(gx) * np.float64(gw)))
    y = Q.linear_nvfp4_f64(xc, xs, wc, ws, alpha)
    h = np.kron(np.eye(K // b), sylvester(b) / np.sqrt(b))
    assert np.allclose((x @ h.T) @ (w @ h.T).T, x.astype(np.float64) @ w.T, rtol=1e-5, atol=1e-6)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 0.25


# ---------------------------------------------------------------------------
# calibration amax after the rotation ("QUTLASS NVFP4 online transforms",
# Implementation: the block-diagonal rotation is applied before quantization,
# so the global scale is calibrated on rotated values)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("b", [16, 32, 64, 128])
def test_calibration_amax_is_that_of_the_dense_rotation(b):
    # against the dense float64 product (H_b / sqrt(b)) v per chunk, within the
    # FWHT's float32 error bound (log2(b) add stages and one multiply)
    r = np.random.default_rng(700 + b)
    K = 8 * b
    x = synthetic.bf16_bits_to_f32(synthetic.f32_to_bf16_bits(
        r.standard_t(3, size=(24, K)).astype(np.float32)))
    h = sylvester(b).astype(np.float64) / np.sqrt(b)
    dense = (x.astype(np.float64).reshape(24, K // b, b) @ h.T).reshape(24, K)
    bound = (np.log2(b) + 2) * 2.0 ** -24 * np.abs(x.astype(np.float64)).reshape(
        24, K // b, b).sum(-1).max()
    got = float(Q.amax_for_calibration(x, b))
    assert abs(got - np.abs(dense).max()) <= bound
    # the rotation changes the answer for these inputs, so skipping it fails
    assert abs(float(Q.amax_for_calibration(x, 0)) - np.abs(dense).max()) > 100 * bound


@pytest.mark.parametrize("b", [16, 32, 64, 128])
def test_calibration_amax_closed_form_constant_chunk(b):
    # a chunk of equal values c rotates to (c * b, 0, ..., 0) / sqrt(b): the FWHT
    # sums are exact, so the rotated amax is fl32(fl32(c * b) * fl32(1/sqrt(b)))
    c = np.float32(0.75)
    x = np.zeros((3, 4 * b), np.float32)
    x[1, 2 * b:3 * b] = c
    x[2, :b] = -c / 2
    cb = np.float32(1.0 / np.sqrt(np.float64(b)))
    expect = np.float32(np.float32(c * b) * cb)
    assert Q.amax_for_calibration(x, b) == expect
    if b in (16, 64):  # 1/sqrt(b) is a power of two: exactly c * sqrt(b)
        assert float(expect) == 0.75 * math.sqrt(b)


@pytest.mark.parametrize("b", [16, 32, 64, 128])
def test_calibrated_rotated_scale_hits_the_format_maximum(b):
    # global-scale invariant on rotated values: the block holding the rotated
    # amax gets scale 448 (0x7E) and that element code +-6
    r = np.random.default_rng(800 + b)
    x = (r.standard_t(3, size=(16, 4 * b)) * 3).astype(np.float32)
    g = Q.global_scale_from_amax(Q.amax_for_calibration(x, b))
    codes, scales = Q.quant_nvfp4(x, g, b)
    h = sylvester(b).astype(np.float64) / np.sqrt(b)
    dense = (x.astype(np.float64).reshape(16, 4, b) @ h.T).reshape(16, 4 * b)
    m, k = np.unravel_index(np.argmax(np.abs(dense)), dense.shape)
    assert scales[m, k // 16] == 0x7E
    assert Q.unpack_nibbles(codes)[m, k] & 7 == 7
    assert np.all(scales <= 0x7E)
