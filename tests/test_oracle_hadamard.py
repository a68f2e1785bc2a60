"""Pins for the oracle's block-diagonal Hadamard rotation (CPU).

The write-up on QUTLASS online transforms fixes the block sizes
{16, 32, 64, 128}, the block-diagonal structure and the 1/sqrt(n)
normalisation; the tests tie the float32 FWHT to integer identities of the
Sylvester matrix, to the dense float64 product (the module's dense GEMM
branch) and to the invariance that makes the rotation free for the layer.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle.hadamard import HADAMARD_BLOCKS, fwht_fp32, hadamard_scale_fp32, sylvester


@pytest.mark.parametrize("b", HADAMARD_BLOCKS)
def test_sylvester_orthogonal_in_integers(b):
    h = sylvester(b)
    assert np.array_equal(h @ h.T, b * np.eye(b, dtype=np.int64))
    assert np.array_equal(h, h.T)
    # entry (i, j) = (-1)^popcount(i & j)
    i, j = np.meshgrid(np.arange(b), np.arange(b), indexing="ij")
    pc = np.vectorize(lambda t: bin(int(t)).count("1"))(i & j)
    assert np.array_equal(h, np.where(pc % 2 == 0, 1, -1))


@pytest.mark.parametrize("b", HADAMARD_BLOCKS)
def test_scale_is_nearest_float32_to_inverse_sqrt(b):
    c = hadamard_scale_fp32(b)
    # compare |c^2 b - 1| exactly against both float32 neighbours
    def err(v):
        f = Fraction(float(v))
        return abs(f * f * b - 1)
    lo = np.nextafter(c, np.float32(0))
    hi = np.nextafter(c, np.float32(1))
    assert err(c) <= err(lo) and err(c) <= err(hi)
    expected_bits = {16: 0x3E800000, 32: 0x3E3504F3, 64: 0x3E000000, 128: 0x3DB504F3}
    assert int(c.view(np.uint32)) == expected_bits[b]


@pytest.mark.parametrize("b", HADAMARD_BLOCKS)
def test_unit_vectors_map_to_scaled_rows(b):
    K = 2 * b
    eye = np.eye(K, dtype=np.float32)
    out = fwht_fp32(eye, b)
    h = sylvester(b).astype(np.float64) / np.sqrt(b)
    for j in range(K):
        chunk, r = divmod(j, b)
        expect = np.zeros(K)
        expect[chunk * b:(chunk + 1) * b] = h[r]
        # exact for b = 16, 64 (power-of-two scale); one float32 rounding otherwise
        assert np.allclose(out[j], expect, rtol=0, atol=1e-7)
        if b in (16, 64):
            assert np.array_equal(out[j].astype(np.float64), expect)


@pytest.mark.parametrize("b", HADAMARD_BLOCKS)
def test_fwht_matches_dense_product_within_fp32_bound(b):
    r = np.random.default_rng(b)
    v = r.standard_normal((64, 4 * b)).astype(np.float32)
    out = fwht_fp32(v, b).astype(np.float64)
    h = sylvester(b).astype(np.float64)
    exact = (v.astype(np.float64).reshape(64, 4, b) @ h.T / np.sqrt(b)).reshape(64, 4 * b)
    # log2(b) float32 add stages plus one multiply, each at most 2^-24 relative
    # of the running magnitude, which is bounded by sum |v_i| of the chunk
    bound = (np.log2(b) + 2) * 2.0 ** -24 * np.repeat(
        np.abs(v.astype(np.float64)).reshape(64, 4, b).sum(-1), b, axis=1)
    assert np.all(np.abs(out - exact) <= bound)


@pytest.mark.parametrize("b", HADAMARD_BLOCKS)
def test_parseval(b):
    r = np.random.default_rng(100 + b)
    v = r.standard_normal((32, 8 * b)).astype(np.float32)
    out = fwht_fp32(v, b)
    n_in = np.linalg.norm(v.astype(np.float64), axis=1)
    n_out = np.linalg.norm(out.astype(np.float64), axis=1)
    assert np.allclose(n_out, n_in, rtol=2e-6)


@pytest.mark.parametrize("b", HADAMARD_BLOCKS)
def test_rotation_cancels_in_the_layer(b):
    r = np.random.default_rng(200 + b)
    K = 4 * b
    x = r.standard_normal((8, K))
    w = r.standard_normal((16, K))
    h = np.kron(np.eye(K // b), sylvester(b).astype(np.float64) / np.sqrt(b))
    lhs = (x @ h.T) @ (w @ h.T).T
    rhs = x @ w.T
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_chunks_are_independent():
    b = 32
    r = np.random.default_rng(9)
    v = r.standard_normal((4, 4 * b)).astype(np.float32)
    base = fwht_fp32(v, b)
    v2 = v.copy()
    v2[:, 2 * b:3 * b] += np.float32(1.0)
    pert = fwht_fp32(v2, b)
    keep = np.r_[0:2 * b, 3 * b:4 * b]
    assert np.array_equal(base[:, keep], pert[:, keep])
    assert not np.array_equal(base[:, 2 * b:3 * b], pert[:, 2 * b:3 * b])


def test_rejects_bad_block():
    with pytest.raises(ValueError):
        fwht_fp32(np.zeros((1, 48), np.float32), 24)
    with pytest.raises(ValueError):
        fwht_fp32(np.zeros((1, 48), np.float32), 32)
