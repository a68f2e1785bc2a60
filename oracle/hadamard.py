"""Block-diagonal Sylvester Hadamard rotation (oracle; test infrastructure).

Source: "QUTLASS NVFP4 online transforms" write-up, motivation and
implementation sections: activations are rotated by a block-diagonal
transform before NVFP4 quantization, the transform block size is one of
16, 32, 64, 128, and the normalisation 1/sqrt(n) is folded into the matrix
(HadamardTransform key code: the stored partition is divided by sqrt(n)).
The dense branch of that module applies the rotation as a plain GEMM.

Readings where the page is silent:
* The Hadamard matrix is Sylvester's construction in natural order,
  H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]], so H[i][j] = (-1)^popcount(i & j).
* It is applied per row and per b-element chunk as the radix-2 fast
  Walsh-Hadamard transform in float32, butterfly strides h = 1, 2, 4, ...,
  b/2 in ascending order, each butterfly writing (a + b, a - b); the 1/sqrt(b)
  factor is one float32 multiply at the end by c_b = fl32(1/sqrt(b)).
  This fixes every float32 rounding, which bit-exact code parity needs.

Pins (tests/test_oracle_hadamard.py): H_b H_b^T = b I in integers; the
normalised rows have unit norm; the FWHT matches the dense float64 product
H_b v / sqrt(b) within the float32 error bound; (xH)(WH)^T = x W^T; chunks are
independent.
"""

import numpy as np

HADAMARD_BLOCKS = (16, 32, 64, 128)


def sylvester(b):
    """Integer Sylvester Hadamard matrix of order b (a power of two)."""
    if b < 1 or (b & (b - 1)) != 0:
        raise ValueError("order must be a power of two")
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < b:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_scale_fp32(b):
    """c_b = 1/sqrt(b) rounded once to float32."""
    return np.float32(1.0 / np.sqrt(np.float64(b)))


def fwht_fp32(v, b):
    """Rotate each b-element chunk of every row of v (float32 [..., K]).

    Returns a new float32 array: per chunk H_b v / sqrt(b), with the
    float32 operation order described in the module docstring.
    """
    v = np.array(v, dtype=np.float32, copy=True)
    K = v.shape[-1]
    if b not in HADAMARD_BLOCKS:
        raise ValueError("hadamard block must be one of 16, 32, 64, 128")
    if K % b != 0:
        raise ValueError("K must be a multiple of the hadamard block")
    lead = v.shape[:-1]
    w = v.reshape(-1, K // b, b)
    h = 1
    while h < b:
        # pair element i (with (i mod 2h) < h) with i + h
        w4 = w.reshape(w.shape[0], w.shape[1], b // (2 * h), 2, h)
        lo = w4[:, :, :, 0, :].copy()
        hi = w4[:, :, :, 1, :].copy()
        w4[:, :, :, 0, :] = lo + hi
        w4[:, :, :, 1, :] = lo - hi
        h *= 2
    w = w * hadamard_scale_fp32(b)
    return w.reshape(*lead, K).astype(np.float32)
