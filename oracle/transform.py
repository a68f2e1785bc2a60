"""General block-diagonal transform before NVFP4 quantization, and the dynamic
activation global scale (oracle; test infrastructure).

Only tests/, the smoke check and bench.py's CPU baseline use this module;
the HIP path shares no code with it.

Source: "QUTLASS NVFP4 online transforms" write-up.
* Motivation: the fused quantizer accepts any block-diagonal transform, not
  only a deterministic Hadamard matrix.
* Implementation, weight post-processing: the transform matrix is read from
  the layer's input-transform weight (one b x b partition, b in
  {16, 32, 64, 128}) and handed to the fused quantizer with the activation.
* HadamardTransform key code: the normalisation 1/sqrt(n) is folded into the
  stored matrix once at load time, and the dense branch applies the matrix
  to the activation as an ordinary linear layer, i.e. x @ T^T per chunk.

Steps, per row of x and per b-element chunk c:
  T1  v[c*b + i] = fl32( sum_j T[i][j] * x[c*b + j] ): the sum of the exact
      products, rounded once to float32. An exactly zero sum is +0.
  T2  the NVFP4 quantizer steps Q2-Q6 (nvfp4.py) on v with global scale g.
Dynamic activation global scale (the same write-up names the global scale a
per-call input of the fused quantizer; computing it from the activation is
the in-kernel option):
  D1  a = max |v| over the whole tensor, v after T1 (or after the Hadamard
      rotation, or x itself without a transform).
  D2  g = fl32(2688 / a) (2688 = 448 * 6), g = 1 when a = 0, capped at
      2^118 (a below 2688 * 2^-118).
  D3  alpha = fl32((1 / g_x) * (1 / g_w)) evaluated in float64.

Readings (the pages are silent on these):
* T holds bfloat16 values: the write-up drops the partition's explicit
  dtype, so it takes the model's dtype.
* T1 rounds the exact sum once (the plainest float32 result). A fused kernel
  accumulates in float32 in its own order, so its v may differ from T1 in
  the last bits. Codes and scales are then compared by a near-tie rule:
  each value the kernel produces must be a correct rounding of some number
  within the kernel's accumulation bound eps * sum_j |T[i][j] x[j]| of the
  exact sum (see transform_abs_sum), and the share of elements that differ
  from the oracle is capped.
* D2's cap is ours: without it a tensor of tiny values gives g = inf (or a
  g so large that r = g / s_d overflows in Q4) and 0 * inf = NaN in Q5. At
  2^118, r stays finite for every nonzero E4M3 scale (the smallest is 2^-9).

T1 as computed here: a float64 matmul of the exactly widened operands, then
one rounding to float32. Each product is exact in float64 (at most 8 + 24
significant bits). The float64 sum errs by at most b * 2^-53 of sum |T x|,
2^-29 * b below float32's half unit, so it can move the float32 result only
for sums within that distance of a float32 rounding midpoint; the pin
against an exact rational evaluation checks it on random inputs.

Pins (tests/test_oracle_transform.py): identity T reproduces the plain
quantizer, the Sylvester matrix times fl32(1/sqrt(b)) reproduces the
Hadamard quantizer on inputs whose FWHT sums are exact, a permutation
matrix permutes the input, a power-of-two diagonal scales it, exact
rational evaluation on small random cases, chunk independence, the
dynamic-scale invariant (the tensor's largest element gets scale 448 and
code +-6), and the zero / overflow cases of D2.
"""

import numpy as np

from .formats import bf16_round_bits, bf16_bits_to_f64
from .nvfp4 import global_scale_from_amax, quant_nvfp4

TRANSFORM_BLOCKS = (16, 32, 64, 128)


def _check(x, T):
    x = np.asarray(x)
    T = np.asarray(T, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("x must be 2-D [M, K]")
    b = T.shape[0]
    if T.shape != (b, b) or b not in TRANSFORM_BLOCKS:
        raise ValueError("T must be b x b with b in {16, 32, 64, 128}")
    if x.shape[1] % b:
        raise ValueError("K must be a multiple of the transform block")
    return b


def bf16_matrix(T):
    """Round a float matrix to bfloat16 values (float64 array of those values)."""
    return bf16_bits_to_f64(bf16_round_bits(np.asarray(T, dtype=np.float64)))


def transform_f64(x, T):
    """The exact per-chunk products summed in float64: [M, K] float64 (before T1's rounding)."""
    b = _check(x, T)
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    M, K = x64.shape
    chunks = x64.reshape(M, K // b, b)
    return (chunks @ np.asarray(T, dtype=np.float64).T).reshape(M, K)


def block_transform(x, T):
    """T1: v = fl32(sum_j T[i][j] x[j]) per chunk, float32 [M, K]; zero sums are +0."""
    return (transform_f64(x, T) + 0.0).astype(np.float32)


def transform_abs_sum(x, T):
    """sum_j |T[i][j] * x[j]| per output element, float64 [M, K] (the scale of
    a float32 accumulation's rounding error)."""
    b = _check(x, T)
    x64 = np.abs(np.asarray(x, dtype=np.float32).astype(np.float64))
    M, K = x64.shape
    return (x64.reshape(M, K // b, b) @ np.abs(np.asarray(T, np.float64)).T).reshape(M, K)


def quant_nvfp4_transform(x, T, global_scale):
    """T1 then T2: (codes uint8 [M, K/2], scales uint8 [M, K/16])."""
    return quant_nvfp4(block_transform(x, T), global_scale)


def dynamic_global_scale(amax):
    """D2: g = fl32(2688 / a); 1 when a == 0; at most 2^118 (the static
    calibration rule of nvfp4.py, applied per call)."""
    return global_scale_from_amax(amax)


def dynamic_alpha(g_x, g_w):
    """D3: alpha = fl32((1 / g_x) * (1 / g_w)) in float64."""
    return np.float32((1.0 / np.float64(np.float32(g_x))) * (1.0 / np.float64(np.float32(g_w))))


def tensor_amax(v):
    """D1: max |v| over the whole float32 tensor (0 for an empty one)."""
    v = np.asarray(v, dtype=np.float32)
    return np.float32(np.max(np.abs(v))) if v.size else np.float32(0)
