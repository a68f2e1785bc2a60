"""NVFP4 quantizer and W4A4 linear layer (oracle; test infrastructure).

What the layer computes, per the three vLLM write-ups:
* "TorchNvFp4LinearKernel", key code (apply_weights): the activation is
  quantized to packed FP4 bytes plus block scales using the layer's input
  global scale; the scaled GEMM multiplies it with the pre-packed weight;
  the result is multiplied by alpha, described as the product of the
  activation and weight global dequant scales; padded output columns are
  dropped; the bias is added last; the output keeps the input dtype and the
  shape [*x.shape[:-1], N]. Two FP4 values share one byte.
* "QUTLASS NVFP4 online transforms": the quantizer may first rotate the
  activation by a block-diagonal Hadamard transform (see hadamard.py), and
  its outputs are an E2M1 code tensor and an E4M3 scale tensor written into
  caller-provided buffers.
* "B12X CuTe-DSL linear backends", NVFP4 key code: the same sequence, with
  alpha handed to the GEMM and the bias added afterwards; strided (non
  contiguous) activations are quantized without a copy.

Quantizer Q(x, g, b) -> (codes, scales), steps in order:
  Q0  v = float32(x) (exact from bfloat16).
  Q1  if b > 0: v = FWHT_b(v) / sqrt(b) per chunk (hadamard.py).
  Q2  per 16-element block: a = max |v_i| (exact).
  Q3  s_f = fl32(fl32(a / 6) * g); s = E4M3_RNE_satfinite(s_f); s_d = decode(s).
  Q4  r = fl32(g / s_d) (correctly rounded division), r = 0 when s_d = 0.
  Q5  q_i = E2M1_RNE_satfinite(fl32(v_i * r)), sign copied from v_i.
  Q6  byte j of a row = q[2j] | q[2j+1] << 4; scales row-major [M, K/16].
Readings (the pages are silent on these): the 16-element block, E4M3 block
scales and the float32 global scale g = 448*6/amax; the operation order in
Q3 and Q4; RNE with saturation; even element in the low nibble.

GEMM G(x_q, w_q, alpha, bias) -> y:
  G1  x_hat = e2m1(q) * s_d per element (exact in float64), same for w_hat.
  G2  y64 = alpha * (x_hat @ w_hat^T) + bias, float64.
  G3  y = bfloat16_RNE(y64).

Pins (tests/test_oracle_nvfp4.py): global-scale invariant (the amax block
gets scale 448 and code +-6), exact round trip of representable blocks,
per-element error bound, all-zero / underflowing / saturating / subnormal
blocks, a scalar pure-Python re-derivation on small random inputs, the
GEMM against math.fsum brute force, and the epilogue closed form with an
identity weight.
"""

import numpy as np

from .formats import (
    bf16_round_bits,
    e2m1_decode,
    e2m1_encode,
    e4m3_decode,
    e4m3_encode,
)
from .hadamard import fwht_fp32

NVFP4_BLOCK = 16
E2M1_MAX = 6.0
E4M3_MAX = 448.0
GLOBAL_SCALE_MAX = 2.0 ** 118


def amax_for_calibration(x, hadamard_block=0):
    """max |v| over the whole tensor after the optional rotation (float32)."""
    v = np.asarray(x, dtype=np.float32)
    if hadamard_block:
        v = fwht_fp32(v, hadamard_block)
    return np.float32(np.max(np.abs(v))) if v.size else np.float32(0)


def global_scale_from_amax(amax):
    """g = fl32(448 * 6 / amax); g = 1 when amax is zero; at most 2^118.

    The cap (ours; the pages give only 448 * 6 / amax) binds only for amax
    below 2688 * 2^-118, a tensor of values near the float32 subnormal range.
    It keeps Q4's r = g / s_d finite for every nonzero E4M3 scale (the
    smallest is 2^-9), so no product in Q5 meets an infinity.
    """
    amax = np.float32(amax)
    if amax == 0:
        return np.float32(1.0)
    with np.errstate(over="ignore"):
        g = np.float32(np.float32(E4M3_MAX * E2M1_MAX) / amax)
    return np.float32(min(float(g), GLOBAL_SCALE_MAX))


def pack_nibbles(q):
    """Pack E2M1 codes [..., K] into bytes [..., K/2], even element low."""
    q = np.asarray(q, dtype=np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << np.uint8(4))).astype(np.uint8)


def unpack_nibbles(p):
    """Inverse of pack_nibbles: bytes [..., K/2] -> codes [..., K]."""
    p = np.asarray(p, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & np.uint8(0xF)
    out[..., 1::2] = p >> np.uint8(4)
    return out


def quant_nvfp4(x, global_scale, hadamard_block=0):
    """NVFP4-quantize rows of x ([M, K], bfloat16-valued or float32).

    Returns (codes uint8 [M, K/2], scales uint8 [M, K/16] E4M3).
    """
    v = np.asarray(x, dtype=np.float32)
    if v.ndim != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = v.shape
    if K % NVFP4_BLOCK != 0:
        raise ValueError("K must be a multiple of 16")
    g = np.float32(global_scale)
    # Q1
    if hadamard_block:
        v = fwht_fp32(v, hadamard_block)
    blocks = v.reshape(M, K // NVFP4_BLOCK, NVFP4_BLOCK)
    # Q2
    a = np.max(np.abs(blocks), axis=-1)
    # Q3
    s_f = (a / np.float32(6.0)) * g
    s = e4m3_encode(s_f)
    s_d = e4m3_decode(s).astype(np.float32)
    # Q4
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s_d == 0, np.float32(0.0), g / s_d).astype(np.float32)
    # Q5
    u = (blocks * r[..., None]).astype(np.float32)
    q = e2m1_encode(u).reshape(M, K)
    # Q6
    return pack_nibbles(q), s


def dequant_nvfp4(codes, scales):
    """x_hat[m, k] = e2m1(q[m, k]) * s_d[m, k // 16] in float64 (exact)."""
    q = unpack_nibbles(codes)
    M, K = q.shape
    s = e4m3_decode(scales)
    return e2m1_decode(q) * np.repeat(s, NVFP4_BLOCK, axis=1)[:, :K]


def linear_nvfp4(x_codes, x_scales, w_codes, w_scales, alpha, bias=None):
    """y = bfloat16_RNE(alpha * x_hat @ w_hat^T + bias), returned as uint16 bits.

    x_codes [M, K/2], x_scales [M, K/16], w_codes [N, K/2], w_scales [N, K/16],
    alpha a float scalar (the caller's float32 value), bias None or float64
    values [N] (decoded bfloat16).
    """
    y64 = linear_nvfp4_f64(x_codes, x_scales, w_codes, w_scales, alpha, bias)
    return bf16_round_bits(y64)


def linear_nvfp4_f64(x_codes, x_scales, w_codes, w_scales, alpha, bias=None):
    """The float64 value of the linear layer before the bfloat16 cast."""
    return linear_dequantized_f64(dequant_nvfp4(x_codes, x_scales),
                                  dequant_nvfp4(w_codes, w_scales), alpha, bias)


def linear_dequantized_f64(x_hat, w_hat, alpha, bias=None):
    """G2 on operands already decoded by G1 (float64 x_hat [M, K], w_hat [N, K])."""
    y = np.float64(alpha) * (np.asarray(x_hat, np.float64) @ np.asarray(w_hat, np.float64).T)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y
