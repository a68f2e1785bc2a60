"""MXFP4 quantizer and W4A4 linear layer (oracle; test infrastructure).

Only tests/, the smoke check and bench.py's CPU baseline use this module;
the HIP path shares no code with it.

The B12X write-up ("B12X quantized linear backends for SM12x",
Implementation: the five linear kernels) lists MXFP4 beside NVFP4, with the
activation quantized dynamically at run time. The element and scale formats
are the OCP Microscaling v1.0 ones: E2M1 elements and one E8M0 (power of two)
scale per 32 consecutive elements along K, no global scale.

Quantizer X(x) -> (codes, scales), per 32-element block:
  X1  a = max |v_i| (exact).
  X2  shared exponent E = floor(log2 a) - 2 (2 is the largest E2M1 exponent:
      6 = 1.5 * 2^2), clamped to [-127, 127]; a = 0 gives E = -127.
      The scale byte is E + 127 (E8M0: value 2^(byte - 127)).
  X3  q_i = E2M1_RNE_satfinite(v_i * 2^-E), sign copied from v_i. The product
      is one IEEE float32 multiply by a power of two (exact unless the result
      is subnormal, where it rounds once like any float32 multiply).
  X4  byte j of a row = q[2j] | q[2j+1] << 4; scales row-major [rows, K/32].
Reading (the pages do not define the exponent choice): the OCP rule above,
which maps the block maximum into [4, 8) so that values above 6 saturate to
6. The alternative ceil(log2(a / 6)) never saturates but is not the OCP rule;
only the OCP rule is used here.

Linear L(x_q, w_q, alpha, bias) -> y:
  L1  x_hat = e2m1(q) * 2^E (exact in float64), same for w_hat.
  L2  y64 = alpha * (x_hat @ w_hat^T) + bias, float64 (alpha = 1 unless given).
  L3  y = bfloat16_RNE(y64).
"""

import numpy as np

from . import formats as F

MX_BLOCK = 32
E2M1_EMAX = 2


def shared_exponent(amax):
    """X2: E = floor(log2 amax) - 2 clamped to [-127, 127]; amax = 0 -> -127."""
    a = np.asarray(amax, dtype=np.float64)
    mant, exp = np.frexp(np.where(a > 0, a, 1.0))  # a = mant * 2^exp, mant in [0.5, 1)
    e = exp.astype(np.int64) - 1 - E2M1_EMAX
    e = np.where(a > 0, e, -127)
    return np.clip(e, -127, 127)


def quant_mxfp4(x):
    """X1-X4 on float32 x [rows, K] (K % 32 == 0) -> (codes u8 [rows, K/2], scales u8 [rows, K/32])."""
    x = np.asarray(x, dtype=np.float32)
    rows, K = x.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = x.reshape(rows, K // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=2)
    E = shared_exponent(amax)
    # one float32 multiply by the exact power of two 2^-E (float64 product, one rounding)
    scaled = (blocks.astype(np.float64) * np.ldexp(1.0, -E)[:, :, None]).astype(np.float32)
    q = F.e2m1_encode(scaled).reshape(rows, K)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    scales = (E + 127).astype(np.uint8)
    return codes, scales


def dequant_mxfp4(codes, scales):
    """L1: exact float64 values e2m1(q) * 2^(byte - 127), shape [rows, K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, half = codes.shape
    q = np.empty((rows, half * 2), dtype=np.uint8)
    q[:, 0::2] = codes & 15
    q[:, 1::2] = codes >> 4
    vals = F.e2m1_decode(q).astype(np.float64)
    s = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return vals * np.repeat(s, MX_BLOCK, axis=1)


def linear_mxfp4_f64(x_codes, x_scales, w_codes, w_scales, alpha=1.0, bias=None):
    """L1-L2: float64 y64 = alpha * x_hat @ w_hat^T + bias."""
    xh = dequant_mxfp4(x_codes, x_scales)
    wh = dequant_mxfp4(w_codes, w_scales)
    y = float(alpha) * (xh @ wh.T)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y


def linear_mxfp4(x_codes, x_scales, w_codes, w_scales, alpha=1.0, bias=None):
    """L1-L3: bfloat16 bits of the layer output."""
    return F.bf16_round_bits(linear_mxfp4_f64(x_codes, x_scales, w_codes, w_scales, alpha, bias))
