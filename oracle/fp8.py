"""FP8 (E4M3) siblings of the linear layer (oracle; test infrastructure).

Only tests/, the smoke check and bench.py's CPU baseline use this module;
the HIP path shares no code with it.

The B12X write-up ("B12X quantized linear backends for SM12x",
Implementation: the five linear kernels) lists three FP8 formats beside the
two FP4 ones. Elements are E4M3 ("fn": largest finite 448) in all three; they
differ in how the scale is shared:

MXFP8 (OCP Microscaling v1.0: one E8M0 scale per 32 consecutive elements
along K, activation quantized dynamically), per 32-block:
  M1  a = max |v_i|.
  M2  E = floor(log2 a) - 8 (8 is the largest E4M3 exponent: 448 = 1.75 *
      2^8), clamped to [-127, 127]; a = 0 gives E = -127. Scale byte E + 127.
  M3  q_i = E4M3_RNE_satfinite(fl32(v_i * 2^-E)) (one float32 multiply by a
      power of two), sign copied.
  Reading: the same OCP rule as the MXFP4 sibling; the block maximum lands in
  [256, 512), so magnitudes in [464, 512) * 2^E saturate to 448 * 2^E.

Block FP8 (write-up: activation groups of 1 x 128, weight groups of
128 x 128, feature dimensions multiples of 128, float32 scales; weight scales
stored as UE8M0 are widened to float32 before the GEMM), per group:
  B1  a = max |v| over the group.
  B2  s = fl32(a / 448) (float32 scale; a = 0 gives s = 0).
  B3  r = fl32(1 / s) (r = 0 when s = 0; the largest finite float32 when
      1 / s overflows, i.e. a group whose maximum is a float32 subnormal
      below 448 * 2^-128: its products v * r then stay finite).
  B4  q = E4M3_RNE_satfinite(fl32(v * r)), sign kept.
  Scales: activation [M][K/128], weight [N/128][K/128], float32.
  Reading: the pages give the group shapes and the float32 scale type but no
  scale rule; amax / 448 (the largest element maps onto the largest E4M3
  value) and the multiply by the rounded reciprocal are the plainest choice.
  The overflow rule of B3 is ours (the pages are silent; without it a
  subnormal group would multiply by infinity).

Per-tensor FP8 (write-up: the activation is quantized with a static
per-tensor scale and the two scales are merged into one output scale):
  T1  q = E4M3_RNE_satfinite(fl32(v * fl32(1 / s))) for a given float32 s > 0
      (calibration: s = fl32(amax / 448)).
  T2  output scale alpha = fl32(s_x * s_w).
  Reading: same reciprocal-multiply quantizer as B3-B4.

Linear, all three: y64 = (alpha *) sum_k x_hat[m][k] * w_hat[n][k] + bias in
float64 over the exactly decoded values (block FP8: x_hat = e4m3(q) * s of
the element's group, which is the per-group promotion written out), then
bf16_RNE(y64).
"""

import numpy as np

from . import formats as F

MX_BLOCK = 32
E4M3_EMAX = 8
FP8_GROUP = 128


def _f32(a):
    return np.asarray(a, dtype=np.float32)


# ---------------------------------------------------------------------------
# MXFP8
# ---------------------------------------------------------------------------

def mx8_shared_exponent(amax):
    """M2: floor(log2 amax) - 8 clamped to [-127, 127]; amax = 0 -> -127."""
    a = np.asarray(amax, dtype=np.float64)
    _, exp = np.frexp(np.where(a > 0, a, 1.0))
    e = np.where(a > 0, exp.astype(np.int64) - 1 - E4M3_EMAX, -127)
    return np.clip(e, -127, 127)


def quant_mxfp8(x):
    """M1-M3 on float32 x [rows, K] (K % 32 == 0) -> (codes u8 [rows, K], scales u8 [rows, K/32])."""
    x = _f32(x)
    rows, K = x.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = x.reshape(rows, K // MX_BLOCK, MX_BLOCK)
    E = mx8_shared_exponent(np.abs(blocks).max(axis=2))
    scaled = (blocks.astype(np.float64) * np.ldexp(1.0, -E)[:, :, None]).astype(np.float32)
    codes = F.e4m3_encode(scaled).reshape(rows, K)
    return codes, (E + 127).astype(np.uint8)


def dequant_mxfp8(codes, scales):
    """Exact float64 e4m3(q) * 2^(byte - 127), shape [rows, K]."""
    v = F.e4m3_decode(codes)
    s = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return v * np.repeat(s, MX_BLOCK, axis=1)


def linear_mxfp8_f64(xc, xs, wc, ws, alpha=1.0, bias=None):
    y = float(alpha) * (dequant_mxfp8(xc, xs) @ dequant_mxfp8(wc, ws).T)
    return y if bias is None else y + np.asarray(bias, dtype=np.float64)[None, :]


def linear_mxfp8(xc, xs, wc, ws, alpha=1.0, bias=None):
    return F.bf16_round_bits(linear_mxfp8_f64(xc, xs, wc, ws, alpha, bias))


# ---------------------------------------------------------------------------
# shared E4M3 quantizer with a float32 scale
# ---------------------------------------------------------------------------

def scale_from_amax(amax):
    """B2: s = fl32(amax / 448) (float32 division, one rounding)."""
    return _f32(np.asarray(amax, dtype=np.float32).astype(np.float64) / 448.0)


FLT_MAX = float(np.finfo(np.float32).max)


def reciprocal(s):
    """B3: r = fl32(1 / s), 0 where s == 0, and the largest finite float32
    where 1/s overflows (s below 2^-128, a group of float32 subnormals)."""
    s = np.asarray(s, dtype=np.float32)
    with np.errstate(divide="ignore"):
        r = np.where(s > 0, 1.0 / np.where(s > 0, s.astype(np.float64), 1.0), 0.0)
    return _f32(np.minimum(r, FLT_MAX))


def encode_with_scale(v, r):
    """B4 / T1: E4M3_RNE_satfinite(fl32(v * r)) for float32 v and r (broadcast)."""
    prod = _f32(np.asarray(v, dtype=np.float32).astype(np.float64) * np.asarray(r, np.float32).astype(np.float64))
    return F.e4m3_encode(prod)


# ---------------------------------------------------------------------------
# block FP8
# ---------------------------------------------------------------------------

def quant_fp8_block_act(x):
    """B1-B4 over 1 x 128 groups: x [M, K] float32 -> (codes u8 [M, K], scales f32 [M, K/128])."""
    x = _f32(x)
    M, K = x.shape
    if K % FP8_GROUP:
        raise ValueError("K must be a multiple of 128")
    g = x.reshape(M, K // FP8_GROUP, FP8_GROUP)
    s = scale_from_amax(np.abs(g).max(axis=2))
    codes = encode_with_scale(g, reciprocal(s)[:, :, None]).reshape(M, K)
    return codes, s


def quant_fp8_block_weight(w):
    """B1-B4 over 128 x 128 tiles: w [N, K] float32 -> (codes u8 [N, K], scales f32 [N/128, K/128])."""
    w = _f32(w)
    N, K = w.shape
    if N % FP8_GROUP or K % FP8_GROUP:
        raise ValueError("N and K must be multiples of 128")
    t = w.reshape(N // FP8_GROUP, FP8_GROUP, K // FP8_GROUP, FP8_GROUP)
    s = scale_from_amax(np.abs(t).max(axis=(1, 3)))
    codes = encode_with_scale(t, reciprocal(s)[:, None, :, None]).reshape(N, K)
    return codes, s


def dequant_fp8_block_act(codes, scales):
    return F.e4m3_decode(codes) * np.repeat(np.asarray(scales, np.float64), FP8_GROUP, axis=1)


def dequant_fp8_block_weight(codes, scales):
    s = np.repeat(np.repeat(np.asarray(scales, np.float64), FP8_GROUP, axis=0), FP8_GROUP, axis=1)
    return F.e4m3_decode(codes) * s


def linear_fp8_block_f64(xc, xs, wc, ws, bias=None):
    y = dequant_fp8_block_act(xc, xs) @ dequant_fp8_block_weight(wc, ws).T
    return y if bias is None else y + np.asarray(bias, dtype=np.float64)[None, :]


def linear_fp8_block(xc, xs, wc, ws, bias=None):
    return F.bf16_round_bits(linear_fp8_block_f64(xc, xs, wc, ws, bias))


# ---------------------------------------------------------------------------
# per-tensor FP8
# ---------------------------------------------------------------------------

def quant_fp8_tensor(x, s):
    """T1: codes u8 [rows, K] of float32 x with the per-tensor float32 scale s > 0."""
    return encode_with_scale(_f32(x), reciprocal(np.float32(s)))


def output_scale(s_x, s_w):
    """T2: alpha = fl32(s_x * s_w)."""
    return np.float32(np.float64(np.float32(s_x)) * np.float64(np.float32(s_w)))


def linear_fp8_tensor_f64(xc, wc, alpha, bias=None):
    y = float(np.float32(alpha)) * (F.e4m3_decode(xc) @ F.e4m3_decode(wc).T)
    return y if bias is None else y + np.asarray(bias, dtype=np.float64)[None, :]


def linear_fp8_tensor(xc, wc, alpha, bias=None):
    return F.bf16_round_bits(linear_fp8_tensor_f64(xc, wc, alpha, bias))
