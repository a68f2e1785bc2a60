"""GPU parity of the MXFP4 sibling (quantizer, packer, linear) against the oracle.

Codes and scale bytes must be bit-identical to oracle/mx.py; linear outputs
must agree with the oracle's float64 product of the decoded operands, rounded
to bf16, within a relative Frobenius error of 1e-3. Called through the C-ABI
binding. Inputs come from the `synthetic` generators (the sibling workload is
K = 4096, N = 14336, x ~ N(0, 1), W ~ N(0, 0.02^2)).
"""

import numpy as np
import pytest
import torch

import fp8_quantized_linear_amd as fql
import synthetic
from oracle import formats as F
from oracle import mx as X

from gpu_helpers import (DEV, REL_FROB_TOL, announce, bf16_bits_to_dev, cached_activations,
                         cached_weight, dev_bf16_to_bits, f32_to_dev, full_rows_sample, rel_frob)

pytestmark = pytest.mark.gpu


def _special_blocks(M, K, seed):
    """bf16 activations whose 32-blocks hit the quantizer's edge cases."""
    g = np.random.default_rng(seed)
    x = g.standard_normal((M, K)).astype(np.float32)
    nb = K // 32
    for r in range(M):
        kind = r % 8
        b = (r * 7) % nb
        blk = x[r, 32 * b: 32 * b + 32]
        if kind == 0:
            blk[:] = 0.0                                   # all-zero block -> scale byte 0
        elif kind == 1:
            blk *= np.float32(1e-39)                       # bf16 subnormals
        elif kind == 2:
            blk[:] = g.choice([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], 32) * 2.0 ** 9
            blk[0] = 6.0 * 2.0 ** 9                        # exactly representable
        elif kind == 3:
            blk[:] = 7.9                                   # saturates to 6 * 2^0
            blk[1::2] = -6.5
        elif kind == 4:
            blk[:] = 1.0
            blk[3] = -1e-30                                # rounds to -0 (code 8)
            blk[4] = 5.0                                   # tie 4 / 6 -> even (4)
        elif kind == 5:
            blk *= np.float32(3e37)                        # near the top of the range
        elif kind == 6:
            blk[:] = 8.0                                   # power-of-two maximum -> E = 1
            blk[2] = 0.25 * 2.0                            # tie at the smallest subnormal code
    return synthetic.f32_to_bf16_bits(x)


def _check_quant(xbits, label, ldx_pad=0):
    M, K = xbits.shape
    x32 = synthetic.bf16_bits_to_f32(xbits)
    ref_c, ref_s = X.quant_mxfp4(x32)
    announce(f"mxfp4 quant {label} M={M} K={K} ldx_pad={ldx_pad}")
    if ldx_pad:
        big = np.zeros((M, K + ldx_pad), dtype=np.uint16)
        big[:, ldx_pad:] = xbits
        xd = bf16_bits_to_dev(big)[:, ldx_pad:]
    else:
        xd = bf16_bits_to_dev(xbits)
    codes, scales = fql.quant_mxfp4(xd)
    torch.cuda.synchronize()
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(s, ref_s), f"scales differ at {np.argwhere(s != ref_s)[:5]}"
    assert np.array_equal(c, ref_c), f"codes differ at {np.argwhere(c != ref_c)[:5]}"


def test_mx_quant_tiny():
    _check_quant(synthetic.activations("normal", 16, 256, config="tiny"), "tiny")


@pytest.mark.parametrize("M", [1, 4096])
def test_mx_quant_siblings(M):
    _check_quant(cached_activations("normal", M, 4096, "siblings"), "siblings")


@pytest.mark.parametrize("M,K,pad", [(64, 1024, 0), (37, 160, 3), (8, 14336, 1)])
def test_mx_quant_edge_blocks(M, K, pad):
    _check_quant(_special_blocks(M, K, seed=M + K), "edge", ldx_pad=pad)


def test_mx_quant_weight_f32_subnormals():
    g = np.random.default_rng(5)
    w = (g.standard_normal((48, 512)) * 0.02).astype(np.float32)
    w[3, :32] = (g.standard_normal(32) * 1e-40).astype(np.float32)   # float32 subnormals
    w[4, 32:64] = 0.0
    w[5, 64:96] = np.float32(3.0e38)
    ref_c, ref_s = X.quant_mxfp4(w)
    announce("mxfp4 weight quant f32")
    codes, scales = fql.quant_mxfp4_weight(f32_to_dev(w))
    torch.cuda.synchronize()
    assert np.array_equal(scales.cpu().numpy(), ref_s)
    assert np.array_equal(codes.cpu().numpy(), ref_c)


def _mx_weight(W):
    codes, scales = fql.quant_mxfp4_weight(f32_to_dev(W))
    return fql.MXFP4Weight(fql.pack_weight_mxfp4(codes, scales), W.shape[0], W.shape[1])


def _run_linear(config, M, K, N, with_bias, rows=None, cols=None, alpha=1.0, label=""):
    xb = cached_activations("normal", M, K, config)
    x32 = synthetic.bf16_bits_to_f32(xb)
    W = cached_weight(config, N, K)
    r_sel = np.arange(M) if rows is None else np.asarray(rows)
    c_sel = np.arange(N) if cols is None else np.asarray(cols)
    bias_bits = synthetic.bias(N, config=config) if with_bias else None
    announce(f"mxfp4 linear {label} {config} M={M} K={K} N={N} bias={with_bias}")
    wobj = _mx_weight(W)
    bd = bf16_bits_to_dev(bias_bits) if with_bias else None
    y = fql.linear_mxfp4(bf16_bits_to_dev(xb), wobj, alpha=alpha, bias=bd)
    torch.cuda.synchronize()
    yb = dev_bf16_to_bits(y)
    xc, xs = X.quant_mxfp4(x32[r_sel])
    wc, ws = X.quant_mxfp4(W[c_sel])
    b64 = F.bf16_bits_to_f64(bias_bits[c_sel]) if with_bias else None
    ref = X.linear_mxfp4(xc, xs, wc, ws, alpha, b64)
    err = rel_frob(yb[np.ix_(r_sel, c_sel)], ref)
    assert err <= REL_FROB_TOL, f"rel Frobenius {err:.3e}"
    return err


def test_mx_linear_tiny():
    _run_linear("tiny", 16, 256, 512, False, label="tiny")


@pytest.mark.parametrize("M", [1, 4, 64, 4096])
def test_mx_linear_siblings(M):
    # every output column; at M = 4096 a seeded sample of 256 whole rows
    _run_linear("siblings", M, 4096, 14336, False, rows=full_rows_sample(M, seed=17),
                label="siblings")


@pytest.mark.parametrize("M,K,N", [(1, 96, 100), (3, 160, 520), (17, 416, 33), (33, 2080, 200),
                                   (100, 1056, 130), (65, 128, 16), (130, 4096, 48)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_mx_linear_ragged(M, K, N, with_bias):
    _run_linear("decode", M, K, N, with_bias, alpha=0.75, label="ragged")


def test_mx_linear_strided_and_deterministic():
    M, K, N = 24, 1024, 320
    xb = synthetic.activations("normal", M, K, config="decode", seed=4)
    x32 = synthetic.bf16_bits_to_f32(xb)
    W = cached_weight("decode", N, K)
    announce("mxfp4 linear strided/3-D/determinism")
    wobj = _mx_weight(W)
    big = np.zeros((M, K + 40), np.uint16)
    big[:, 40:] = xb
    xd = bf16_bits_to_dev(big)[:, 40:]
    ybig = torch.zeros((M, N + 8), dtype=torch.bfloat16, device=DEV)
    fql.linear_mxfp4(xd, wobj, out=ybig[:, :N])
    ref = X.linear_mxfp4(*X.quant_mxfp4(x32), *X.quant_mxfp4(W))
    assert rel_frob(dev_bf16_to_bits(ybig[:, :N]), ref) <= REL_FROB_TOL
    assert torch.all(ybig[:, N:] == 0)
    y3 = fql.linear_mxfp4(bf16_bits_to_dev(xb).view(2, 12, K), wobj)
    assert tuple(y3.shape) == (2, 12, N)
    y4 = fql.linear_mxfp4(bf16_bits_to_dev(xb).view(2, 12, K), wobj)
    assert torch.equal(y3.view(torch.int16), y4.view(torch.int16))


def test_mx_linear_identity_weight_exact():
    # identity weight (code 2 = 1.0, scale byte 127) and a power-of-two alpha:
    # every output is one exact product, so y equals bf16(alpha * x_hat) exactly
    K = 256
    xb = synthetic.activations("normal", 8, K, config="tiny", seed=3)
    x32 = synthetic.bf16_bits_to_f32(xb)
    q = np.zeros((K, K), np.uint8)
    np.fill_diagonal(q, 2)
    wc = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    ws = np.full((K, K // 32), 127, np.uint8)
    announce("mxfp4 identity weight")
    packed = fql.pack_weight_mxfp4(torch.from_numpy(wc).to(DEV), torch.from_numpy(ws).to(DEV))
    wobj = fql.MXFP4Weight(packed, K, K)
    y = fql.linear_mxfp4(bf16_bits_to_dev(xb), wobj, alpha=0.25)
    xhat = X.dequant_mxfp4(*X.quant_mxfp4(x32))
    # compared as values: a sum that starts at +0 turns a -0 product into +0
    got = F.bf16_bits_to_f64(dev_bf16_to_bits(y))
    assert np.array_equal(got, F.bf16_bits_to_f64(F.bf16_round_bits(0.25 * xhat)))

# Every GEMM configuration of the scaled formats (MXFP4 included) is covered
# by tests/test_gpu_fp8.py::test_every_sc_config.
