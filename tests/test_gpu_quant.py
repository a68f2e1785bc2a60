"""GPU parity of the NVFP4 quantizer (K1) against the oracle: codes and scales
must be bit-identical. Called through the C-ABI binding."""

import numpy as np
import pytest
import torch

import fp8_quantized_linear_amd as fql
import synthetic
from oracle import nvfp4 as Q
from oracle.hadamard import fwht_fp32

from gpu_helpers import DEV, announce, bf16_bits_to_dev, f32_to_dev

pytestmark = pytest.mark.gpu


def _check_quant(xbits, hb=0, g=None, M=None, K=None, ldx_pad=0, offset=0, label=""):
    M, K = xbits.shape
    x32 = synthetic.bf16_bits_to_f32(xbits)
    if g is None:
        g = Q.global_scale_from_amax(Q.amax_for_calibration(x32, hb))
    ref_c, ref_s = Q.quant_nvfp4(x32, g, hb)
    announce(f"quant {label} M={M} K={K} hb={hb} ldx_pad={ldx_pad} offset={offset}")
    if ldx_pad or offset:
        big = np.zeros((M, K + ldx_pad + offset), dtype=np.uint16)
        big[:, offset:offset + K] = xbits
        xd = bf16_bits_to_dev(big)[:, offset:offset + K]
    else:
        xd = bf16_bits_to_dev(xbits)
    codes, scales = fql.quant_nvfp4(xd, float(g), hb)
    torch.cuda.synchronize()
    c = codes.cpu().numpy()
    s = scales.cpu().numpy()
    assert np.array_equal(s, ref_s), f"scales differ at {np.argwhere(s != ref_s)[:5]}"
    assert np.array_equal(c, ref_c), f"codes differ at {np.argwhere(c != ref_c)[:5]}"


def test_quant_tiny():
    _check_quant(synthetic.activations("normal", 16, 256, config="tiny"), label="tiny")


@pytest.mark.parametrize("M", [1, 8, 32, 128])
@pytest.mark.parametrize("K", [4096, 14336])
def test_quant_decode_shapes(M, K):
    _check_quant(synthetic.activations("normal", M, K, config="decode"), label="decode")


@pytest.mark.parametrize("K", [4096, 14336])
def test_quant_prefill_outliers(K):
    M = 2048
    _check_quant(synthetic.activations("normal_outliers", M, K, config="prefill"), label="prefill")


@pytest.mark.parametrize("hb", [16, 32, 64, 128])
@pytest.mark.parametrize("K", [5120, 25600])
def test_quant_hadamard_student_t(hb, K):
    _check_quant(synthetic.activations("student_t3", 33, K, config="hadamard"), hb=hb,
                 label="hadamard")


@pytest.mark.parametrize("hb", [0, 32])
def test_quant_strided_rows(hb):
    x = synthetic.activations("normal", 20, 1024, config="decode", seed=5)
    _check_quant(x, hb=hb, ldx_pad=64, label="strided-aligned")
    _check_quant(x, hb=hb, ldx_pad=3, offset=1, label="strided-unaligned")


@pytest.mark.parametrize("gmode", ["saturate", "subnormal", "underflow"])
def test_quant_global_scale_regimes(gmode):
    xb = synthetic.activations("normal", 8, 512, config="decode", seed=7)
    x32 = synthetic.bf16_bits_to_f32(xb)
    g0 = Q.global_scale_from_amax(Q.amax_for_calibration(x32))
    g = {"saturate": np.float32(40.0) * g0, "subnormal": np.float32(0.01),
         "underflow": np.float32(1e-4)}[gmode]
    _check_quant(xb, g=g, label=gmode)


def test_quant_special_values():
    M, K = 4, 256
    x = np.zeros((M, K), dtype=np.float32)
    r = np.random.default_rng(3)
    x[0] = r.standard_normal(K)
    x[1, :16] = -0.0                                  # all negative zeros
    x[1, 16:32] = 1e-40                               # float32/bf16 denormals
    x[1, 32:48] = -3e-39
    x[1, 48:64] = r.standard_normal(16) * 1e-38
    x[2] = r.standard_normal(K) * 1e4                 # large values
    x[3, ::2] = 6.0                                   # exact representable
    x[3, 1::2] = -0.5
    xb = synthetic.f32_to_bf16_bits(x)
    for g in (np.float32(1.0), np.float32(0.37), np.float32(1e30)):
        _check_quant(xb, g=g, label=f"special g={g}")
    for hb in (16, 128):
        _check_quant(xb, g=np.float32(3.0), hb=hb, label="special-hadamard")


@pytest.mark.parametrize("hb", [0, 16, 128])
def test_weight_quant_f32(hb):
    N, K = 96, 5120
    W = synthetic.weight(N, K, config="hadamard")
    amax = Q.amax_for_calibration(W, hb)
    g = Q.global_scale_from_amax(amax)
    ref_c, ref_s = Q.quant_nvfp4(fwht_fp32(W, hb) if hb else W, g)
    announce(f"weight quant N={N} K={K} hb={hb}")
    codes, scales = fql.quant_nvfp4_weight(f32_to_dev(W), float(g), hb)
    assert np.array_equal(scales.cpu().numpy(), ref_s)
    assert np.array_equal(codes.cpu().numpy(), ref_c)


@pytest.mark.parametrize("hb", [0, 32, 128])
def test_amax_matches_oracle(hb):
    xb = synthetic.activations("student_t3", 64, 5120, config="hadamard", seed=2)
    x32 = synthetic.bf16_bits_to_f32(xb)
    announce(f"amax hb={hb}")
    a = fql.amax(bf16_bits_to_dev(xb), hb).item()
    assert np.float32(a) == Q.amax_for_calibration(x32, hb)
    W = synthetic.weight(64, 5120, config="hadamard")
    aw = fql.amax(f32_to_dev(W), hb).item()
    assert np.float32(aw) == Q.amax_for_calibration(W, hb)


def test_quant_3d_input_and_preallocated_outputs():
    xb = synthetic.activations("normal", 24, 512, config="decode", seed=9)
    x32 = synthetic.bf16_bits_to_f32(xb)
    g = Q.global_scale_from_amax(Q.amax_for_calibration(x32))
    ref_c, ref_s = Q.quant_nvfp4(x32, g)
    xd = bf16_bits_to_dev(xb).view(2, 12, 512)
    codes = torch.full((2, 12, 256), 0xAA, dtype=torch.uint8, device=DEV)
    scales = torch.full((2, 12, 32), 0xAA, dtype=torch.uint8, device=DEV)
    announce("quant 3-D preallocated")
    c2, s2 = fql.quant_nvfp4(xd, float(g), 0, codes=codes, scales=scales)
    assert c2.data_ptr() == codes.data_ptr() and s2.data_ptr() == scales.data_ptr()
    assert np.array_equal(codes.cpu().numpy().reshape(24, 256), ref_c)
    assert np.array_equal(scales.cpu().numpy().reshape(24, 32), ref_s)
