"""The allocation-free NVFP4 linear entry point (GPU).

fql_linear_nvfp4_noalloc runs the plan and kernels of fql_linear_nvfp4 with a
static per-device scratch array instead of a caller workspace. Its outputs
must equal fql_linear_nvfp4's bit for bit on the same inputs, on consecutive
calls of different sizes (the array keeps the previous call's contents), and
lie within the oracle's 1e-3 bar; a call needing more scratch than the array
holds is rejected before any launch.
"""

import ctypes

import numpy as np
import pytest
import torch

import fp8_quantized_linear_amd as fql
import synthetic
from oracle import nvfp4 as Q

from gpu_helpers import (DEV, REL_FROB_TOL, alpha_of, announce, bf16_bits_to_dev,
                         dev_bf16_to_bits, f32_to_dev, rel_frob)

pytestmark = pytest.mark.gpu


def _case(M, K, N, seed):
    xb = synthetic.activations("normal", M, K, config="decode", seed=seed)
    W = synthetic.weight(N, K, config="decode", seed=seed)
    x32 = synthetic.bf16_bits_to_f32(xb)
    gx = Q.global_scale_from_amax(Q.amax_for_calibration(x32))
    gw = Q.global_scale_from_amax(Q.amax_for_calibration(W))
    ref = Q.linear_nvfp4(*Q.quant_nvfp4(x32, gx), *Q.quant_nvfp4(W, gw), alpha_of(gx, gw))
    w = fql.NVFP4Weight.from_float(f32_to_dev(W), input_global_scale=float(gx),
                                   weight_global_scale=float(gw))
    return bf16_bits_to_dev(xb), w, ref


def test_noalloc_matches_the_workspace_call_twice_in_a_row():
    # the second call is smaller and runs another plan on the scratch the first one used
    for (M, K, N, seed) in ((300, 4096, 1024, 1), (5, 1152, 640, 2), (128, 14336, 512, 3)):
        announce(f"noalloc M={M} K={K} N={N}")
        x, w, ref = _case(M, K, N, seed)
        y_ws = fql.linear_nvfp4(x, w, alpha=w.alpha)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        fql.linear_nvfp4_noalloc(x, w, out=y, alpha=w.alpha)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ws.view(torch.int16)), fql.linear_plan(M, N, K)
        assert rel_frob(dev_bf16_to_bits(y), ref) <= REL_FROB_TOL


def test_noalloc_rejects_a_plan_larger_than_its_scratch():
    M, K, N = 8192, 14336, 4096  # x_hat alone is 235 MB
    lib = fql.lib()
    p = ctypes.c_void_p(256)
    st = lib.fql_linear_nvfp4_noalloc(p, M, K, K, 1.0, 0, p, N, 1.0, ctypes.c_void_p(0), p, N,
                                      ctypes.c_void_p(0))
    assert st == -4 and "scratch" in lib.fql_last_error().decode()
