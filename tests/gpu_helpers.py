"""Shared helpers for the GPU parity tests (not a test module).

Inputs come from the `synthetic` generators; expected values come from the
`oracle` package only. The HIP path is reached through the C-ABI binding.
"""

import functools
import sys

import numpy as np
import torch

import synthetic
from oracle import formats as F
from oracle import nvfp4 as Q
from oracle.hadamard import fwht_fp32

DEV = "cuda:0"
REL_FROB_TOL = 1e-3  # GEMM output tolerance (relative Frobenius, bf16 vs bf16)


def announce(msg):
    """Print the case name before a GPU step (survives a crash of the box)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def bf16_bits_to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def dev_bf16_to_bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def f32_to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def rel_frob(y_bits, ref_bits):
    a = F.bf16_bits_to_f64(y_bits)
    b = F.bf16_bits_to_f64(ref_bits)
    den = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (den if den > 0 else 1.0)


def alpha_of(gx, gw):
    return np.float32((1.0 / np.float64(np.float32(gx))) * (1.0 / np.float64(np.float32(gw))))


@functools.lru_cache(maxsize=3)
def cached_weight(config, N, K):
    return synthetic.weight(N, K, config=config)


@functools.lru_cache(maxsize=4)
def cached_activations(kind, M, K, config):
    return synthetic.activations(kind, M, K, config=config)


@functools.lru_cache(maxsize=8)
def weight_case(config, N, K, hb, rows=None):
    """Oracle-side weight: (W fp32, g_w, codes, scales) for all rows or a row subset.

    g_w is calibrated on the rows the oracle quantizes (any positive g is a
    legal static scale; the GPU is given the same g).
    """
    W = cached_weight(config, N, K)
    sel = W if rows is None else W[list(rows)]
    amax = Q.amax_for_calibration(sel, hb)
    gw = Q.global_scale_from_amax(amax)
    Wr = fwht_fp32(sel, hb) if hb else sel
    codes, scales = Q.quant_nvfp4(Wr, gw)
    return W, gw, codes, scales
