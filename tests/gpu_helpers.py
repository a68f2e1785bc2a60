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
    Wr = fwht_fp32(sel, hb) if hb else sel
    gw = Q.global_scale_from_amax(Q.amax_for_calibration(Wr))  # amax of the rotated rows
    codes, scales = Q.quant_nvfp4(Wr, gw)
    return W, gw, codes, scales


@functools.lru_cache(maxsize=8)
def weight_hat(config, N, K, hb):
    """The oracle's exactly decoded weight (G1, float64 [N, K]) of weight_case."""
    _, _, codes, scales = weight_case(config, N, K, hb)
    return Q.dequant_nvfp4(codes, scales)


def full_rows_sample(M, n=256, seed=0):
    """A seeded, sorted sample of n distinct rows of M (all rows when M <= n),
    always holding the first and the last row."""
    if M <= n:
        return np.arange(M)
    r = np.random.default_rng(seed)
    rows = np.sort(r.choice(np.arange(1, M - 1), n - 2, replace=False))
    return np.concatenate([[0], rows, [M - 1]])


def plan_rows(plan, M):
    """Rows Mp of the activation operand a launch plan writes (M padded to its row tile)."""
    import re

    m = re.search(r"gemm_lds32_kernel<MT=(\d+),NT=\d+,ST=\d+(?:,(WM|WN)=(\d+))?>", plan)
    if m:
        t = 32 * int(m.group(1)) * (int(m.group(3)) if m.group(2) == "WM" else 1)
    elif "gemm_tiled_kernel" in plan:
        m = re.search(r"gemm_tiled_kernel<MT=(\d+),NT=\d+,WM=(\d+)>", plan)
        t = 16 * int(m.group(1)) * int(m.group(2))
    else:
        m = re.search(r"gemv_ring_kernel<W=\d+,MT=(\d+)", plan)
        return 16 * int(m.group(1))
    return -(-M // t) * t


def decode_xhat(buf, Mp, Kp):
    """x_hat operand (float16 in MFMA A-fragment order [Mp/16][Kp/32][64 lanes][8],
    lane = kq*16 + m holding row m, k = 32*step + 8*kq + 0..7) -> float64 [Mp, Kp]."""
    h = np.frombuffer(buf, dtype=np.float16, count=Mp * Kp)
    h = h.reshape(Mp // 16, Kp // 32, 4, 16, 8).transpose(0, 3, 1, 2, 4)
    return h.reshape(Mp, Kp).astype(np.float64)


def decode_packed(buf, rows_p, Kp):
    """Packed NVFP4 layout (the packed weight's, also the packed activation's)
    -> canonical (codes uint8 [rows_p, Kp/2], scales uint8 [rows_p, Kp/16]).

    codes [rows_p/16][KC][64 lanes][16 B]: lane = kq*16 + n, dword j holds the
    eight codes of row n at k = 128c + 32j + 8kq + 0..7, element i in nibble i.
    scales [rows_p/16][ceil(KC/4)][32 slots][16 B]: slot n*2 + h, byte 4q + j is
    the scale of row n, 16-block 8c + 2j + h of chunk c = 4*group + q.
    """
    T, KC = rows_p // 16, Kp // 128
    KC4 = -(-KC // 4)
    b = np.frombuffer(buf, dtype=np.uint8)
    c = b[:rows_p * Kp // 2].reshape(T, KC, 4, 16, 4, 4).transpose(0, 3, 1, 4, 2, 5)
    codes = c.reshape(rows_p, Kp // 2)
    s = b[rows_p * Kp // 2:rows_p * Kp // 2 + T * KC4 * 512].reshape(T, KC4, 16, 2, 4, 4)
    scales = s.transpose(0, 2, 1, 4, 5, 3).reshape(rows_p, KC4 * 32)[:, :Kp // 16]
    return np.ascontiguousarray(codes), np.ascontiguousarray(scales)


def strided_output(M, N, ld, off, fill=-7.0):
    """An M x N bf16 output view with row stride ld starting `off` elements into
    a flat buffer filled with `fill` (odd ld or off give a view whose rows are
    not 16-byte aligned), the flat buffer, and the mask of the elements the
    view covers."""
    import torch
    flat = torch.full((off + M * ld + 8,), fill, dtype=torch.bfloat16, device=DEV)
    y = torch.as_strided(flat, (M, N), (ld, 1), off)
    covered = torch.zeros(flat.numel(), dtype=torch.bool)
    idx = off + torch.arange(M).unsqueeze(1) * ld + torch.arange(N).unsqueeze(0)
    covered[idx.reshape(-1)] = True
    return y, flat, covered.to(DEV)
