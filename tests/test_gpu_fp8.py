"""GPU parity of the FP8 siblings (MXFP8, per-tensor FP8, block FP8) against the
oracle, and of every scaled-MFMA GEMM configuration for all four scaled formats.

Codes and scales must be bit-identical to oracle/fp8.py (and oracle/mx.py);
linear outputs must agree with the oracle's float64 product of the decoded
operands, rounded to bf16, within a relative Frobenius error of 1e-3. The FP8
matrix cores add the 128 products of one instruction with an internal
precision of roughly 2^-13 of the sum of their magnitudes (measured), which
keeps the output error near 1e-4, inside that bound.
"""

import numpy as np
import pytest
import torch

import fp8_quantized_linear_amd as fql
import synthetic
from oracle import formats as F
from oracle import fp8 as P
from oracle import mx as X

from gpu_helpers import (DEV, REL_FROB_TOL, announce, bf16_bits_to_dev, cached_activations,
                         cached_weight, dev_bf16_to_bits, f32_to_dev, full_rows_sample, rel_frob,
                         strided_output)

pytestmark = pytest.mark.gpu


def _dev_x(xbits, pad=0):
    if not pad:
        return bf16_bits_to_dev(xbits)
    M, K = xbits.shape
    big = np.zeros((M, K + pad), dtype=np.uint16)
    big[:, pad:] = xbits
    return bf16_bits_to_dev(big)[:, pad:]


def _edge_rows(M, K, seed):
    """bf16 activations with zero, subnormal, saturating and huge groups."""
    g = np.random.default_rng(seed)
    x = g.standard_normal((M, K)).astype(np.float32)
    for r in range(M):
        kind = r % 6
        b = (r * 5) % (K // 128)
        grp = x[r, 128 * b:128 * b + 128]
        if kind == 0:
            grp[:] = 0.0
        elif kind == 1:
            grp *= np.float32(1e-39)
        elif kind == 2:
            grp *= np.float32(2e37)
        elif kind == 3:
            grp[:32] = 500.0          # one MX block whose values saturate
            grp[1:32:2] = -470.0
        elif kind == 4:
            grp[5] = -1e-30           # tiny negative -> -0 code
    return synthetic.f32_to_bf16_bits(x)


# ---------------------------------------------------------------------------
# quantizers (bit-exact)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,pad", [(16, 256, 0), (37, 384, 3), (64, 4096, 0), (6, 14336, 1)])
def test_mxfp8_quant(M, K, pad):
    xb = _edge_rows(M, K, seed=M + K)
    ref_c, ref_s = P.quant_mxfp8(synthetic.bf16_bits_to_f32(xb))
    announce(f"mxfp8 quant M={M} K={K} pad={pad}")
    c, s = fql.quant_mxfp8(_dev_x(xb, pad))
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), ref_s)
    c = c.cpu().numpy()
    assert np.array_equal(c, ref_c), f"codes differ at {np.argwhere(c != ref_c)[:5]}"


@pytest.mark.parametrize("M,K,pad", [(16, 256, 0), (37, 384, 3), (64, 4096, 0)])
def test_fp8_block_quant(M, K, pad):
    xb = _edge_rows(M, K, seed=3 * M + K)
    ref_c, ref_s = P.quant_fp8_block_act(synthetic.bf16_bits_to_f32(xb))
    announce(f"fp8 block quant M={M} K={K} pad={pad}")
    c, s = fql.quant_fp8_block(_dev_x(xb, pad))
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    c = c.cpu().numpy()
    assert np.array_equal(c, ref_c), f"codes differ at {np.argwhere(c != ref_c)[:5]}"


@pytest.mark.parametrize("scale", [0.0137, 1.0, 3.5e-3, 2.0 ** -7])
def test_fp8_tensor_quant(scale):
    xb = _edge_rows(24, 512, seed=11)
    x32 = synthetic.bf16_bits_to_f32(xb)
    ref = P.quant_fp8_tensor(x32, np.float32(scale))
    announce(f"fp8 tensor quant scale={scale}")
    c = fql.quant_fp8(_dev_x(xb, 5), scale)
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy(), ref)


def test_fp8_weight_quantizers_f32():
    g = np.random.default_rng(12)
    w = (g.standard_normal((256, 512)) * 0.02).astype(np.float32)
    w[3, :64] = (g.standard_normal(64) * 1e-40).astype(np.float32)
    w[130:, 256:384] *= 300.0
    w[200, 400] = 3.0e38
    announce("fp8 weight quantizers (f32)")
    wd = f32_to_dev(w)
    c, s = fql.quant_mxfp8_weight(wd)
    rc, rs = P.quant_mxfp8(w)
    assert np.array_equal(s.cpu().numpy(), rs) and np.array_equal(c.cpu().numpy(), rc)
    c, s = fql.quant_fp8_block_weight(wd)
    rc, rs = P.quant_fp8_block_weight(w)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(c.cpu().numpy(), rc)
    sw = np.float32(0.021)
    c = fql.quant_fp8_weight(wd, float(sw))
    assert np.array_equal(c.cpu().numpy(), P.quant_fp8_tensor(w, sw))


# ---------------------------------------------------------------------------
# linear layers
# ---------------------------------------------------------------------------

def _weight(fmt, W, input_scale=None):
    """The GPU weight; per-tensor FP8 takes the oracle's calibration scales."""
    wd = f32_to_dev(W)
    if fmt == "mxfp4":
        return fql.MXFP4Weight.from_float(wd)
    if fmt == "mxfp8":
        return fql.MXFP8Weight.from_float(wd)
    if fmt == "fp8_block":
        return fql.FP8BlockWeight.from_float(wd)
    sw = P.scale_from_amax(np.abs(W).max())
    return fql.FP8Weight.from_float(wd, input_scale, weight_scale=float(sw))


def _fp8_scales(x32, W):
    """Oracle-side per-tensor FP8 scales (s_x, s_w) and output scale alpha."""
    s_in = P.scale_from_amax(np.abs(x32).max())
    s_w = P.scale_from_amax(np.abs(W).max())
    return s_in, s_w, P.output_scale(s_in, s_w)


def _oracle(fmt, x32, W, wobj, alpha, bias64, cols=None, s_in=None, s_w=None):
    """Oracle output [rows of x32, cols] (all columns when cols is None).

    Every weight scale covers whole rows of W except block FP8's 128 x 128
    tiles, so the oracle quantizes just the selected rows of W (the tiles
    that hold them, for block FP8)."""
    cols = np.arange(W.shape[0]) if cols is None else np.asarray(cols)
    b = None if bias64 is None else bias64[cols]
    if fmt == "mxfp4":
        return X.linear_mxfp4(*X.quant_mxfp4(x32), *X.quant_mxfp4(W[cols]), alpha, b)
    if fmt == "mxfp8":
        return P.linear_mxfp8(*P.quant_mxfp8(x32), *P.quant_mxfp8(W[cols]), alpha, b)
    if fmt == "fp8_block":
        tiles = np.unique(cols // 128)
        Wt = np.concatenate([W[128 * t:128 * t + 128] for t in tiles])
        wc, ws = P.quant_fp8_block_weight(Wt)
        pos = {t: i for i, t in enumerate(tiles)}
        local = np.array([128 * pos[c // 128] + c % 128 for c in cols])
        y = P.linear_fp8_block_f64(*P.quant_fp8_block_act(x32), wc, ws, None)[:, local]
        y = float(np.float32(alpha)) * y
        return F.bf16_round_bits(y if b is None else y + b[None, :])
    xc = P.quant_fp8_tensor(x32, s_in)
    wc = P.quant_fp8_tensor(W[cols], s_w)
    return P.linear_fp8_tensor(xc, wc, np.float32(alpha), b)


def _run(fmt, config, M, K, N, with_bias, rows=None, cols=None, alpha=None, label=""):
    """One sibling linear call against the oracle on rows `rows` and columns `cols`
    (all when None). Per-tensor FP8 without an explicit alpha runs on the
    weight's device output scale and the oracle applies its own fl32(s_x s_w)."""
    xb = cached_activations("normal", M, K, config)
    x32 = synthetic.bf16_bits_to_f32(xb)
    W = cached_weight(config, N, K)
    r_sel = np.arange(M) if rows is None else np.asarray(rows)
    c_sel = np.arange(N) if cols is None else np.asarray(cols)
    bias_bits = synthetic.bias(N, config=config) if with_bias else None
    announce(f"{fmt} linear {label} {config} M={M} K={K} N={N} bias={with_bias}")
    s_in, s_w, alpha_fp8 = _fp8_scales(x32, W)
    wobj = _weight(fmt, W, float(s_in))
    bd = bf16_bits_to_dev(bias_bits) if with_bias else None
    fn = {"mxfp4": fql.linear_mxfp4, "mxfp8": fql.linear_mxfp8, "fp8": fql.linear_fp8,
          "fp8_block": fql.linear_fp8_block}[fmt]
    if alpha is None and fmt == "fp8":
        y = fn(bf16_bits_to_dev(xb), wobj, bias=bd)  # device output scale of the weight
        a = alpha_fp8
    else:
        a = 1.0 if alpha is None else alpha
        y = fn(bf16_bits_to_dev(xb), wobj, alpha=a, bias=bd)
    torch.cuda.synchronize()
    yb = dev_bf16_to_bits(y)
    b64 = F.bf16_bits_to_f64(bias_bits) if with_bias else None
    ref = _oracle(fmt, x32[r_sel], W, wobj, a, b64, c_sel, s_in=s_in, s_w=s_w)
    err = rel_frob(yb[np.ix_(r_sel, c_sel)], ref)
    assert err <= REL_FROB_TOL, f"rel Frobenius {err:.3e}"
    return err


@pytest.mark.parametrize("fmt", ["mxfp8", "fp8", "fp8_block"])
def test_linear_tiny(fmt):
    _run(fmt, "tiny", 16, 256, 512, False, label="tiny")


@pytest.mark.parametrize("M", [1, 64, 4096])
@pytest.mark.parametrize("fmt", ["mxfp8", "fp8", "fp8_block"])
def test_linear_siblings(fmt, M):
    # every output column; at M = 4096 a seeded sample of 256 whole rows
    _run(fmt, "siblings", M, 4096, 14336, False, rows=full_rows_sample(M, seed=17),
         label="siblings")


@pytest.mark.parametrize("fmt,N", [("mxfp4", 24576), ("mxfp8", 12288), ("fp8", 12288), ("fp8_block", 12288)])
def test_linear_last_round_split_every_row(fmt, N):
    # 4 row groups x 96 column groups = 384 tiles: the last 128 are split in
    # two along K; 1000 rows (ragged), every row and column compared
    # (forced: the plan splits the last round itself only for long K)
    M, K = 1000, 1024
    spec = "2,4,8,4,4,0,2" if fmt == "mxfp4" else "4,2,4,4,3,0,2"
    with fql.plan_override(spec, which="sc_gemm"):
        assert "grid=512 splits=1 tail=128x2" in fql.linear_sc_plan(fmt, M, N, K)
        _run(fmt, "siblings", M, K, N, True, label="tail-split")


@pytest.mark.parametrize("M,K,N", [(1, 96, 100), (3, 160, 520), (17, 416, 33), (33, 2080, 200),
                                   (130, 4096, 48)])
@pytest.mark.parametrize("fmt", ["mxfp8", "fp8"])
def test_linear_ragged(fmt, M, K, N):
    _run(fmt, "decode", M, K, N, True, alpha=None if fmt == "fp8" else 0.75, label="ragged")


@pytest.mark.parametrize("M,K,N", [(1, 128, 128), (3, 384, 640), (33, 2048, 256), (130, 4096, 384)])
def test_linear_fp8_block_ragged(M, K, N):
    _run("fp8_block", "decode", M, K, N, True, alpha=0.75, label="ragged")


def test_fp8_block_power_of_two_weight_scales():
    # UE8M0 weight scales widened to float32 (the write-up's upcast): the packer
    # and GEMM take any float32 scale; compare against the oracle's decode.
    rng = np.random.default_rng(21)
    N, K, M = 256, 512, 8
    wc = rng.integers(0, 256, (N, K), dtype=np.uint8)
    wc[(wc & 0x7F) == 0x7F] = 0  # no NaN codes
    ws = np.ldexp(1.0, rng.integers(-12, -4, (N // 128, K // 128))).astype(np.float32)
    xb = synthetic.activations("normal", M, K, config="tiny", seed=5)
    x32 = synthetic.bf16_bits_to_f32(xb)
    announce("fp8 block with power-of-two weight scales")
    packed = fql.pack_weight_fp8_block(torch.from_numpy(wc).to(DEV), torch.from_numpy(ws).to(DEV))
    y = fql.linear_fp8_block(bf16_bits_to_dev(xb), fql.FP8BlockWeight(packed, N, K))
    xc, xs = P.quant_fp8_block_act(x32)
    ref = F.bf16_round_bits(P.linear_fp8_block_f64(xc, xs, wc, ws))
    assert rel_frob(dev_bf16_to_bits(y), ref) <= REL_FROB_TOL


def test_fp8_strided_3d_and_deterministic():
    M, K, N = 24, 1024, 384
    xb = synthetic.activations("normal", M, K, config="decode", seed=4)
    x32 = synthetic.bf16_bits_to_f32(xb)
    W = cached_weight("decode", N, K)
    announce("fp8 family strided / 3-D / determinism")
    for fmt in ("mxfp8", "fp8", "fp8_block"):
        s_in = float(P.scale_from_amax(np.abs(x32).max()))
        wobj = _weight(fmt, W, s_in)
        fn = {"mxfp8": fql.linear_mxfp8, "fp8": fql.linear_fp8, "fp8_block": fql.linear_fp8_block}[fmt]
        ybig = torch.zeros((M, N + 8), dtype=torch.bfloat16, device=DEV)
        fn(_dev_x(xb, 40), wobj, out=ybig[:, :N])
        s_x, s_w, a = _fp8_scales(x32, W)
        if fmt != "fp8":
            a = 1.0
        ref = _oracle(fmt, x32, W, wobj, a, None, s_in=s_x, s_w=s_w)
        assert rel_frob(dev_bf16_to_bits(ybig[:, :N]), ref) <= REL_FROB_TOL, fmt
        assert torch.all(ybig[:, N:] == 0)
        y3 = fn(bf16_bits_to_dev(xb).view(2, 12, K), wobj)
        y4 = fn(bf16_bits_to_dev(xb).view(2, 12, K), wobj)
        assert tuple(y3.shape) == (2, 12, N)
        assert torch.equal(y3.view(torch.int16), y4.view(torch.int16))


@pytest.mark.parametrize("pad,off", [(1, 5), (8, 8)])
def test_sibling_tile_writeout_any_output_stride(pad, off):
    # whole tiles of the scaled-MFMA GEMM leave as 16-byte row pieces when y
    # is 16-byte aligned with ldy a multiple of 8, element by element
    # otherwise; either way the values equal a contiguous output's bit for bit
    # and nothing outside the view is written
    M, K, N = 2100, 1024, 6144
    xb = synthetic.activations("normal", M, K, config="prefill", seed=9)
    x32 = synthetic.bf16_bits_to_f32(xb)
    W = cached_weight("prefill", N, K)
    xd = bf16_bits_to_dev(xb)
    for fmt in ("mxfp4", "mxfp8", "fp8", "fp8_block"):
        announce(f"{fmt} tile write-out M={M} N={N} K={K} ldy=N+{pad} offset={off}")
        assert "splits=1" in fql.linear_sc_plan(fmt, M, N, K)
        wobj = _weight(fmt, W, float(P.scale_from_amax(np.abs(x32).max())))
        fn = {"mxfp4": fql.linear_mxfp4, "mxfp8": fql.linear_mxfp8, "fp8": fql.linear_fp8,
              "fp8_block": fql.linear_fp8_block}[fmt]
        y0 = fn(xd, wobj).clone()
        y, flat, covered = strided_output(M, N, N + pad, off)
        fn(xd, wobj, out=y)
        torch.cuda.synchronize()
        assert torch.equal(y.contiguous().view(torch.int16), y0.view(torch.int16)), fmt
        assert torch.all(flat[~covered] == -7.0), fmt


# Every scaled-MFMA GEMM configuration built into the library (wave grid
# WM x WN, MTW x NTW 16x16 tiles per wave, ring depth ST: the planner's
# choices), with and without split K, on a ragged shape: several row groups,
# 9 chunks of 128, a partial column group.
SC_CONFIGS = [(1, 4, 4, 2, 4), (2, 2, 4, 4, 3), (4, 2, 4, 4, 3), (1, 4, 1, 2, 4)]
SC_CONFIGS_FP4 = SC_CONFIGS + [(2, 4, 8, 4, 4)]  # its 8-bit ring would not fit in LDS


def _sc_cases():
    for fmt in ("mxfp4", "mxfp8", "fp8", "fp8_block"):
        for cfg in (SC_CONFIGS_FP4 if fmt == "mxfp4" else SC_CONFIGS):
            for splits in (1, 3):
                yield pytest.param(fmt, cfg, splits, id=f"{fmt}-{cfg}-s{splits}")


@pytest.mark.parametrize("fmt,cfg,splits", list(_sc_cases()))
def test_every_sc_config(fmt, cfg, splits, plan_override):
    M, K = 150, 1152
    N = 384 if fmt == "fp8_block" else 400
    wm, wn, mtw, ntw, st = cfg
    plan_override(f"{wm},{wn},{mtw},{ntw},{st},{splits}", "sc_gemm")
    plan = fql.linear_sc_plan(fmt, M, N, K)
    want = f"gemm_sc_kernel<{fmt},WM={wm},WN={wn},MTW={mtw},NTW={ntw},ST={st}>"
    assert want in plan and f"splits={splits}" in plan, plan
    _run(fmt, "tiny", M, K, N, True, alpha=None if fmt == "fp8" else 1.5, label=f"{cfg} splits={splits}")


# Every small-M GEMV configuration built (W waves splitting K, NT column tiles
# per workgroup, D chunks in flight per wave) at M = 1, 16 (one row tile) and
# 17, 32 (two), on a ragged shape: 9 chunks of 128, a partial column tile; the
# one-row-tile configuration also with the in-workgroup quantizer (fq = 1).
SCV_ONE_TILE = {"mxfp4": (4, 4, 3), "mxfp8": (4, 2, 3), "fp8": (4, 2, 3), "fp8_block": (4, 2, 3)}
SCV_TWO_TILES = (4, 2, 3)


def _scv_cases():
    for fmt, one in SCV_ONE_TILE.items():
        for M in (1, 16):
            for fq in (0, 1):
                yield pytest.param(fmt, one, M, fq, id=f"{fmt}-{one}-M{M}-fq{fq}")
        for M in (17, 32):
            yield pytest.param(fmt, SCV_TWO_TILES, M, 0, id=f"{fmt}-{SCV_TWO_TILES}-M{M}")


@pytest.mark.parametrize("fmt,cfg,M,fq", list(_scv_cases()))
def test_every_gemv_config(fmt, cfg, M, fq, plan_override):
    K = 1152
    N = 384 if fmt == "fp8_block" else 400
    w, nt, d = cfg
    plan_override(f"{w},{nt},{d},{fq}", "sc_gemv")
    plan = fql.linear_sc_plan(fmt, M, N, K)
    want = f"gemv_sc_kernel<{fmt},W={w},MT={(M + 15) // 16},NT={nt},D={d}" + (",FQ=1>" if fq else ">")
    assert want in plan, plan
    _run(fmt, "tiny", M, K, N, True, alpha=None if fmt == "fp8" else 1.5, label=f"gemv {cfg} fq={fq}")


def _sc_weight(fmt, N, K):
    W = f32_to_dev(synthetic.weight(N, K, config="siblings", seed=3))
    if fmt == "fp8":
        return fql.FP8Weight.from_float(W, input_scale=0.02)
    return {"mxfp4": fql.MXFP4Weight, "mxfp8": fql.MXFP8Weight, "fp8_block": fql.FP8BlockWeight}[fmt].from_float(W)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8", "fp8", "fp8_block"])
@pytest.mark.parametrize("M,K", [(1, 4096), (7, 1024), (16, 384), (3, 4096), (5, 1152)])
def test_fused_gemv_equals_two_launch_path(fmt, M, K, plan_override):
    # the in-workgroup quantizer produces the same operand bytes as the
    # standalone quantizer, so the fused call is bit-identical to quantizer + GEMV
    N = 2048 if fmt == "fp8_block" else 2000
    w = _sc_weight(fmt, N, K)
    fn = {"mxfp4": fql.linear_mxfp4, "mxfp8": fql.linear_mxfp8, "fp8": fql.linear_fp8,
          "fp8_block": fql.linear_fp8_block}[fmt]
    xb = cached_activations("normal", M, K, "siblings")
    x = _dev_x(xb, pad=1 if M == 5 else 0)  # one unaligned case
    nt = 4 if fmt == "mxfp4" else 2
    outs = []
    for fq in (1, 0):
        plan_override(f"4,{nt},3,{fq}", "sc_gemv")
        plan = fql.linear_sc_plan(fmt, M, N, K)
        assert (",FQ=1>" in plan) == bool(fq), plan
        announce(f"fused gemv {fmt} M={M} K={K} fq={fq}")
        outs.append(fn(x, w))
        torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))

