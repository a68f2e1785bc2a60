"""GPU parity of the NVFP4 W4A4 linear layer against the oracle.

The HIP path quantizes the activation, runs the block-scaled GEMM and the
fused epilogue; the oracle quantizes independently and evaluates the float64
product of the decoded operands, rounded to bf16. Outputs must agree within a
relative Frobenius error of 1e-3 (bf16 vs bf16). The activation global scale
is calibrated on the whole activation; large configurations compare a seeded
sample of at least 256 whole rows (every output column, the first and the
last row included) with the oracle.
"""

import numpy as np
import pytest
import torch

import fp8_quantized_linear_amd as fql
import synthetic
from oracle import formats as F
from oracle import nvfp4 as Q
from oracle.hadamard import fwht_fp32

from gpu_helpers import (DEV, REL_FROB_TOL, alpha_of, announce, bf16_bits_to_dev,
                         cached_activations, dev_bf16_to_bits, f32_to_dev, full_rows_sample,
                         rel_frob, strided_output, weight_case, weight_hat)

pytestmark = pytest.mark.gpu


def _gpu_weight(W, gw, hb, gx):
    """Quantize + pack on the GPU with the oracle's g_w; check codes bit-exactly."""
    codes, scales = fql.quant_nvfp4_weight(f32_to_dev(W), float(gw), hb)
    packed = fql.pack_weight_nvfp4(codes, scales)
    return fql.NVFP4Weight(packed, W.shape[0], W.shape[1], float(gx), float(gw), hb), codes, scales


def _run_case(config, M, K, N, hb, with_bias, rows=None, xkind=None, label=""):
    """One linear call against the oracle: the GPU weight codes and scales bit for
    bit, then y on the rows `rows` (all rows when None), every column. The call
    runs twice, with alpha passed by value and with the weight's device alpha
    (from the library's alpha formula), which must agree bit for bit."""
    xkind = xkind or synthetic.WORKLOADS[config]["x"]
    xb = cached_activations(xkind, M, K, config)
    x32 = synthetic.bf16_bits_to_f32(xb)
    r_sel = np.arange(M) if rows is None else np.asarray(rows)
    gx = Q.global_scale_from_amax(Q.amax_for_calibration(x32, hb))
    W, gw, wc_ref, ws_ref = weight_case(config, N, K, hb)
    bias_bits = synthetic.bias(N, config=config) if with_bias else None
    alpha = alpha_of(gx, gw)

    announce(f"linear {label} {config} M={M} K={K} N={N} hb={hb} bias={with_bias}")
    wobj, wcodes, wscales = _gpu_weight(W, gw, hb, gx)
    assert np.array_equal(wcodes.cpu().numpy(), wc_ref)
    assert np.array_equal(wscales.cpu().numpy(), ws_ref)
    del wcodes, wscales
    xd = bf16_bits_to_dev(xb)
    bd = bf16_bits_to_dev(bias_bits) if with_bias else None
    y = fql.linear_nvfp4(xd, wobj, alpha=float(alpha), bias=bd)
    y_dev_alpha = fql.linear_nvfp4(xd, wobj, bias=bd)  # alpha from the weight's device scalar
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_dev_alpha.view(torch.int16))
    yb = dev_bf16_to_bits(y)

    xc, xs = Q.quant_nvfp4(x32[r_sel], gx, hb)
    bias64 = F.bf16_bits_to_f64(bias_bits) if with_bias else None
    # G1 of the weight decoded once per weight and kept for the other cases
    ref = F.bf16_round_bits(Q.linear_dequantized_f64(Q.dequant_nvfp4(xc, xs),
                                                     weight_hat(config, N, K, hb), alpha, bias64))
    err = rel_frob(yb[r_sel], ref)
    assert err <= REL_FROB_TOL, f"rel Frobenius {err:.3e}"
    return err


def test_linear_tiny():
    _run_case("tiny", 16, 256, 512, 0, False, label="tiny")


@pytest.mark.parametrize("M", [1, 8, 32, 128])
@pytest.mark.parametrize("shape", ["qkv", "gate_up", "down"])
def test_linear_decode(M, shape):
    K, N = synthetic.LLAMA_SHAPES[shape]
    _run_case("decode", M, K, N, 0, True, label=shape)


@pytest.mark.parametrize("M", [2048, 8192])
@pytest.mark.parametrize("shape", ["qkv", "gate_up", "down"])
def test_linear_prefill_full_rows(M, shape):
    K, N = synthetic.LLAMA_SHAPES[shape]
    _run_case("prefill", M, K, N, 0, False, rows=full_rows_sample(M, seed=M + K + N), label=shape)


@pytest.mark.parametrize("hb", [16, 32, 64, 128])
@pytest.mark.parametrize("shape", ["gate_up", "down"])
@pytest.mark.parametrize("M", [1, 256, 4096])
def test_linear_hadamard_full_rows(hb, shape, M):
    K, N = synthetic.QWEN_SHAPES[shape]
    _run_case("hadamard", M, K, N, hb, False, rows=full_rows_sample(M, seed=hb + M + K),
              label=f"qwen-{shape}")


@pytest.mark.parametrize("M,K,N", [(1, 272, 100), (3, 144, 520), (17, 400, 33), (33, 2064, 200),
                                   (100, 1040, 130), (65, 128, 16), (130, 4096, 48)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_linear_ragged(M, K, N, with_bias):
    _run_case("decode", M, K, N, 0, with_bias, label="ragged")


@pytest.mark.parametrize("M,K,N,hb", [(1, 288, 100, 32), (1, 2048, 5000, 128), (1, 1024, 48, 16)])
def test_linear_rotated_single_row_ragged(M, K, N, hb):
    # the fused kernel at M = 1 with a rotation takes two column tiles per
    # workgroup; odd tile counts leave the last workgroup one
    _run_case("hadamard", M, K, N, hb, True, label="rotated-ragged")


@pytest.mark.parametrize("M,K,N,spec", [(2048, 1024, 6144, "tail=2"), (1650, 2048, 5120, "tail=4"),
                                        (2048, 2048, 6144, "tail=3"), (1650, 8192, 5120, None)])
def test_linear_last_round_split_every_row(M, K, N, spec):
    # tiles of the last, part-filled round of workgroups split along K (the
    # plan's own choice for long K, here 64 chunks; forced at shorter K):
    # 2048 x 6144 has 384 tiles, the last 128 in halves or thirds; 1650 x 5120
    # has 260, the last 4 in quarters (ragged rows). Every row is compared.
    with fql.plan_override(spec or ""):
        assert "tail=" in fql.linear_plan(M, N, K)
        _run_case("prefill", M, K, N, 0, True, label=f"tail-split {spec}")


def test_linear_strided_3d_input_and_output_stride():
    M, K, N = 24, 1024, 320
    xb = synthetic.activations("normal", M, K, config="decode", seed=4)
    x32 = synthetic.bf16_bits_to_f32(xb)
    gx = Q.global_scale_from_amax(Q.amax_for_calibration(x32))
    W, gw, wc, ws = weight_case("decode", N, K, 0)
    alpha = alpha_of(gx, gw)
    announce("linear strided/3-D")
    wobj, _, _ = _gpu_weight(W, gw, 0, gx)
    big = np.zeros((M, K + 64), np.uint16)
    big[:, 32:32 + K] = xb
    xd = bf16_bits_to_dev(big)[:, 32:32 + K]                      # non-contiguous rows
    ybig = torch.zeros((M, N + 8), dtype=torch.bfloat16, device=DEV)
    y = ybig[:, :N]
    fql.linear_nvfp4(xd, wobj, alpha=float(alpha), out=y)
    ref = Q.linear_nvfp4(*Q.quant_nvfp4(x32, gx), wc, ws, alpha)
    assert rel_frob(dev_bf16_to_bits(y), ref) <= REL_FROB_TOL
    assert torch.all(ybig[:, N:] == 0)                              # nothing past N written
    x3 = bf16_bits_to_dev(xb).view(2, 12, K)
    y3 = fql.linear_nvfp4(x3, wobj, alpha=float(alpha))
    assert tuple(y3.shape) == (2, 12, N) and y3.dtype == torch.bfloat16
    assert rel_frob(dev_bf16_to_bits(y3).reshape(M, N), ref) <= REL_FROB_TOL


@pytest.mark.parametrize("M,N,K,pad,off,spec", [(300, 517, 1024, 3, 1, "splits=1"),
                                                (300, 512, 1024, 8, 0, "splits=1"),
                                                (2100, 6144, 1024, 1, 5, None),
                                                (2100, 6144, 1024, 8, 8, None)])
def test_linear_tile_writeout_any_output_stride(M, N, K, pad, off, spec):
    # whole tiles of the LDS-ring GEMM leave as 16-byte row pieces when y is
    # 16-byte aligned with ldy a multiple of 8, element by element otherwise
    # (odd ldy or start, ragged last piece); either way the values equal a
    # contiguous output's bit for bit and nothing outside the view is written
    xb = synthetic.activations("normal", M, K, config="prefill", seed=9)
    W, gw, _, _ = weight_case("prefill", N, K, 0)
    announce(f"tile write-out M={M} N={N} K={K} ldy=N+{pad} offset={off}")
    wobj, _, _ = _gpu_weight(W, gw, 0, 1.0)
    xd = bf16_bits_to_dev(xb)
    bd = bf16_bits_to_dev(synthetic.bias(N, config="prefill"))
    with fql.plan_override(spec):
        assert "gemm_lds32_kernel" in fql.linear_plan(M, N, K) and "splits=1" in fql.linear_plan(M, N, K)
        y0 = fql.linear_nvfp4(xd, wobj, bias=bd).clone()
        y, flat, covered = strided_output(M, N, N + pad, off)
        fql.linear_nvfp4(xd, wobj, bias=bd, out=y)
    torch.cuda.synchronize()
    assert torch.equal(y.contiguous().view(torch.int16), y0.view(torch.int16))
    assert torch.all(flat[~covered] == -7.0)


@pytest.mark.parametrize("M,N,K", [(1, 6144, 4096), (128, 4096, 14336), (300, 256, 512)])
def test_linear_deterministic(M, N, K):
    xb = synthetic.activations("normal", M, K, config="decode", seed=11)
    W, gw, _, _ = weight_case("decode", N, K, 0)
    announce(f"determinism M={M} N={N} K={K}")
    wobj, _, _ = _gpu_weight(W, gw, 0, 1.0)
    xd = bf16_bits_to_dev(xb)
    y1 = fql.linear_nvfp4(xd, wobj).clone()
    y2 = fql.linear_nvfp4(xd, wobj).clone()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_linear_identity_weight_closed_form():
    # identity weight: codes 2 (1.0) on the diagonal with E4M3 scale 1.0
    K = 256
    xb = synthetic.activations("normal", 8, K, config="tiny", seed=3)
    x32 = synthetic.bf16_bits_to_f32(xb)
    gx = Q.global_scale_from_amax(Q.amax_for_calibration(x32))
    q = np.zeros((K, K), np.uint8)
    np.fill_diagonal(q, 2)
    wc = Q.pack_nibbles(q)
    ws = np.full((K, K // 16), 0x38, np.uint8)
    bias_bits = synthetic.bias(K, config="tiny")
    announce("identity weight")
    packed = fql.pack_weight_nvfp4(torch.from_numpy(wc).to(DEV), torch.from_numpy(ws).to(DEV))
    wobj = fql.NVFP4Weight(packed, K, K, float(gx), 1.0, 0)
    xd = bf16_bits_to_dev(xb)
    xc, xs = Q.quant_nvfp4(x32, gx)
    xhat = Q.dequant_nvfp4(xc, xs)
    # no bias: one exact product per output and a power-of-two alpha -> exact
    y0 = fql.linear_nvfp4(xd, wobj, alpha=0.125)
    expect0 = F.bf16_round_bits(0.125 * xhat)
    assert np.array_equal(F.bf16_bits_to_f64(dev_bf16_to_bits(y0)), F.bf16_bits_to_f64(expect0))
    # with bias: the float32 sum may round once before the bf16 cast -> 1 ulp
    y = fql.linear_nvfp4(xd, wobj, alpha=0.125, bias=bf16_bits_to_dev(bias_bits))
    expect = F.bf16_round_bits(0.125 * xhat + F.bf16_bits_to_f64(bias_bits)[None, :])
    got = F.bf16_bits_to_f64(dev_bf16_to_bits(y))
    ref = F.bf16_bits_to_f64(expect)
    ulp = np.abs(ref) * 2.0 ** -7 + 1e-30
    assert np.all(np.abs(got - ref) <= ulp)
    assert np.mean(got == ref) > 0.999


# Every tiled GEMM configuration built into the library (workgroup tile of
# (WM*MT*16) rows x ((4/WM)*NT*16) columns), with and without split K, on a
# ragged shape: several row groups, an odd chunk count, a partial column tile.
TILED_CONFIGS = [(1, 1, 1), (2, 1, 1), (2, 2, 2), (4, 2, 2), (8, 4, 1)]


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("mt,nt,wm", TILED_CONFIGS)
def test_linear_every_tiled_config(mt, nt, wm, splits, plan_override):
    M, K, N = 150, 1152, 400
    plan_override(f"kind=1,mt={mt},nt={nt},wm={wm},splits={splits}")
    plan = fql.linear_plan(M, N, K)
    assert f"MT={mt},NT={nt},WM={wm}>" in plan and f"splits={splits}" in plan, plan
    _run_case("tiny", M, K, N, 0, True, label=f"tiled<{mt},{nt},{wm}> splits={splits}")


# Every 32x32-MFMA LDS-ring configuration (workgroup tile (MT*32) rows x
# (4*NT*32) columns), same ragged shape (N = 400 leaves half a 32-column tile).
# (WM = 2: two row halves of 4 waves each, two waves per SIMD.)
# (WN = 8: eight column waves, two per SIMD.)
LDS32_CONFIGS = [(4, 1, 3, 4), (2, 1, 4, 4), (4, 1, 3, 8), (2, 1, 4, 8)]


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("mt,nt,st,cw", LDS32_CONFIGS)
def test_linear_every_lds32_config(mt, nt, st, cw, splits, plan_override):
    M, K, N = 150, 1152, 400
    plan_override(f"kind=3,mt={mt},nt={nt},st={st},cw={cw},splits={splits}")
    plan = fql.linear_plan(M, N, K)
    want = f"gemm_lds32_kernel<MT={mt},NT={nt},ST={st}" + (f",WN={cw}>" if cw != 4 else ">")
    assert want in plan and f"splits={splits}" in plan, plan
    _run_case("tiny", M, K, N, 0, True, label=f"lds32<{mt},{nt},{st},{cw}> splits={splits}")


# The XCD-grouped tile order (bands of xg row groups per XCD) only renumbers
# the output tiles: on a grid that is not a multiple of 8 workgroups, with a
# ragged last row group and a last band shorter than xg, every order matches
# the oracle and all orders agree bit for bit (xg = 0: row-major order).
@pytest.mark.parametrize("xg", [0, 1, 3, 4, 9])
def test_linear_xcd_tile_order(xg, plan_override):
    M, K, N = 1100, 1152, 2100
    plan_override(f"kind=3,mt=4,nt=1,st=3,cw=8,splits=1,xg={xg}")
    plan = fql.linear_plan(M, N, K)
    assert "grid=81 " in plan and (f"xcd_bands={xg}" in plan if xg else "xcd_bands" not in plan), plan
    _run_case("tiny", M, K, N, 0, True, label=f"xcd bands {xg}")
    xb = cached_activations(synthetic.WORKLOADS["tiny"]["x"], M, K, "tiny")
    W, gw, _, _ = weight_case("tiny", N, K, 0)
    gx = Q.global_scale_from_amax(Q.amax_for_calibration(synthetic.bf16_bits_to_f32(xb), 0))
    wobj, _, _ = _gpu_weight(W, gw, 0, gx)
    xd = bf16_bits_to_dev(xb)
    y = fql.linear_nvfp4(xd, wobj)
    plan_override("kind=3,mt=4,nt=1,st=3,cw=8,splits=1,xg=0")
    y0 = fql.linear_nvfp4(xd, wobj)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y0.view(torch.int16))


# Every per-wave-ring small-M configuration built into the library (W waves
# splitting K, interleaved, MT row tiles, NT column tiles per workgroup, D
# chunks in flight per wave: the planner's choices), on a ragged shape. M = 1
# and 16 fill one row tile, 17 and 32 two.
GEMV_RING_BUILT = [(4, 1, 2, 3), (4, 1, 4, 3), (8, 1, 1, 3), (4, 2, 2, 3), (8, 2, 1, 3)]


def _ring_cases():
    for w, mt, nt, d in GEMV_RING_BUILT:
        for M in ((1, 16) if mt == 1 else (17, 32)):
            yield pytest.param(w, nt, d, M, id=f"W{w}-NT{nt}-D{d}-M{M}")


@pytest.mark.parametrize("w,nt,d,M", list(_ring_cases()))
def test_linear_every_gemv_ring_config(w, nt, d, M, plan_override):
    K, N = 1152, 400
    plan_override(f"kind=4,waves={w},nt={nt},st={d}")
    plan = fql.linear_plan(M, N, K)
    want = f"quant_nvfp4_apack_kernel + gemv_ring_kernel<W={w},MT={(M + 15) // 16},NT={nt},D={d}>"
    assert want in plan, plan
    _run_case("tiny", M, K, N, 0, True, label=f"gemv_ring<{w},{nt},{d}>")


@pytest.mark.parametrize("w,nt,d,M", [(4, 2, 3, 3), (4, 2, 3, 17), (4, 2, 3, 32), (8, 1, 3, 5),
                                      (8, 1, 3, 24), (4, 4, 3, 9)])
def test_linear_ring_uneven_chunk_shares(w, nt, d, M, plan_override):
    # waves take chunks wave, wave + W, ...; K = 1664 is 13 chunks, so some waves
    # get one chunk fewer
    K, N = 1664, 272
    plan_override(f"kind=4,waves={w},nt={nt},st={d}")
    plan = fql.linear_plan(M, N, K)
    assert f"gemv_ring_kernel<W={w},MT={(M + 15) // 16},NT={nt},D={d}>" in plan, plan
    _run_case("tiny", M, K, N, 0, True, label=f"gemv_ring<{w},{nt},{d}> 13 chunks")


@pytest.mark.parametrize("cfg,M,N,K", [("waves=8,nt=1,st=3", 1, 1, 16), ("waves=8,nt=1,st=3", 8, 17, 16),
                                        ("waves=8,nt=1,st=3", 32, 33, 48),
                                        ("waves=8,nt=1,st=3", 17, 1, 112),
                                        ("waves=4,nt=4,st=3", 3, 200, 144),
                                        ("waves=4,nt=4,st=3", 16, 1, 16),
                                        ("waves=4,nt=2,st=3", 32, 33, 48),
                                        ("waves=4,nt=2,st=3", 1, 17, 112)])
def test_linear_ring_edge_shapes(cfg, M, N, K, plan_override):
    # one chunk or less of K (most waves have no chunk), one or a few columns
    plan_override(f"kind=4,{cfg}")
    plan = fql.linear_plan(M, N, K)
    assert "gemv_ring_kernel" in plan, plan
    _run_case("tiny", M, K, N, 0, True, label=f"ring edge {plan}")


@pytest.mark.parametrize("M,K,hb", [(1, 1040, 0), (5, 4096, 0), (16, 1040, 16), (17, 2064, 0),
                                    (32, 4096, 128), (8, 14336, 0), (24, 3072, 64)])
def test_linear_packed_activation_ring_matches_xhat_gemm(M, K, hb, plan_override):
    # the packed activation (small-M ring) and x_hat (LDS-ring GEMM) carry the same
    # fp16 operand values; the two kernels sum in different orders, so both are
    # held to the oracle and to each other within the output bar (K with a
    # ragged tail past the last 128-chunk; rotations through the same quantizer)
    N = 400
    xb = synthetic.activations("normal", M, K, config="decode", seed=31)
    x32 = synthetic.bf16_bits_to_f32(xb)
    gx = Q.global_scale_from_amax(Q.amax_for_calibration(x32, hb))
    W, gw, wc, ws = weight_case("decode", N, K, hb)
    alpha = alpha_of(gx, gw)
    announce(f"ring packed activation vs x_hat M={M} K={K} hb={hb}")
    wobj, _, _ = _gpu_weight(W, gw, hb, gx)
    xd = bf16_bits_to_dev(xb)
    outs = {}
    for spec in ("kind=4,waves=4,nt=2,st=3", "kind=3,mt=2,nt=1,st=4,cw=4"):
        plan_override(spec)
        outs[spec[:6]] = dev_bf16_to_bits(fql.linear_nvfp4(xd, wobj, alpha=float(alpha)))
    ref = Q.linear_nvfp4(*Q.quant_nvfp4(x32, gx, hb), wc, ws, alpha)
    for y in outs.values():
        assert rel_frob(y, ref) <= REL_FROB_TOL
    assert rel_frob(outs["kind=4"], outs["kind=3"]) <= REL_FROB_TOL
