"""Bit-exact parity of the activation operand each NVFP4 linear call consumes (GPU).

A linear call quantizes x into one of three forms before (or inside) its GEMM:
* x_hat, the dequantized values e2m1(q) * s as float16 in MFMA A-fragment
  order, written by a quantizer pass (kinds 1 and 3);
* the packed activation, codes and E4M3 scales in the packed weight layout,
  written by a quantizer pass (kind 4, the small-M ring);
* no stored form: the one-launch small-M kernel (kind 0) quantizes into LDS.
The stored forms are read back from the workspace after the diagnostic
quantizer half of the call (fql_linear_nvfp4_quantize) and decoded on the
host: x_hat must equal the oracle's dequantized values exactly, and the
packed codes and scales must equal the oracle's codes and scales bit for bit,
with zero padding. The forms that are never stored are checked through an
identity weight: one exact product per output and a power-of-two alpha make
y = bf16(alpha * x_hat) exact, so every plan kind's output reveals its
operand values bit for bit ("TorchNvFp4LinearKernel", Key code: the
activation is quantized with the layer's input global scale before the
scaled GEMM; "QUTLASS NVFP4 online transforms", Implementation: the rotation
comes first).
"""

import numpy as np
import pytest
import torch

import fp8_quantized_linear_amd as fql
import synthetic
from oracle import formats as F
from oracle import nvfp4 as Q

from gpu_helpers import (DEV, announce, bf16_bits_to_dev, cached_activations, decode_packed,
                         decode_xhat, dev_bf16_to_bits, f32_to_dev, full_rows_sample, plan_rows)

pytestmark = pytest.mark.gpu

OPERAND_OFFSET = 64 * 1024  # after the workspace's arrival counters


def _operand(x32_rows_all, xb, M, K, N, hb, gx):
    """Run the quantizer half of the call; returns (plan, raw operand bytes)."""
    xd = bf16_bits_to_dev(xb)
    w = fql.NVFP4Weight(torch.empty(16, dtype=torch.uint8, device=DEV), N, K, float(gx), 1.0, hb)
    ws = fql.new_workspace(fql.linear_workspace_bytes(M, N, K), DEV)
    ws.fill_(0xA5)  # poison: every byte of the operand, padding included, must be written
    ws[:OPERAND_OFFSET].zero_()
    fql.linear_nvfp4_quantize(xd, w, ws)
    torch.cuda.synchronize()
    return fql.linear_plan(M, N, K), ws[OPERAND_OFFSET:].cpu().numpy().tobytes()


def _check_operand(config, M, K, hb, N, rows=None, xkind=None):
    xkind = xkind or synthetic.WORKLOADS[config]["x"]
    xb = cached_activations(xkind, M, K, config)
    x32 = synthetic.bf16_bits_to_f32(xb)
    gx = Q.global_scale_from_amax(Q.amax_for_calibration(x32, hb))
    announce(f"operand {config} M={M} K={K} N={N} hb={hb}")
    plan, raw = _operand(x32, xb, M, K, N, hb, gx)
    Kp = -(-K // 128) * 128
    Mp = plan_rows(plan, M)
    r = np.arange(M) if rows is None else np.asarray(rows)
    xc, xs = Q.quant_nvfp4(x32[r], gx, hb)
    if "apack" in plan:
        codes, scales = decode_packed(raw, Mp, Kp)
        assert np.array_equal(codes[r, :K // 2], xc), plan
        assert np.array_equal(scales[r, :K // 16], xs), plan
        assert not codes[M:].any() and not codes[:, K // 2:].any()      # zero padding
        assert not scales[M:].any() and not scales[:, K // 16:].any()
    else:
        assert "xhat" in plan, plan
        xh = decode_xhat(raw, Mp, Kp)
        assert np.array_equal(xh[r, :K], Q.dequant_nvfp4(xc, xs)), plan
        assert not xh[M:].any() and not xh[:, K:].any()
    return plan


@pytest.mark.parametrize("M", [1, 17, 32])
@pytest.mark.parametrize("K,hb", [(4096, 0), (14336, 0), (1040, 16), (3072, 64), (4096, 128)])
def test_small_m_packed_operand(M, K, hb, plan_override):
    # the per-wave-ring GEMM's operand: the activation packed like a weight
    plan_override("kind=4,waves=4,nt=2,st=3")
    plan = _check_operand("decode", M, K, hb, 4096)
    assert "apack" in plan, plan


@pytest.mark.parametrize("M,K,hb", [(1, 4096, 0), (17, 1040, 16), (32, 3072, 64)])
def test_small_m_xhat_operand(M, K, hb, plan_override):
    # the same activations as x_hat, the operand of the LDS-ring GEMM
    plan_override("kind=3,mt=2,nt=1,st=4,cw=4")
    plan = _check_operand("decode", M, K, hb, 4096)
    assert "xhat" in plan and "gemm_lds32_kernel" in plan, plan


@pytest.mark.parametrize("M,K", [(128, 4096), (128, 14336), (300, 1152), (2048, 4096),
                                 (2048, 14336)])
def test_xhat_operand_llama_shapes(M, K):
    plan = _check_operand("prefill" if M >= 2048 else "decode", M, K, 0, 4096)
    assert "gemm_lds32_kernel" in plan


def test_xhat_operand_prefill_8192_rows_sampled():
    K = 14336
    plan = _check_operand("prefill", 8192, K, 0, 4096, rows=full_rows_sample(8192, seed=5))
    assert "gemm_lds32_kernel" in plan


@pytest.mark.parametrize("hb", [16, 32, 64, 128])
@pytest.mark.parametrize("M,K", [(256, 5120), (256, 25600), (4096, 5120), (4096, 25600)])
def test_xhat_operand_qwen_hadamard(M, K, hb):
    rows = None if M <= 256 else full_rows_sample(M, seed=hb)
    _check_operand("hadamard", M, K, hb, 5120, rows=rows)


def test_packed_decoder_matches_the_weight_packer():
    # the test's layout decoder, applied to the library's packed weight of
    # oracle codes and scales, gives those codes and scales back
    N, K = 200, 1040
    W = synthetic.weight(N, K, config="decode", seed=8)
    gw = Q.global_scale_from_amax(Q.amax_for_calibration(W))
    wc, ws = Q.quant_nvfp4(W, gw)
    announce("packed layout decoder")
    packed = fql.pack_weight_nvfp4(torch.from_numpy(wc).to(DEV), torch.from_numpy(ws).to(DEV))
    torch.cuda.synchronize()
    Np, Kp = -(-N // 16) * 16, -(-K // 128) * 128
    codes, scales = decode_packed(packed.cpu().numpy().tobytes(), Np, Kp)
    assert np.array_equal(codes[:N, :K // 2], wc) and np.array_equal(scales[:N, :K // 16], ws)
    assert not codes[N:].any() and not codes[:, K // 2:].any()


# ---------------------------------------------------------------------------
# identity weight: every plan kind's operand through the output
# ---------------------------------------------------------------------------

def _identity_weight(K):
    q = np.zeros((K, K), np.uint8)
    np.fill_diagonal(q, 2)                    # E2M1 code 2 = 1.0
    wc = Q.pack_nibbles(q)
    ws = np.full((K, K // 16), 0x38, np.uint8)  # E4M3 1.0
    return wc, ws


IDENTITY_KINDS = {
    "kind0": "kind=0",
    "kind1": "kind=1",
    "kind3": "kind=3",
    "kind4": "kind=4,waves=4,nt=2,st=3",
}


def _identity_cases():
    for kind, spec in IDENTITY_KINDS.items():
        for M in (1, 16, 17, 32, 128, 300):
            if kind == "kind0" and M > 16:
                continue
            if kind == "kind4" and M > 32:
                continue
            for K, hb in ((1152, 0), (1040, 16), (1152, 32), (2048, 64), (1152, 128)):
                if kind == "kind0" and M * K * 2 > 64 * 1024:
                    continue
                yield pytest.param(kind, M, K, hb, id=f"{kind}-M{M}-K{K}-hb{hb}")


@pytest.mark.parametrize("kind,M,K,hb", list(_identity_cases()))
def test_identity_weight_exposes_operand_every_kind(kind, M, K, hb, plan_override):
    spec = IDENTITY_KINDS[kind]
    plan_override(spec)
    plan = fql.linear_plan(M, K, K)
    want = {"kind0": "linear_gemv_kernel<", "kind1": "gemm_tiled_kernel<",
            "kind3": "gemm_lds32_kernel<", "kind4": "gemv_ring_kernel<"}[kind]
    assert want in plan, plan
    xb = synthetic.activations("student_t3", M, K, config="hadamard", seed=M + hb)
    x32 = synthetic.bf16_bits_to_f32(xb)
    gx = Q.global_scale_from_amax(Q.amax_for_calibration(x32, hb))
    wc, ws = _identity_weight(K)
    announce(f"identity weight {kind} M={M} K={K} hb={hb}: {plan}")
    packed = fql.pack_weight_nvfp4(torch.from_numpy(wc).to(DEV), torch.from_numpy(ws).to(DEV))
    w = fql.NVFP4Weight(packed, K, K, float(gx), 1.0, hb)
    y = fql.linear_nvfp4(bf16_bits_to_dev(xb), w, alpha=0.125)
    torch.cuda.synchronize()
    expect = F.bf16_round_bits(0.125 * Q.dequant_nvfp4(*Q.quant_nvfp4(x32, gx, hb)))
    got = dev_bf16_to_bits(y)
    # equal values; the float32 accumulator starts at +0, so an operand of -0
    # (a negative value that rounds to zero keeps its sign) comes out as +0
    gv, ev = F.bf16_bits_to_f64(got), F.bf16_bits_to_f64(expect)
    assert np.array_equal(gv, ev), f"{int((gv != ev).sum())} of {got.size} differ"
    assert np.all((got == expect) | ((expect == 0x8000) & (got == 0)))


def test_quantize_and_gemm_halves_equal_one_call():
    # the diagnostic halves compute exactly what one linear call computes
    M, K, N = 300, 4096, 1024
    xb = synthetic.activations("normal", M, K, config="decode", seed=12)
    W = synthetic.weight(N, K, config="decode", seed=12)
    announce("quantize + gemm halves")
    w = fql.NVFP4Weight.from_float(f32_to_dev(W), input_global_scale=0.5)
    x = bf16_bits_to_dev(xb)
    y1 = fql.linear_nvfp4(x, w, alpha=w.alpha)
    ws = fql.new_workspace(fql.linear_workspace_bytes(M, N, K), DEV)
    fql.linear_nvfp4_quantize(x, w, ws)
    y2 = fql.linear_nvfp4_gemm(M, w, ws, w.alpha)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
