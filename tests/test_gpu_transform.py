"""GPU parity of the general block-diagonal transform and the dynamic global
scale against the oracle (oracle/transform.py), through the C-ABI binding.

The transform's float32 sum is accumulated by the matrix cores in their own
order, so bit-exactness holds only where every partial sum is exact; those
cases (identity, permutations, the normalised Sylvester matrix on small
multiples of 1/4) are compared bit for bit. Elsewhere the near-tie rule
applies:
* every transformed value lies within EPS * sum_j |T[i][j] x[j]| (plus half
  a float32 unit) of the exact sum;
* every block scale is the E4M3 rounding of some block maximum within that
  bound, and every code the E2M1 rounding, under the kernel's own scale, of
  some value within it;
* at most MAX_MISMATCH of the scales and of the codes differ from the
  oracle's.
"""

import numpy as np
import pytest
import torch

import fp8_quantized_linear_amd as fql
import synthetic
from oracle import formats as F
from oracle import nvfp4 as Q
from oracle import transform as TR
from oracle.hadamard import fwht_fp32, hadamard_scale_fp32, sylvester

from gpu_helpers import (DEV, REL_FROB_TOL, alpha_of, announce, bf16_bits_to_dev,
                         dev_bf16_to_bits, f32_to_dev, rel_frob)

pytestmark = pytest.mark.gpu

# Bound on the matrix cores' float32 accumulation error, relative to
# sum_j |T[i][j] x[j]| (the worst case measured on the inputs below is
# printed by test_transform_values_within_bound).
EPS = 2.0 ** -20
MAX_MISMATCH = 1e-3


def _x(M, K, seed=0, kind="student_t3"):
    return synthetic.activations(kind, M, K, config="transform", seed=seed)


def _T_bits(b, kind="orthogonal", seed=0):
    return synthetic.transform_matrix(b, kind, seed)


def _T_dev(bits):
    return bf16_bits_to_dev(bits)


def _half_ulp(v):
    v = np.abs(np.asarray(v, np.float32))
    return (np.spacing(np.maximum(v, np.float32(2.0 ** -126))).astype(np.float64)) / 2


def _bound(x32, T64):
    v64 = TR.transform_f64(x32, T64)
    return v64, EPS * TR.transform_abs_sum(x32, T64) + _half_ulp(v64)


def _check_rule(x32, T64, g, codes, scales, label):
    """The near-tie rule for GPU codes/scales of the transformed x32."""
    ref_c, ref_s = TR.quant_nvfp4_transform(x32, T64, g)
    v64, err = _bound(x32, T64)
    M, K = x32.shape
    g = np.float32(g)
    # scales: E4M3(fl32(fl32(a/6) * g)) is monotone in a
    lo = np.maximum(np.abs(v64) - err, 0.0).reshape(M, K // 16, 16).max(axis=2)
    hi = (np.abs(v64) + err).reshape(M, K // 16, 16).max(axis=2)
    lo32 = np.nextafter(lo.astype(np.float32), np.float32(0))
    hi32 = np.nextafter(hi.astype(np.float32), np.float32(np.inf))

    def e4(a):
        return F.e4m3_encode(((a / np.float32(6.0)).astype(np.float32) * g).astype(np.float32))

    s_lo, s_hi = e4(lo32), e4(hi32)
    assert np.all((scales >= s_lo) & (scales <= s_hi)), \
        f"{label}: scale outside its near-tie interval at {np.argwhere((scales < s_lo) | (scales > s_hi))[:5]}"
    # codes under the kernel's scale: E2M1(fl32(v * r)) is monotone in v for r >= 0
    sd = F.e4m3_decode(scales).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(sd == 0, np.float32(0), g / sd).astype(np.float32)
    rr = np.repeat(r, 16, axis=1)
    vlo = np.nextafter((v64 - err).astype(np.float32), np.float32(-np.inf))
    vhi = np.nextafter((v64 + err).astype(np.float32), np.float32(np.inf))
    d_lo = F.e2m1_decode(F.e2m1_encode((vlo * rr).astype(np.float32)))
    d_hi = F.e2m1_decode(F.e2m1_encode((vhi * rr).astype(np.float32)))
    q = Q.unpack_nibbles(codes)
    d = F.e2m1_decode(q)
    bad = (d < d_lo) | (d > d_hi)
    assert not bad.any(), f"{label}: code outside its near-tie interval at {np.argwhere(bad)[:5]}"
    # exact zeros (every product zero) are +0
    zero = TR.transform_abs_sum(x32, T64) == 0
    assert np.all(q[zero] == 0), f"{label}: zero sums must encode as +0"
    s_rate = np.mean(scales != ref_s)
    c_rate = np.mean(q != Q.unpack_nibbles(ref_c))
    print(f"[rule] {label}: scale mismatch {s_rate:.2e}, code mismatch {c_rate:.2e}")
    assert s_rate <= MAX_MISMATCH and c_rate <= MAX_MISMATCH, (s_rate, c_rate)


# ---------------------------------------------------------------------------
# the transform alone
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("b", [16, 32, 64, 128])
@pytest.mark.parametrize("kind", ["orthogonal", "gaussian"])
def test_transform_values_within_bound(b, kind):
    M, K = 37, 40 * b
    xb = _x(M, K, seed=b)
    Tb = _T_bits(b, kind)
    x32 = synthetic.bf16_bits_to_f32(xb)
    T64 = F.bf16_bits_to_f64(Tb)
    announce(f"transform values b={b} {kind} M={M} K={K}")
    v = fql.transform_bf16(bf16_bits_to_dev(xb), _T_dev(Tb))
    torch.cuda.synchronize()
    v = v.cpu().numpy().astype(np.float64)
    v64 = TR.transform_f64(x32, T64)
    S = TR.transform_abs_sum(x32, T64)
    ratio = np.max(np.maximum(np.abs(v - v64) - _half_ulp(v64), 0) / np.maximum(S, 1e-300))
    print(f"[eps] b={b} {kind}: max |v - exact| beyond half an ulp = {ratio:.3e} * sum|T x| "
          f"(2^{np.log2(ratio) if ratio > 0 else -np.inf:.1f})")
    _, err = _bound(x32, T64)
    assert np.all(np.abs(v - v64) <= err)


@pytest.mark.parametrize("b", [16, 64])
def test_transform_exact_cases_bit_identical(b):
    g = synthetic.rng(9, b)
    x32 = (g.integers(-24, 25, size=(19, 8 * b)) * 0.25).astype(np.float32)
    xb = synthetic.f32_to_bf16_bits(x32)
    xd = bf16_bits_to_dev(xb)
    H = sylvester(b).astype(np.float64) * float(hadamard_scale_fp32(b))
    perm = synthetic.rng(10, b).permutation(b)
    P = np.zeros((b, b))
    P[np.arange(b), perm] = 1.0
    for name, T64 in (("identity", np.eye(b)), ("permutation", P), ("sylvester", H)):
        Td = _T_dev(synthetic.f32_to_bf16_bits(T64.astype(np.float32)))
        announce(f"transform exact {name} b={b}")
        v = fql.transform_bf16(xd, Td)
        codes, scales = fql.quant_nvfp4_transform(xd, Td, 37.5)
        torch.cuda.synchronize()
        ref_v = TR.block_transform(x32, T64)
        assert np.array_equal(v.cpu().numpy().view(np.uint32), ref_v.view(np.uint32)), name
        rc, rs = TR.quant_nvfp4_transform(x32, T64, np.float32(37.5))
        assert np.array_equal(scales.cpu().numpy(), rs), name
        assert np.array_equal(codes.cpu().numpy(), rc), name
        if name == "sylvester":  # the same codes as the Hadamard quantizer
            hc, hs = fql.quant_nvfp4(xd, 37.5, b)
            torch.cuda.synchronize()
            assert np.array_equal(hc.cpu().numpy(), rc) and np.array_equal(hs.cpu().numpy(), rs)


# ---------------------------------------------------------------------------
# transform + quantize
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("b", [16, 32, 64, 128])
@pytest.mark.parametrize("kind", ["orthogonal", "gaussian"])
@pytest.mark.parametrize("M", [1, 37])
def test_transform_quant_near_tie_rule(b, kind, M):
    K = 5120
    xb = _x(M, K, seed=M + b)
    Tb = _T_bits(b, kind, seed=1)
    x32 = synthetic.bf16_bits_to_f32(xb)
    T64 = F.bf16_bits_to_f64(Tb)
    g = Q.global_scale_from_amax(TR.tensor_amax(TR.block_transform(x32, T64)))
    announce(f"transform quant b={b} {kind} M={M} K={K}")
    codes, scales = fql.quant_nvfp4_transform(bf16_bits_to_dev(xb), _T_dev(Tb), float(g))
    torch.cuda.synchronize()
    _check_rule(x32, T64, g, codes.cpu().numpy(), scales.cpu().numpy(), f"b={b} {kind} M={M}")


@pytest.mark.parametrize("b", [16, 128])
def test_transform_quant_strided_and_unaligned(b):
    # row stride with padding, and a start offset of one element (unaligned loads)
    M, K = 21, 4 * 128
    xb = _x(M, K, seed=5)
    Tb = _T_bits(b, seed=2)
    Td = _T_dev(Tb)
    g = 211.0
    ref = fql.quant_nvfp4_transform(bf16_bits_to_dev(xb), Td, g)
    for pad, off in ((40, 0), (3, 1)):
        big = np.zeros((M, K + pad + off), np.uint16)
        big[:, off:off + K] = xb
        xd = bf16_bits_to_dev(big)[:, off:off + K]
        announce(f"transform quant strided b={b} pad={pad} off={off}")
        c, s = fql.quant_nvfp4_transform(xd, Td, g)
        torch.cuda.synchronize()
        assert torch.equal(c, ref[0]) and torch.equal(s, ref[1])
    _check_rule(synthetic.bf16_bits_to_f32(xb), F.bf16_bits_to_f64(Tb), np.float32(g),
                ref[0].cpu().numpy(), ref[1].cpu().numpy(), f"strided b={b}")


def test_transform_rejects_bad_arguments():
    x = torch.zeros((4, 96), dtype=torch.bfloat16, device=DEV)
    T = torch.zeros((64, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fql.FQLError):
        fql.quant_nvfp4_transform(x, T, 1.0)  # K % 64 != 0
    with pytest.raises(fql.FQLError):
        fql.quant_nvfp4_transform(x, torch.zeros((48, 48), dtype=torch.bfloat16, device=DEV), 1.0)
    with pytest.raises(fql.FQLError):
        fql.quant_nvfp4_transform(x, T[:32, :32].float(), 1.0)


# ---------------------------------------------------------------------------
# linear with the transform
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M", [1, 8, 32, 100, 300])
@pytest.mark.parametrize("b", [32, 128])
def test_linear_transform(M, b):
    K, N = 2048, 1152
    xb = _x(M, K, seed=M)
    Tb = _T_bits(b, seed=3)
    x32 = synthetic.bf16_bits_to_f32(xb)
    T64 = F.bf16_bits_to_f64(Tb)
    W = synthetic.weight(N, K, config="transform")
    gw = Q.global_scale_from_amax(Q.amax_for_calibration(W))
    wc, ws = Q.quant_nvfp4(W, gw)
    gx = Q.global_scale_from_amax(TR.tensor_amax(TR.block_transform(x32, T64)))
    xc, xs = TR.quant_nvfp4_transform(x32, T64, gx)
    alpha = alpha_of(gx, gw)
    ref = Q.linear_nvfp4(xc, xs, wc, ws, alpha)
    w = fql.NVFP4Weight.from_float(f32_to_dev(W), float(gx), weight_global_scale=float(gw),
                                   transform=_T_dev(Tb))
    announce(f"linear transform M={M} b={b} plan={fql.linear_plan(M, N, K, aligned=False, transform=True)}")
    y = fql.linear_nvfp4(bf16_bits_to_dev(xb), w)
    torch.cuda.synchronize()
    err = rel_frob(dev_bf16_to_bits(y), ref)
    assert err <= REL_FROB_TOL, err


# ---------------------------------------------------------------------------
# dynamic global scale
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["none", "hadamard64", "transform32", "transform128"])
def test_quant_dynamic(mode):
    M, K = 45, 5120
    xb = _x(M, K, seed=17)
    x32 = synthetic.bf16_bits_to_f32(xb)
    xd = bf16_bits_to_dev(xb)
    announce(f"dynamic quant {mode}")
    if mode.startswith("transform"):
        b = int(mode[len("transform"):])
        Tb = _T_bits(b, seed=4)
        T64 = F.bf16_bits_to_f64(Tb)
        codes, scales, sc = fql.quant_nvfp4_dynamic(xd, T=_T_dev(Tb))
    else:
        hb = 64 if mode == "hadamard64" else 0
        codes, scales, sc = fql.quant_nvfp4_dynamic(xd, hadamard_block=hb)
    torch.cuda.synchronize()
    amax_gpu, g_gpu = sc.cpu().numpy()[:2]
    # D2 on the device is bit-identical to the oracle's D2 of the same amax
    assert np.float32(g_gpu) == TR.dynamic_global_scale(np.float32(amax_gpu))
    if mode.startswith("transform"):
        v64, err = _bound(x32, T64)
        assert abs(float(amax_gpu) - np.max(np.abs(v64))) <= np.max(err)
        _check_rule(x32, T64, np.float32(g_gpu), codes.cpu().numpy(), scales.cpu().numpy(),
                    f"dynamic {mode}")
    else:
        a = Q.amax_for_calibration(x32, hb)
        assert np.float32(amax_gpu) == a
        rc, rs = Q.quant_nvfp4(x32, TR.dynamic_global_scale(a), hb)
        assert np.array_equal(codes.cpu().numpy(), rc) and np.array_equal(scales.cpu().numpy(), rs)


def test_quant_dynamic_edge_cases():
    K = 256
    zero = torch.zeros((3, K), dtype=torch.bfloat16, device=DEV)
    announce("dynamic quant zeros")
    c, s, sc = fql.quant_nvfp4_dynamic(zero)
    torch.cuda.synchronize()
    assert sc[1].item() == 1.0 and not c.any().item() and not s.any().item()
    # a tiny tensor: g reaches the 2^118 cap and codes stay finite (no NaN)
    tiny = np.full((2, K), 1e-34, np.float32)
    tiny[1, ::3] = -3e-35
    tb = synthetic.f32_to_bf16_bits(tiny)
    announce("dynamic quant tiny")
    c, s, sc = fql.quant_nvfp4_dynamic(bf16_bits_to_dev(tb))
    torch.cuda.synchronize()
    t32 = synthetic.bf16_bits_to_f32(tb)
    g = TR.dynamic_global_scale(TR.tensor_amax(t32))
    assert g == np.float32(2.0 ** 118) and sc[1].item() == float(g)
    rc, rs = Q.quant_nvfp4(t32, g)
    assert np.array_equal(c.cpu().numpy(), rc) and np.array_equal(s.cpu().numpy(), rs)


@pytest.mark.parametrize("M", [1, 24, 100, 300])
@pytest.mark.parametrize("mode", ["none", "hadamard32", "transform64"])
def test_linear_dynamic(M, mode):
    K, N = 2048, 640
    xb = _x(M, K, seed=M + 3)
    x32 = synthetic.bf16_bits_to_f32(xb)
    W = synthetic.weight(N, K, config="transform")
    hb = 32 if mode == "hadamard32" else 0
    gw = Q.global_scale_from_amax(Q.amax_for_calibration(W, hb))
    wc, ws = Q.quant_nvfp4(W, gw, hb)  # the weight is rotated with the same block
    T = None
    v = x32
    if mode == "transform64":
        Tb = _T_bits(64, seed=5)
        v = TR.block_transform(x32, F.bf16_bits_to_f64(Tb))
        T = _T_dev(Tb)
    elif mode == "hadamard32":
        v = fwht_fp32(x32, hb)
    gx = TR.dynamic_global_scale(TR.tensor_amax(v))
    xc, xs = Q.quant_nvfp4(v, gx)
    ref = Q.linear_nvfp4(xc, xs, wc, ws, TR.dynamic_alpha(gx, gw))
    w = fql.NVFP4Weight.from_float(f32_to_dev(W), 1.0, hadamard_block=hb,
                                   weight_global_scale=float(gw), transform=T,
                                   dynamic_input_scale=True)
    announce(f"linear dynamic M={M} {mode}")
    y = fql.linear_nvfp4(bf16_bits_to_dev(xb), w)
    torch.cuda.synchronize()
    err = rel_frob(dev_bf16_to_bits(y), ref)
    assert err <= REL_FROB_TOL, err
    if mode != "transform64":  # no accumulation-order freedom: alpha and x_hat are exact
        # the same codes as the static path given the same g and alpha
        ws_ = fql.NVFP4Weight.from_float(f32_to_dev(W), float(gx), hadamard_block=hb,
                                         weight_global_scale=float(gw))
        y2 = fql.linear_nvfp4(bf16_bits_to_dev(xb), ws_, alpha=float(TR.dynamic_alpha(gx, gw)))
        torch.cuda.synchronize()
        if M > 16:  # both take x_hat plans (below, the static path may fuse the quantizer)
            assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("b,K", [(16, 1040), (32, 1056), (64, 1088), (128, 1152), (128, 5120)])
@pytest.mark.parametrize("M", [1, 5, 17, 32])
def test_linear_transform_packed_ring_and_xhat_gemm(b, K, M, plan_override):
    # the transform kernel's packed activation (small-M ring) and its x_hat
    # (LDS-ring GEMM) hold the same quantized values; the kernels sum in
    # different orders, so both are held to the oracle and to each other within
    # the output bar (K not a multiple of 128: the packed blocks past K are zero)
    N = 272
    xb = _x(M, K, seed=M + b)
    Tb = _T_bits(b, seed=b)
    W = synthetic.weight(N, K, config="transform")
    w = fql.NVFP4Weight.from_float(f32_to_dev(W), 5.0, transform=_T_dev(Tb))
    announce(f"transform packed vs x_hat b={b} K={K} M={M}")
    outs = []
    for spec, kernel in (("kind=4,waves=4,nt=2,st=3", "gemv_ring_kernel"),
                         ("kind=3,mt=2,nt=1,st=4,cw=4", "gemm_lds32_kernel")):
        plan_override(spec)
        assert kernel in fql.linear_plan(M, N, K, aligned=False, transform=True)
        outs.append(dev_bf16_to_bits(fql.linear_nvfp4(bf16_bits_to_dev(xb), w)))
    assert rel_frob(outs[0], outs[1]) <= REL_FROB_TOL
    v = TR.block_transform(synthetic.bf16_bits_to_f32(xb), F.bf16_bits_to_f64(Tb))
    xc, xs = Q.quant_nvfp4(v, np.float32(5.0))
    gw = np.float32(w.weight_global_scale)
    wc, ws = Q.quant_nvfp4(W, gw)
    ref = Q.linear_nvfp4(xc, xs, wc, ws, alpha_of(np.float32(5.0), gw))
    for y in outs:
        assert rel_frob(y, ref) <= REL_FROB_TOL


@pytest.mark.parametrize("mode", ["none", "hadamard32", "transform64"])
def test_linear_dynamic_small_m_ring(mode, plan_override):
    # the small-M ring: the dynamic scale reaches the quantizer pass through the
    # device scalar; under a transform the transform kernel writes the packed
    # activation
    plan_override("kind=4,waves=4,nt=2,st=3")
    M, K, N = 24, 2048, 640
    xb = _x(M, K, seed=77)
    x32 = synthetic.bf16_bits_to_f32(xb)
    W = synthetic.weight(N, K, config="transform")
    hb = 32 if mode == "hadamard32" else 0
    gw = Q.global_scale_from_amax(Q.amax_for_calibration(W, hb))
    wc, ws = Q.quant_nvfp4(W, gw, hb)
    T = None
    v = x32
    if mode == "transform64":
        Tb = _T_bits(64, seed=5)
        v = TR.block_transform(x32, F.bf16_bits_to_f64(Tb))
        T = _T_dev(Tb)
    elif mode == "hadamard32":
        v = fwht_fp32(x32, hb)
    gx = TR.dynamic_global_scale(TR.tensor_amax(v))
    ref = Q.linear_nvfp4(*Q.quant_nvfp4(v, gx), wc, ws, TR.dynamic_alpha(gx, gw))
    w = fql.NVFP4Weight.from_float(f32_to_dev(W), 1.0, hadamard_block=hb,
                                   weight_global_scale=float(gw), transform=T,
                                   dynamic_input_scale=True)
    announce(f"linear dynamic small-M ring {mode}")
    plan = fql.linear_plan(M, N, K, aligned=False, transform=T is not None)
    assert "gemv_ring_kernel" in plan, plan
    if T is not None:
        assert plan.startswith("transform_quant_kernel + "), plan
    y = fql.linear_nvfp4(bf16_bits_to_dev(xb), w)
    torch.cuda.synchronize()
    err = rel_frob(dev_bf16_to_bits(y), ref)
    assert err <= REL_FROB_TOL, err


@pytest.mark.parametrize("mode", ["transform", "dynamic"])
def test_graph_replay(mode):
    M, K, N = 24, 1024, 512
    xb = _x(M, K, seed=8)
    Tb = _T_bits(32, seed=6)
    W = f32_to_dev(synthetic.weight(N, K, config="transform"))
    w = fql.NVFP4Weight.from_float(W, 3.0, transform=_T_dev(Tb),
                                   dynamic_input_scale=(mode == "dynamic"))
    x = bf16_bits_to_dev(xb)
    other = bf16_bits_to_dev(_x(M, K, seed=9))
    ws = fql.new_workspace(fql.linear_workspace_bytes(M, N, K), DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    announce(f"graph replay {mode}")
    fql.linear_nvfp4(x, w, out=y, workspace=ws)
    torch.cuda.synchronize()
    eager = y.clone()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        fql.linear_nvfp4(x, w, out=y, workspace=ws)
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            fql.linear_nvfp4(x, w, out=y, workspace=ws)
    for r in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
        fql.linear_nvfp4(other, w, workspace=ws)  # eager call on the same workspace in between
        torch.cuda.synchronize()


@pytest.mark.parametrize("K,b,M", [(208, 16, 1), (208, 16, 40), (96, 32, 17), (64, 64, 3),
                                   (128, 128, 1), (384, 128, 33)])
def test_linear_transform_ragged_k(K, b, M):
    # K not a multiple of 128 (x_hat columns K..Kp are zero padded; K = 208 leaves
    # half of a 32-column step), a single chunk (K = b), and ragged row counts
    N = 80
    xb = _x(M, K, seed=K + M)
    Tb = _T_bits(b, "gaussian", seed=7)
    x32 = synthetic.bf16_bits_to_f32(xb)
    T64 = F.bf16_bits_to_f64(Tb)
    W = synthetic.weight(N, K, config="transform", seed=1)
    gw = Q.global_scale_from_amax(Q.amax_for_calibration(W))
    wc, ws = Q.quant_nvfp4(W, gw)
    gx = Q.global_scale_from_amax(TR.tensor_amax(TR.block_transform(x32, T64)))
    xc, xs = TR.quant_nvfp4_transform(x32, T64, gx)
    ref = Q.linear_nvfp4(xc, xs, wc, ws, alpha_of(gx, gw))
    Td = _T_dev(Tb)
    xd = bf16_bits_to_dev(xb)
    announce(f"linear transform ragged K={K} b={b} M={M}")
    codes, scales = fql.quant_nvfp4_transform(xd, Td, float(gx))
    w = fql.NVFP4Weight.from_float(f32_to_dev(W), float(gx), weight_global_scale=float(gw), transform=Td)
    y = fql.linear_nvfp4(xd, w)
    wd = fql.NVFP4Weight.from_float(f32_to_dev(W), 1.0, weight_global_scale=float(gw), transform=Td,
                                    dynamic_input_scale=True)
    yd = fql.linear_nvfp4(xd, wd)
    torch.cuda.synchronize()
    _check_rule(x32, T64, gx, codes.cpu().numpy(), scales.cpu().numpy(), f"ragged K={K} b={b} M={M}")
    assert rel_frob(dev_bf16_to_bits(y), ref) <= REL_FROB_TOL
    gxd = TR.dynamic_global_scale(TR.tensor_amax(TR.block_transform(x32, T64)))
    xcd, xsd = TR.quant_nvfp4_transform(x32, T64, gxd)
    refd = Q.linear_nvfp4(xcd, xsd, wc, ws, TR.dynamic_alpha(gxd, gw))
    assert rel_frob(dev_bf16_to_bits(yd), refd) <= REL_FROB_TOL


def test_transform_values_3d_input_and_row_stride():
    # [B, S, K] input flattened without a copy, and a padded row stride for the values
    b, K = 32, 256
    xb = _x(6, K, seed=30)
    Tb = _T_bits(b, seed=8)
    x3 = bf16_bits_to_dev(xb).view(2, 3, K)
    announce("transform values 3-d")
    v = fql.transform_bf16(x3, _T_dev(Tb))
    torch.cuda.synchronize()
    assert v.shape == (2, 3, K)
    x32 = synthetic.bf16_bits_to_f32(xb)
    v64, err = _bound(x32, F.bf16_bits_to_f64(Tb))
    assert np.all(np.abs(v.reshape(6, K).cpu().numpy().astype(np.float64) - v64) <= err)


@pytest.mark.parametrize("b", [16, 128])
@pytest.mark.parametrize("shape", ["gate_up", "down"])
@pytest.mark.parametrize("M", [1, 256, 4096])
def test_linear_transform_full_size_sampled(b, shape, M):
    # the general-transform workload at its full sizes (Qwen3-32B gate_up /
    # down), the launch configuration the bench times; the oracle computes a
    # seeded sample of rows and columns in full
    from gpu_helpers import cached_activations, cached_weight

    K, N = synthetic.QWEN_SHAPES[shape]
    r = np.random.default_rng(b + M + K)
    rows = np.arange(M) if M == 1 else np.sort(r.choice(M, 24, replace=False))
    cols = np.sort(r.choice(N, 48, replace=False))
    cols[-1] = N - 1
    xb = cached_activations("student_t3", M, K, "transform")
    Tb = _T_bits(b)
    T64 = F.bf16_bits_to_f64(Tb)
    x32s = synthetic.bf16_bits_to_f32(xb[rows])
    W = cached_weight("transform", N, K)
    gw = Q.global_scale_from_amax(Q.amax_for_calibration(W[cols]))
    wc, ws = Q.quant_nvfp4(W[cols], gw)
    gx = Q.global_scale_from_amax(TR.tensor_amax(TR.block_transform(x32s, T64)))
    xc, xs = TR.quant_nvfp4_transform(x32s, T64, gx)
    ref = Q.linear_nvfp4(xc, xs, wc, ws, alpha_of(gx, gw))
    announce(f"linear transform full size {shape} M={M} b={b} plan={fql.linear_plan(M, N, K, aligned=False, transform=True)}")
    w = fql.NVFP4Weight.from_float(f32_to_dev(W), float(gx), weight_global_scale=float(gw),
                                   transform=_T_dev(Tb))
    y = fql.linear_nvfp4(bf16_bits_to_dev(xb), w)
    torch.cuda.synchronize()
    got = dev_bf16_to_bits(y)[np.ix_(rows, cols)]
    err = rel_frob(got, ref)
    assert err <= REL_FROB_TOL, err


def test_linear_dynamic_full_size_sampled():
    # dynamic scale over the whole 4096 x 25600 transformed activation
    from gpu_helpers import cached_activations, cached_weight

    M, b = 4096, 128
    K, N = synthetic.QWEN_SHAPES["down"]
    r = np.random.default_rng(7)
    rows = np.sort(r.choice(M, 24, replace=False))
    cols = np.sort(r.choice(N, 48, replace=False))
    xb = cached_activations("student_t3", M, K, "transform")
    Tb = _T_bits(b)
    T64 = F.bf16_bits_to_f64(Tb)
    x32 = synthetic.bf16_bits_to_f32(xb)
    amax = np.float32(0)
    for r0 in range(0, M, 512):  # the tensor amax in row blocks (bounded host memory)
        amax = max(amax, TR.tensor_amax(TR.block_transform(x32[r0:r0 + 512], T64)))
    gx = TR.dynamic_global_scale(amax)
    W = cached_weight("transform", N, K)
    gw = Q.global_scale_from_amax(Q.amax_for_calibration(W[cols]))
    wc, ws = Q.quant_nvfp4(W[cols], gw)
    xc, xs = TR.quant_nvfp4_transform(x32[rows], T64, gx)
    ref = Q.linear_nvfp4(xc, xs, wc, ws, TR.dynamic_alpha(gx, gw))
    announce("linear dynamic full size down M=4096 b=128")
    w = fql.NVFP4Weight.from_float(f32_to_dev(W), 1.0, weight_global_scale=float(gw),
                                   transform=_T_dev(Tb), dynamic_input_scale=True)
    y = fql.linear_nvfp4(bf16_bits_to_dev(xb), w)
    torch.cuda.synchronize()
    err = rel_frob(dev_bf16_to_bits(y)[np.ix_(rows, cols)], ref)
    assert err <= REL_FROB_TOL, err
