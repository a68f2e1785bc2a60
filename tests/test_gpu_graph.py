"""HIP-graph capture, in-place repacking and warmup (GPU).

Every linear call is stream-ordered, allocates nothing when given a
workspace and leaves the workspace's arrival counters at zero, so a captured
call replays like the eager one. Each graph here is replayed several times
with other eager work and synchronizations in between; every replay is
compared bit for bit with the eager result (the kernels are deterministic:
split-K partial sums are added in split order) and with the oracle.
Repacking a weight into its own storage keeps the address, and a weight's
alpha lives in device memory, so a captured graph picks up the new weight
and its new global scale (B12X write-up, Implementation: packed storage is
reused so captured graphs stay valid).
"""

import numpy as np
import pytest
import torch

import fp8_quantized_linear_amd as fql
import synthetic
from oracle import fp8 as P
from oracle import mx as X
from oracle import nvfp4 as Q

from gpu_helpers import (DEV, REL_FROB_TOL, alpha_of, announce, bf16_bits_to_dev,
                         dev_bf16_to_bits, f32_to_dev, rel_frob)

pytestmark = pytest.mark.gpu

G_X = 0.37     # static activation global scale of the NVFP4 layer
S_X = 0.011    # static activation scale of the per-tensor FP8 layer


def _w(seed, N, K, config):
    return synthetic.weight(N, K, config=config, seed=seed)


def _gpu_weight(fmt, W):
    """GPU weight from W (global / per-tensor scales from the library's calibration)."""
    wd = f32_to_dev(W)
    if fmt == "nvfp4":
        return fql.NVFP4Weight.from_float(wd, input_global_scale=G_X)
    if fmt == "fp8":
        return fql.FP8Weight.from_float(wd, input_scale=S_X)
    return {"mxfp4": fql.MXFP4Weight, "mxfp8": fql.MXFP8Weight,
            "fp8_block": fql.FP8BlockWeight}[fmt].from_float(wd)


def _oracle(fmt, xb, W):
    """The oracle's output for activation bits xb and float32 weight W (scales
    calibrated by the oracle itself)."""
    x32 = synthetic.bf16_bits_to_f32(xb)
    if fmt == "nvfp4":
        gw = Q.global_scale_from_amax(Q.amax_for_calibration(W))
        return Q.linear_nvfp4(*Q.quant_nvfp4(x32, np.float32(G_X)), *Q.quant_nvfp4(W, gw),
                              alpha_of(G_X, gw))
    if fmt == "fp8":
        s_w = P.scale_from_amax(np.abs(W).max())
        s_x = np.float32(S_X)
        return P.linear_fp8_tensor(P.quant_fp8_tensor(x32, s_x), P.quant_fp8_tensor(W, s_w),
                                   P.output_scale(s_x, s_w))
    if fmt == "mxfp4":
        return X.linear_mxfp4(*X.quant_mxfp4(x32), *X.quant_mxfp4(W))
    if fmt == "mxfp8":
        return P.linear_mxfp8(*P.quant_mxfp8(x32), *P.quant_mxfp8(W))
    return P.linear_fp8_block(*P.quant_fp8_block_act(x32), *P.quant_fp8_block_weight(W))


LINEAR = {"nvfp4": fql.linear_nvfp4, "mxfp4": fql.linear_mxfp4, "mxfp8": fql.linear_mxfp8,
          "fp8": fql.linear_fp8, "fp8_block": fql.linear_fp8_block}


def _ws_bytes(fmt, M, N, K):
    if fmt == "nvfp4":
        return fql.linear_workspace_bytes(M, N, K)
    return fql.linear_sc_workspace_bytes(fmt, M, N, K)


def _capture(fn, x, w, y, ws):
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        fn(x, w, out=y, workspace=ws)  # warm the capture stream
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            fn(x, w, out=y, workspace=ws)
    return g


@pytest.mark.parametrize("fmt,M", [("nvfp4", 1), ("nvfp4", 8), ("nvfp4", 24), ("nvfp4", 100),
                                   ("nvfp4", 300), ("mxfp4", 1), ("mxfp4", 200), ("mxfp8", 16),
                                   ("fp8", 64), ("fp8_block", 5), ("fp8_block", 600)])
def test_graph_replay_matches_eager_and_oracle(fmt, M):
    K, N = 2048, 1152
    config = "decode" if fmt == "nvfp4" else "siblings"
    W = _w(0, N, K, config)
    w = _gpu_weight(fmt, W)
    fn = LINEAR[fmt]
    xb = synthetic.activations("normal", M, K, config="decode", seed=M)
    x = bf16_bits_to_dev(xb)
    other = bf16_bits_to_dev(synthetic.activations("normal", M, K, config="decode", seed=M + 1))
    ws = fql.new_workspace(_ws_bytes(fmt, M, N, K), DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    announce(f"graph replay {fmt} M={M}")
    fn(x, w, out=y, workspace=ws)
    torch.cuda.synchronize()
    eager = y.clone()
    ref = _oracle(fmt, xb, W)
    assert rel_frob(dev_bf16_to_bits(eager), ref) <= REL_FROB_TOL
    g = _capture(fn, x, w, y, ws)
    for r in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {r} differs"
        assert rel_frob(dev_bf16_to_bits(y), ref) <= REL_FROB_TOL
        z = fn(other, w)  # eager work between replays (own workspace and output)
        torch.cuda.synchronize()
        assert z.shape == (M, N)


@pytest.mark.parametrize("fmt,M", [("nvfp4", 4), ("nvfp4", 8), ("nvfp4", 200), ("fp8", 4),
                                   ("fp8", 100), ("mxfp4", 4), ("fp8_block", 4)])
def test_repack_in_place_updates_captured_graph(fmt, M):
    # a graph captured on weight 1 replays weight 2 after repack_ into the same
    # storage, including weight 2's own global scale (alpha kept on the device)
    K, N = 1024, 640
    config = "decode" if fmt == "nvfp4" else "siblings"
    W1, W2 = _w(1, N, K, config), 3.0 * _w(2, N, K, config)  # a different amax
    w = _gpu_weight(fmt, W1)
    fn = LINEAR[fmt]
    xb = synthetic.activations("normal", M, K, config="decode", seed=3)
    x = bf16_bits_to_dev(xb)
    ws = fql.new_workspace(_ws_bytes(fmt, M, N, K), DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    announce(f"repack in place under a graph: {fmt} M={M}")
    g = _capture(fn, x, w, y, ws)
    addr = w.packed.data_ptr()
    W2d = f32_to_dev(W2)
    if fmt == "nvfp4":
        gw2 = fql.global_scale_from_amax(fql.amax(W2d).item())
        w.repack_(*fql.quant_nvfp4_weight(W2d, gw2), weight_global_scale=gw2)
    elif fmt == "fp8":
        sw2 = fql.fp8_scale_from_amax(fql.amax(W2d).item())
        w.repack_(fql.quant_fp8_weight(W2d, sw2), weight_scale=sw2)
    elif fmt == "mxfp4":
        w.repack_(*fql.quant_mxfp4_weight(W2d))
    else:
        w.repack_(*fql.quant_fp8_block_weight(W2d))
    assert w.packed.data_ptr() == addr
    torch.cuda.synchronize()
    ref = _oracle(fmt, xb, W2)
    for r in range(2):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert rel_frob(dev_bf16_to_bits(y), ref) <= REL_FROB_TOL, f"replay {r}"
    eager = fn(x, w)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), eager.view(torch.int16))


def test_repack_rejects_a_new_scale_for_a_transform_weight():
    K, N = 256, 64
    W = f32_to_dev(_w(4, N, K, "decode"))
    T = torch.eye(16, dtype=torch.bfloat16, device=DEV)
    announce("repack scale rejection")
    w = fql.NVFP4Weight.from_float(W, input_global_scale=1.0, transform=T)
    codes, scales = fql.quant_nvfp4_weight(W, w.weight_global_scale)
    w.repack_(codes, scales, weight_global_scale=w.weight_global_scale)  # same scale: fine
    with pytest.raises(fql.FQLError):
        w.repack_(codes, scales, weight_global_scale=2.0 * w.weight_global_scale)


def test_warmup_dedupes_layers_and_counts():
    K, N = 1024, 512
    a = _gpu_weight("nvfp4", _w(4, N, K, "decode"))
    b = _gpu_weight("nvfp4", _w(5, N, K, "decode"))  # same signature as a
    c = _gpu_weight("mxfp8", _w(0, N, K, "siblings"))
    counts = fql.token_counts_for_warmup(256, graph_sizes=(1, 8, 32))
    assert counts == [1, 8, 32, 256]
    announce("warmup")
    n = fql.warmup([a, b, c], counts)
    torch.cuda.synchronize()
    assert n == 2 * len(counts)
