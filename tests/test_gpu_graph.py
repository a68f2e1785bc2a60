"""HIP-graph capture, in-place repacking and warmup (GPU).

Every linear call is stream-ordered, allocates nothing when given a
workspace and leaves the workspace's arrival counters at zero, so a captured
call replays like the eager one. Each graph here is replayed several times
with other eager work and synchronizations in between, and every replay is
compared bit for bit with the eager result (the kernels are deterministic:
split-K partial sums are added in split order). Repacking a weight into its
own storage keeps the address, so a captured graph picks up the new weight
(B12X write-up, Implementation: packed storage reused so captured graphs stay
valid).
"""

import numpy as np
import pytest
import torch

import fp8_quantized_linear_amd as fql
import synthetic

from gpu_helpers import DEV, announce, bf16_bits_to_dev, cached_weight, f32_to_dev

pytestmark = pytest.mark.gpu


def _nvfp4_weight(N, K, seed=0):
    W = synthetic.weight(N, K, config="decode", seed=seed)
    return fql.NVFP4Weight.from_float(f32_to_dev(W), input_global_scale=0.37)


def _sc_weight(fmt, N, K, seed=0):
    W = f32_to_dev(synthetic.weight(N, K, config="siblings", seed=seed))
    if fmt == "fp8":
        return fql.FP8Weight.from_float(W, input_scale=0.01)
    return {"mxfp4": fql.MXFP4Weight, "mxfp8": fql.MXFP8Weight,
            "fp8_block": fql.FP8BlockWeight}[fmt].from_float(W)


LINEAR = {"nvfp4": fql.linear_nvfp4, "mxfp4": fql.linear_mxfp4, "mxfp8": fql.linear_mxfp8,
          "fp8": fql.linear_fp8, "fp8_block": fql.linear_fp8_block}


def _ws_bytes(fmt, M, N, K):
    if fmt == "nvfp4":
        return fql.linear_workspace_bytes(M, N, K)
    return fql.linear_sc_workspace_bytes(fmt, M, N, K)


@pytest.mark.parametrize("fmt,M", [("nvfp4", 1), ("nvfp4", 8), ("nvfp4", 24), ("nvfp4", 100),
                                   ("nvfp4", 300), ("mxfp4", 1), ("mxfp4", 200), ("mxfp8", 16),
                                   ("fp8", 64), ("fp8_block", 5), ("fp8_block", 600)])
def test_graph_replay_matches_eager(fmt, M):
    K, N = 2048, 1152
    w = _nvfp4_weight(N, K) if fmt == "nvfp4" else _sc_weight(fmt, N, K)
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
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        fn(x, w, out=y, workspace=ws)  # warm the capture stream
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            fn(x, w, out=y, workspace=ws)
    for r in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {r} differs"
        z = fn(other, w)  # eager work between replays (own workspace and output)
        torch.cuda.synchronize()
        assert z.shape == (M, N)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4", "fp8_block"])
def test_repack_in_place_updates_captured_graph(fmt):
    K, N, M = 1024, 640, 4
    if fmt == "nvfp4":
        w = _nvfp4_weight(N, K, seed=1)
        w2 = _nvfp4_weight(N, K, seed=2)
        w2.input_global_scale = w.input_global_scale
        codes, scales = fql.unpack_weight_nvfp4(w2.packed, N, K)
    else:
        w = _sc_weight(fmt, N, K, seed=1)
        W2 = f32_to_dev(synthetic.weight(N, K, config="siblings", seed=2))
        codes, scales = (fql.quant_mxfp4_weight(W2) if fmt == "mxfp4"
                         else fql.quant_fp8_block_weight(W2))
    fn = LINEAR[fmt]
    x = bf16_bits_to_dev(synthetic.activations("normal", M, K, config="decode", seed=3))
    ws = fql.new_workspace(_ws_bytes(fmt, M, N, K), DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    announce(f"repack in place under a graph: {fmt}")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        fn(x, w, out=y, workspace=ws)
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            fn(x, w, out=y, workspace=ws)
    addr = w.packed.data_ptr()
    w.repack_(codes, scales)  # new weight, same storage
    assert w.packed.data_ptr() == addr
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    if fmt == "nvfp4":
        ref = fql.linear_nvfp4(x, w, alpha=w.alpha)
    else:
        ref = fn(x, w)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


def test_warmup_dedupes_layers_and_counts():
    K, N = 1024, 512
    a = _nvfp4_weight(N, K, seed=4)
    b = _nvfp4_weight(N, K, seed=5)  # same signature as a
    c = _sc_weight("mxfp8", N, K)
    counts = fql.token_counts_for_warmup(256, graph_sizes=(1, 8, 32))
    assert counts == [1, 8, 32, 256]
    announce("warmup")
    n = fql.warmup([a, b, c], counts)
    torch.cuda.synchronize()
    assert n == 2 * len(counts)
