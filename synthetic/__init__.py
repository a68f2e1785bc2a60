"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module only draws random numbers and casts them to the input dtypes; it
holds none of the method's arithmetic (no quantization, no scales, no
rotation). Every draw uses numpy's PCG64 generator keyed by
(stream, config id, shape...), so any array can be regenerated on its own.

Workloads stand in for the layer shapes the vLLM write-ups benchmark on
(Llama-3.1-8B and Qwen3-32B linear layers; the write-ups' GSM8K and
perplexity runs need trained checkpoints and are not reproduced):

* ``tiny``:    x [16, 256] ~ N(0, 1); W [512, 256] ~ N(0, 0.02^2); no bias.
* ``decode``:  M in {1, 8, 32, 128}; (K, N) in {(4096, 6144) qkv,
               (4096, 28672) gate_up, (14336, 4096) down}; x ~ N(0, 1);
               W ~ N(0, 0.02^2); bias ~ N(0, 0.01^2) in bfloat16.
* ``prefill``: the same shapes at M in {2048, 8192}; x ~ N(0, 1) with
               round(0.01 K) channels (a seeded choice) scaled by 20; no bias.
* ``hadamard``: (K, N) in {(5120, 51200) gate_up, (25600, 5120) down} at
               M in {1, 256, 4096}; x ~ Student-t(3); W ~ N(0, 0.02^2);
               Hadamard block in {16, 32, 64, 128}.
* ``siblings``: K = 4096, N = 14336, M in {1, 4096}; x ~ N(0, 1);
               W ~ N(0, 0.02^2).
* ``transform``: the ``hadamard`` shapes and activations with a general
               b x b transform matrix (b in {16, 32, 64, 128}) drawn by
               ``transform_matrix``: a random orthogonal matrix (QR of a
               Gaussian draw, signs fixed by R's diagonal) or a Gaussian one
               with entries N(0, 1/b), cast to bfloat16.
"""

import numpy as np

STREAM_X, STREAM_W, STREAM_BIAS, STREAM_OUTLIER, STREAM_T = 0, 1, 2, 3, 4

CONFIG_IDS = {"tiny": 0, "decode": 1, "prefill": 2, "hadamard": 3, "siblings": 4, "transform": 5}

LLAMA_SHAPES = {"qkv": (4096, 6144), "gate_up": (4096, 28672), "down": (14336, 4096)}
QWEN_SHAPES = {"gate_up": (5120, 51200), "down": (25600, 5120)}

WORKLOADS = {
    "tiny": {"M": (16,), "shapes": {"tiny": (256, 512)}, "bias": False,
             "x": "normal", "hadamard": (0,)},
    "decode": {"M": (1, 8, 32, 128), "shapes": LLAMA_SHAPES, "bias": True,
               "x": "normal", "hadamard": (0,)},
    "prefill": {"M": (2048, 8192), "shapes": LLAMA_SHAPES, "bias": False,
                "x": "normal_outliers", "hadamard": (0,)},
    "hadamard": {"M": (1, 256, 4096), "shapes": QWEN_SHAPES, "bias": False,
                 "x": "student_t3", "hadamard": (16, 32, 64, 128)},
    "siblings": {"M": (1, 4096), "shapes": {"sib": (4096, 14336)}, "bias": False,
                 "x": "normal", "hadamard": (0,)},
    "transform": {"M": (1, 256, 4096), "shapes": QWEN_SHAPES, "bias": False,
                  "x": "student_t3", "hadamard": (16, 32, 64, 128)},
}


def rng(stream, *key):
    """A PCG64 generator for one named stream and integer key."""
    return np.random.Generator(np.random.PCG64([int(stream)] + [int(k) for k in key]))


def f32_to_bf16_bits(a):
    """Cast float32 values to bfloat16 bit patterns (uint16), round to nearest even.

    Input preparation only: uses torch's CPU cast.
    """
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits):
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def activations(kind, M, K, config="decode", seed=0):
    """x [M, K] as bfloat16 bit patterns (uint16) for the named distribution."""
    cid = CONFIG_IDS[config]
    g = rng(STREAM_X, cid, seed, M, K)
    if kind == "normal":
        x = g.standard_normal((M, K), dtype=np.float32)
    elif kind == "normal_outliers":
        x = g.standard_normal((M, K), dtype=np.float32)
        n_out = int(round(0.01 * K))
        cols = rng(STREAM_OUTLIER, cid, seed, K).permutation(K)[:n_out]
        x[:, cols] *= np.float32(20.0)
    elif kind == "student_t3":
        x = g.standard_t(3, size=(M, K)).astype(np.float32)
    else:
        raise ValueError(kind)
    return f32_to_bf16_bits(x)


def weight(N, K, config="decode", seed=0, std=0.02, rows=None):
    """W [N, K] float32 ~ N(0, std^2), or only its first `rows` rows (the same
    values: the draws fill the matrix row by row)."""
    g = rng(STREAM_W, CONFIG_IDS[config], seed, N, K)
    n = N if rows is None else min(int(rows), N)
    return (g.standard_normal((n, K), dtype=np.float32) * np.float32(std)).astype(np.float32)


def bias(N, config="decode", seed=0, std=0.01):
    """bias [N] as bfloat16 bit patterns ~ N(0, std^2)."""
    g = rng(STREAM_BIAS, CONFIG_IDS[config], seed, N)
    return f32_to_bf16_bits(g.standard_normal(N, dtype=np.float32) * np.float32(std))


def transform_matrix(b, kind="orthogonal", seed=0):
    """A b x b transform matrix as bfloat16 bit patterns (uint16) [b, b]."""
    g = rng(STREAM_T, CONFIG_IDS["transform"], seed, b, 0 if kind == "orthogonal" else 1)
    a = g.standard_normal((b, b))
    if kind == "orthogonal":
        q, r = np.linalg.qr(a)
        a = q * np.sign(np.diag(r))[None, :]
    elif kind == "gaussian":
        a = a / np.sqrt(b)
    else:
        raise ValueError(kind)
    return f32_to_bf16_bits(a.astype(np.float32))


def cases(config):
    """Yield (M, shape_name, K, N, hadamard_block, with_bias) for a workload."""
    w = WORKLOADS[config]
    for name, (K, N) in w["shapes"].items():
        for M in w["M"]:
            for hb in w["hadamard"]:
                yield M, name, K, N, hb, w["bias"]
