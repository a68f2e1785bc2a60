"""The library and the oracle against the numbers the pages fix (CPU only).

tests/golden/pages_facts.json holds each number with its page and section.
"""

import json
import math
import os

import numpy as np
import pytest

import fp8_quantized_linear_amd as fql
from oracle import hadamard as H
from oracle import nvfp4 as Q

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))


def test_hadamard_block_sizes_accepted_exactly():
    sizes = FACTS["hadamard_block_sizes"]["value"]
    for b in range(0, 257):
        ok, _ = fql.can_implement(4096, 2560 * 4, b) if 10240 % max(b, 1) == 0 else (None, None)
        if ok is None:
            continue
        assert ok == (b == 0 or b in sizes), b


@pytest.mark.parametrize("b", FACTS["hadamard_block_sizes"]["value"])
def test_hadamard_normalisation_is_inverse_sqrt(b):
    # the oracle's scale is 1/sqrt(b) rounded once to float32
    assert FACTS["hadamard_normalisation"]["value"] == "1/sqrt(n)"
    assert float(H.hadamard_scale_fp32(b)) == float(np.float32(1.0 / math.sqrt(b)))


def test_two_fp4_values_per_byte():
    per_byte = FACTS["fp4_values_per_byte"]["value"]
    x = np.random.default_rng(5).standard_normal((3, 64)).astype(np.float32)
    codes, scales = Q.quant_nvfp4(x, np.float32(100.0))
    assert codes.shape == (3, 64 // per_byte)
    assert scales.shape == (3, 64 // 16)
    # the packed weight blob stores K/2 code bytes per row (plus scales)
    assert fql.packed_nvfp4_bytes(16, 128) >= 16 * 128 // per_byte


def test_fp8_group_shapes_recorded():
    g = FACTS["fp8_block_group_shapes"]
    assert g["activation"] == [1, 128] and g["weight"] == [128, 128] and g["feature_alignment"] == 128
