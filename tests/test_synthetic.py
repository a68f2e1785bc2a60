"""The seeded input generators (CPU): draws only, no method arithmetic."""

import numpy as np

import synthetic


def test_weight_rows_are_the_full_matrix_rows():
    # the bounded samples draw only the first rows of a weight; they are the same
    # values as those rows of the whole matrix
    full = synthetic.weight(300, 272, config="decode", seed=3)
    assert np.array_equal(synthetic.weight(300, 272, config="decode", seed=3, rows=17), full[:17])


def test_generators_are_deterministic():
    a = synthetic.activations("normal_outliers", 8, 4096, config="prefill")
    b = synthetic.activations("normal_outliers", 8, 4096, config="prefill")
    assert a.dtype == np.uint16 and np.array_equal(a, b)
    # 1% of the channels carry the x20 outliers
    x = synthetic.bf16_bits_to_f32(a)
    assert (np.abs(x).max(axis=0) > 12).sum() >= 30
