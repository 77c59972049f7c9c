"""Pins of the W4A16 product oracle (CPU only).

Each test compares the oracle with something it does not share code with: a
hand-worked fixture, the quantizer's own dequantized weights, a brute-force
loop, or an exact invariance."""
import json
import os

import numpy as np
import pytest

import oracle as O
from oracle import w4a16_oracle as W
from post_weight_quantization_layer_amd import inputs as I

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example():
    g = json.load(open(os.path.join(GOLD, "w4a16_worked.json")))
    bits = np.array([[int(v, 16) for v in row] for row in g["x_f16_bits"]], dtype=np.uint16)
    np.testing.assert_array_equal(W.f16_bits_to_f64(bits), np.array(g["x_values"]))
    What = W.dequantize_stored(g["codes"], g["g_idx"], g["scale"], g["zero"])
    np.testing.assert_array_equal(What, np.array(g["what"]))
    y = W.w4a16_product(bits, g["codes"], g["g_idx"], g["scale"], g["zero"])
    np.testing.assert_array_equal(y, np.array(g["y"]))


@pytest.mark.parametrize("act_order,group", [(False, 32), (True, 32), (True, 64)])
def test_stored_format_reproduces_quantizer_weights(act_order, group):
    """Codes, g_idx, scales and zero points as the quantizer leaves them give
    back exactly its dequantized weights (rounded to float32, the precision
    the quantizer keeps them in)."""
    rng = np.random.default_rng(11 + group + int(act_order))
    X = rng.standard_normal((128, 400))
    X[rng.choice(128, 3, replace=False)] *= 15
    Wt = rng.standard_normal((24, 128)) * 0.02
    H = O.hessian([X])
    diag = O.hessian_diag([X])
    res = O.quantize_layer(Wt, H, diag, bits=4, group=group, block=group,
                           act_order=act_order, percdamp=0.01)
    if act_order:
        assert not np.array_equal(res.g_idx, np.arange(128) // group)
    What = W.dequantize_stored(res.q, res.g_idx, res.sweep.scale, res.sweep.zero)
    np.testing.assert_array_equal(What.astype(np.float32), res.what.astype(np.float32))


def test_product_bruteforce_loops():
    L = I.stored_int4_layer(5, 64, 32, True, seed=3)
    x = I.activations_f16(3, 64, seed=4)
    y = W.w4a16_product(x, L.codes, L.g_idx, L.scale, L.zero)
    xv = x.view(np.float16)
    for b in range(3):
        for r in range(5):
            acc = 0.0
            for c in range(64):
                g = int(L.g_idx[c])
                w = float(L.scale[r, g]) * (int(L.codes[r, c]) - int(L.zero[r, g]))
                acc += float(xv[b, c]) * w
            assert y[b, r] == pytest.approx(acc, rel=1e-12, abs=1e-15)


def test_product_invariant_under_column_permutation():
    """Reordering the columns of x, the codes and g_idx together changes
    nothing: a group is a set of columns, not a range."""
    L = I.stored_int4_layer(7, 96, 32, False, seed=5)
    x = I.activations_f16(2, 96, seed=6)
    p = np.random.default_rng(0).permutation(96)
    y0 = W.w4a16_product(x, L.codes, L.g_idx, L.scale, L.zero)
    y1 = W.w4a16_product(x[:, p], L.codes[:, p], L.g_idx[p], L.scale, L.zero)
    np.testing.assert_allclose(y1, y0, rtol=1e-12, atol=1e-14)


def test_group_of_zero_codes_at_zero_point_contributes_nothing():
    """A group whose codes all equal its zero point has w^ = 0 there, whatever
    its scale: changing that scale leaves y unchanged."""
    L = I.stored_int4_layer(4, 64, 32, True, seed=8)
    codes = L.codes.copy()
    cols = np.nonzero(L.g_idx == 1)[0]
    codes[:, cols] = L.zero[:, [1]]
    x = I.activations_f16(2, 64, seed=9)
    y0 = W.w4a16_product(x, codes, L.g_idx, L.scale, L.zero)
    s2 = L.scale.copy()
    s2[:, 1] *= 1000
    y1 = W.w4a16_product(x, codes, L.g_idx, s2, L.zero)
    np.testing.assert_array_equal(y0, y1)


def test_stored_layer_generator_structure():
    for act in (False, True):
        L = I.stored_int4_layer(16, 256, 64, act, seed=1)
        assert np.all(np.bincount(L.g_idx) == 64)
        assert L.codes.max() < 16 and L.zero.max() < 16 and np.all(L.scale > 0)
        assert np.array_equal(L.g_idx, np.arange(256) // 64) != act
