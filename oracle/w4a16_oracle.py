"""Float64 CPU oracle of the W4A16 product: running a stored 4-bit layer.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The product path (the HIP
library and its Python binding) never imports, links or calls it, and it
shares no code with that path.

Written from these pages (cited by title and section):

* "Hugging Face AutoGPTQ and Transformers Integration", section "Mixed
  Precision Scheme": the weights are stored as int4, the activations stay in
  float16, and the weights are turned back into real values on the fly
  inside the product.
* "GPTQ" (robocikowo.com), section "Hiperparametry" (a scale per group of
  weights) and section "Waskie gardla" (in inference the cost is reading
  memory; that motivates the kernel, not the arithmetic).

What is computed has a plain definition, so the oracle is that definition:

    w^[r][c] = scale[r][g] * (q[r][c] - zero[r][g]),   g = g_idx[c]
    y[b][r]  = sum_c  x[b][c] * w^[r][c]

with x the float16 activations widened exactly, everything else in float64.
Reading (the pages are silent on it): g_idx names the group of each original
column, so with activation order a group's columns are scattered over the
row; scale and zero are indexed by that group.
"""
from __future__ import annotations

import numpy as np


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """float16 bit patterns (uint16) -> float64, exactly."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def dequantize_stored(codes: np.ndarray, g_idx: np.ndarray, scale: np.ndarray,
                      zero: np.ndarray) -> np.ndarray:
    """Real weights of a stored layer, float64 (rows x cols).

    codes (rows, cols) integers, g_idx (cols,) group of each column,
    scale (rows, groups) float, zero (rows, groups) integers."""
    codes = np.asarray(codes, dtype=np.float64)
    g_idx = np.asarray(g_idx, dtype=np.int64)
    s = np.asarray(scale, dtype=np.float64)[:, g_idx]
    z = np.asarray(zero, dtype=np.float64)[:, g_idx]
    return s * (codes - z)


def w4a16_product(x_bits: np.ndarray, codes: np.ndarray, g_idx: np.ndarray,
                  scale: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """y = x W^T in float64 for float16 activations x (batch, cols) given as
    bit patterns.  A subset of W's rows gives that subset of y's columns."""
    x = f16_bits_to_f64(x_bits)
    What = dequantize_stored(codes, g_idx, scale, zero)
    return x @ What.T


def w4a16_abs_product_sum(x_bits: np.ndarray, codes: np.ndarray, g_idx: np.ndarray,
                          scale: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """sum_c |x[b][c] * w^[r][c]| (batch, rows): the scale of the rounding
    error any order of summation can make."""
    x = np.abs(f16_bits_to_f64(x_bits))
    What = np.abs(dequantize_stored(codes, g_idx, scale, zero))
    return x @ What.T
