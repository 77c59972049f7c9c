"""Float64 CPU oracle of sequential multi-linear calibration.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The product path (the HIP
library and its Python binding) never imports, links or calls it, and it
shares no code with that path.

Written from "GPTQ implementation with tensor subclasses", section
"Background": for each linear, (1) collect the activations reaching it,
(2) run GPTQ to update its weight, (3) produce the linear's outputs with the
updated weight, (4) go on to the next linear with those outputs -- once
through the inputs, instead of re-running the model for every linear.

The block is a gated MLP, the shape of the workloads' down_proj inputs:
gate and up read the same activations X (so they share one Hessian), the
down linear reads A = silu(W^_gate X) * (W^_up X).  Activations are stored in
bf16 (the storage type of the workloads' calibration inputs); each stored
value is its exact (float64) value rounded to float32 and then to bf16,
nearest-even, the path the GPU's float32 sums take.
"""
from __future__ import annotations

import numpy as np

from . import gptq_oracle as G


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> bf16 (round to nearest, ties to even), as float64."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16))
    return (r << np.uint64(16)).astype(np.uint32).view(np.float32).astype(np.float64)


def linear_forward(What: np.ndarray, X: np.ndarray) -> np.ndarray:
    """Outputs of the updated layer: bf16(W^ X), W^ rows x cols, X cols x n."""
    return round_bf16(np.asarray(What, np.float64) @ np.asarray(X, np.float64))


def silu_mul(Gt: np.ndarray, Ut: np.ndarray) -> np.ndarray:
    """bf16(silu(G) * U), silu(g) = g / (1 + e^-g)."""
    g = np.asarray(Gt, np.float64)
    return round_bf16(g / (1.0 + np.exp(-g)) * np.asarray(Ut, np.float64))


def calibrate_gated_mlp(W_gate, W_up, W_down, X_chunks, *, bits: int, group: int,
                        block: int | None, act_order: bool, percdamp: float,
                        grid: str = "affine", search: bool = False) -> dict:
    """Quantize gate, up, then down, each from the activations that reach it
    with the earlier linears already quantized.  X_chunks: token chunks of the
    block input (d x n_c, bf16 values as floats)."""
    kw = dict(bits=bits, group=group, block=block, act_order=act_order,
              percdamp=percdamp, grid=grid, search=search)
    H1 = G.hessian(X_chunks)
    d1 = G.hessian_diag(X_chunks)
    gate = G.quantize_layer(W_gate, H1, d1, **kw)
    up = G.quantize_layer(W_up, H1, d1, **kw)
    A_chunks = [silu_mul(linear_forward(gate.what, X), linear_forward(up.what, X))
                for X in X_chunks]
    H2 = G.hessian(A_chunks)
    d2 = G.hessian_diag(A_chunks)
    down = G.quantize_layer(W_down, H2, d2, **kw)
    return dict(gate=gate, up=up, down=down, H1=H1, d1=d1, H2=H2, d2=d2, A=A_chunks)
