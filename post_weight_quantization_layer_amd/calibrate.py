"""Sequential calibration of a gated MLP block through the C ABI, torch as
the allocator ("GPTQ implementation with tensor subclasses", section
Background: for each linear, collect the activations reaching it, update
its weight with GPTQ, produce its outputs with the updated weight, and go on
to the next linear -- one pass over the inputs).

Gate and up read the same activations, so they share one Hessian and one
inverse factor (one accumulation and one gptq_prepare_hinv for two
quantizations).  Their outputs, made with the updated weights
(gptq_linear_forward), give silu(gate) * up (gptq_silu_mul), chunk by chunk;
the down linear's Hessian accumulates over those chunks.  This module only
allocates buffers and sequences the native calls.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import binding as B
from .layer import GptqLayer, QuantizedLayer


@dataclass
class GatedMLPResult:
    gate: QuantizedLayer
    up: QuantizedLayer
    down: QuantizedLayer
    activations: list        # down's input chunks, d_ff x n_c bf16 (padded row stride)


def _bf16_buffer(rows: int, n: int, device) -> torch.Tensor:
    ld = (n + 7) // 8 * 8     # row stride a multiple of 8 (Hessian accumulation)
    return torch.zeros((rows, ld), dtype=torch.bfloat16, device=device)


class GatedMLPCalibrator:
    """Buffers for one gated MLP block (d -> d_ff -> d) on one device."""

    def __init__(self, d: int, d_ff: int, *, bits: int, group: int, block: int,
                 act_order: bool, percdamp: float = 0.01, grid: str = "affine",
                 search: bool = False, device="cuda"):
        kw = dict(bits=bits, group=group, block=block, act_order=act_order,
                  percdamp=percdamp, grid=grid, device=device, search=search)
        self.d, self.d_ff = d, d_ff
        self.device = torch.device(device)
        self.gate_up = GptqLayer(d_ff, d, **kw)    # one Hessian for gate and up
        self.down = GptqLayer(d, d_ff, **kw)

    def run(self, W_gate: torch.Tensor, W_up: torch.Tensor, W_down: torch.Tensor,
            x_chunks, stream=None) -> GatedMLPResult:
        """W_*: float32 device tensors, overwritten with their quantized values.
        x_chunks: block inputs, each d x n_c bf16 on the device."""
        gu, dn = self.gate_up, self.down
        gu.reset_hessian()
        dn.reset_hessian()
        for X in x_chunks:                            # 1. activations reaching gate/up
            B.gptq_hessian_accumulate(gu.H, gu.hdiag, X, n_tok=X.shape[1],
                                      ld_x=X.stride(0), ws=gu.ws, stream=stream)
        gu.prepare(stream=stream)                     # 2. update gate and up
        q_gate = gu.quantize(W_gate, stream=stream)
        q_up = gu.quantize(W_up, stream=stream)
        acts = []
        nmax = max(X.shape[1] for X in x_chunks) if x_chunks else 0
        ws = torch.empty(max(B.gptq_linear_forward_ws_bytes(self.d_ff, self.d, nmax), 256),
                         dtype=torch.uint8, device=self.device)
        for X in x_chunks:                            # 3. outputs with the updated weights
            n = X.shape[1]
            G = _bf16_buffer(self.d_ff, n, self.device)
            Uo = _bf16_buffer(self.d_ff, n, self.device)
            B.gptq_linear_forward(W_gate, X, G, ws, n_tok=n, stream=stream)
            B.gptq_linear_forward(W_up, X, Uo, ws, n_tok=n, stream=stream)
            A = _bf16_buffer(self.d_ff, n, self.device)
            B.gptq_silu_mul(G, Uo, A, n_tok=n, stream=stream)
            B.gptq_hessian_accumulate(dn.H, dn.hdiag, A, n_tok=n, ld_x=A.stride(0),
                                      ws=dn.ws, stream=stream)  # 4. activations reaching down
            acts.append(A[:, :n])
        dn.prepare(stream=stream)
        q_down = dn.quantize(W_down, stream=stream)
        return GatedMLPResult(gate=q_gate, up=q_up, down=q_down, activations=acts)
