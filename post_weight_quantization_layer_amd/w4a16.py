"""A stored 4-bit layer run as y = x W^T through the W4A16 C-ABI calls, with
torch as the allocator ("Hugging Face AutoGPTQ and Transformers
Integration", section Mixed Precision Scheme: int4 weights, fp16
activations, dequantization inside the product kernel).

This module only allocates buffers and sequences the native calls."""
from __future__ import annotations

import torch

from . import binding as B


def pack_zero_points(zero: torch.Tensor) -> torch.Tensor:
    """rows x groups uint8 zero points -> their 4-bit stream (gptq_pack of the
    matrix as one row), padded to whole 32-bit words."""
    flat = zero.reshape(1, -1)
    n = flat.shape[1]
    pad = (-n) % 8
    if pad:
        flat = torch.cat([flat, torch.zeros((1, pad), dtype=flat.dtype, device=flat.device)], 1)
    out = torch.empty((1, (n + pad) // 8), dtype=torch.int32, device=zero.device)
    B.gptq_pack(flat, 4, out)
    return out


class W4A16Linear:
    """Prepared layer plus the scratch of its products, on one device."""

    def __init__(self, packed: torch.Tensor, g_idx: torch.Tensor, scale: torch.Tensor,
                 zero_packed: torch.Tensor, rows: int, cols: int, group: int, stream=None):
        dev = packed.device
        nbytes = B.gptq_w4a16_layer_bytes(rows, cols, group)
        self.mem = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.layer = B.gptq_w4a16_prepare(packed, g_idx, scale, zero_packed, rows, cols, group,
                                          self.mem, stream)
        self.rows, self.cols = rows, cols
        self.device = dev
        self.ws = None

    @classmethod
    def from_codes(cls, codes: torch.Tensor, g_idx: torch.Tensor, scale: torch.Tensor,
                   zero: torch.Tensor, group: int, stream=None) -> "W4A16Linear":
        """From unpacked codes (rows x cols uint8) and zero points (rows x groups
        uint8), packing both on the device first."""
        rows, cols = codes.shape
        packed = torch.empty((rows, cols // 8), dtype=torch.int32, device=codes.device)
        B.gptq_pack(codes, 4, packed, stream=stream)
        return cls(packed, g_idx, scale, pack_zero_points(zero), rows, cols, group, stream)

    def workspace(self, batch: int) -> torch.Tensor | None:
        n = B.gptq_w4a16_workspace_bytes(self.layer, batch)
        if n == 0:
            return None
        if self.ws is None or self.ws.numel() < n:
            self.ws = torch.empty(n, dtype=torch.uint8, device=self.device)
        return self.ws

    def __call__(self, x: torch.Tensor, y: torch.Tensor | None = None, stream=None):
        """x: batch x cols float16 -> y: batch x rows float16."""
        if y is None:
            y = torch.empty((x.shape[0], self.rows), dtype=torch.float16, device=x.device)
        B.gptq_w4a16_gemm(self.layer, x, y, self.workspace(x.shape[0]), stream=stream)
        return y
