"""One linear layer through the four C-ABI calls, with torch as the allocator.

This module sequences the native calls and owns the device buffers; it
performs no arithmetic of the method itself ("GPTQ implementation with
tensor subclasses", section Background: collect the layer's inputs, update
its weight, use the updated weight for the layer's outputs).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import binding as B


@dataclass
class QuantizedLayer:
    q: torch.Tensor            # rows x cols uint8 codes, original column order
    g_idx: torch.Tensor        # cols int32
    W_hat: torch.Tensor        # rows x cols float32 dequantized weights
    perm: torch.Tensor         # cols int32, processing position -> column
    dead: torch.Tensor         # cols uint8
    scale: torch.Tensor | None = None   # affine: rows x groups float32
    zero: torch.Tensor | None = None    # affine: rows x groups uint8
    super_scale: torch.Tensor | None = None  # q4k: rows x cols/256 fp16 bits (int16)
    super_min: torch.Tensor | None = None
    sub_scale: torch.Tensor | None = None    # q4k: rows x cols/32 uint8
    sub_min: torch.Tensor | None = None


def fast_route(rows: int, cols: int, *, group: int, block: int, grid: str = "affine") -> str:
    """The faster of the two routes for a layer; both reach the same codes in
    exact arithmetic.

    The Hessian-factor route needs the affine grid, block 128, a group that
    divides 128 and cols a multiple of 128.  It saves the triangular inverse,
    about d^3/3 products, and costs a read of the uncompensated weights in
    the sweep, which grows with rows * d.  Measured on MI355X: 27.7 against
    30.1 ms per layer at 4096 x 11008, 27.5 against 27.3 ms at 28672 x 8192;
    the rule takes it where rows <= 3e-4 d^2."""
    ok = grid == "affine" and block == 128 and 128 % group == 0 and cols % 128 == 0
    return "hessian" if ok and rows <= 3e-4 * cols * cols else "inverse"


class GptqLayer:
    """Buffers and call order for quantizing one layer on the current device.

    ``route``: "inverse" (U, the Cholesky factor of the inverse Hessian),
    "hessian" (the Hessian's own Cholesky factor times U's diagonal blocks
    between 128-column blocks) or
    "auto" (fast_route)."""

    def __init__(self, rows: int, cols: int, *, bits: int, group: int, block: int,
                 act_order: bool, percdamp: float = 0.01, grid: str = "affine",
                 device: str = "cuda", search: bool = False, route: str = "inverse"):
        self.rows, self.cols = rows, cols
        self.grid = grid
        self.bits = bits
        self.group = 256 if grid == "q4k" else group
        if route == "auto":
            route = fast_route(rows, cols, group=self.group, block=block, grid=grid)
        self.route = route
        self.params = B.make_params(bits, self.group, block, act_order, percdamp, grid, search,
                                    route)
        dev = torch.device(device)
        self.device = dev
        self.H = torch.zeros((cols, cols), dtype=torch.float32, device=dev)
        self.hdiag = torch.zeros(cols, dtype=torch.float64, device=dev)
        self.U = torch.empty((cols, cols), dtype=torch.float32, device=dev)
        self.perm = torch.empty(cols, dtype=torch.int32, device=dev)
        self.dead = torch.empty(cols, dtype=torch.uint8, device=dev)
        nbytes = B.gptq_workspace_bytes(rows, cols, self.params)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def reset_hessian(self):
        self.H.zero_()
        self.hdiag.zero_()

    def add_batch(self, X: torch.Tensor, stream=None):
        """X: cols x tokens, bfloat16 or float32, on the device."""
        B.gptq_hessian_accumulate(self.H, self.hdiag, X, ws=self.ws, stream=stream)

    def prepare(self, stream=None):
        B.gptq_prepare_hinv(self.H, self.hdiag, self.params, self.U, self.perm, self.dead,
                            self.ws, stream=stream)

    def alloc_outputs(self) -> dict:
        r, c, dev = self.rows, self.cols, self.device
        out = dict(q=torch.empty((r, c), dtype=torch.uint8, device=dev),
                   g_idx=torch.empty(c, dtype=torch.int32, device=dev))
        if self.grid == "affine":
            ng = c // self.group
            out.update(scale=torch.empty((r, ng), dtype=torch.float32, device=dev),
                       zero=torch.empty((r, ng), dtype=torch.uint8, device=dev))
        else:
            out.update(q4k_super_scale=torch.empty((r, c // 256), dtype=torch.int16, device=dev),
                       q4k_super_min=torch.empty((r, c // 256), dtype=torch.int16, device=dev),
                       q4k_sub_scale=torch.empty((r, c // 32), dtype=torch.uint8, device=dev),
                       q4k_sub_min=torch.empty((r, c // 32), dtype=torch.uint8, device=dev))
        return out

    def quantize(self, W: torch.Tensor, out: dict | None = None, stream=None) -> QuantizedLayer:
        """W: rows x cols float32 on the device; overwritten with W^."""
        out = self.alloc_outputs() if out is None else out
        B.gptq_quantize_layer(W, self.U, self.perm, self.dead, self.params, ws=self.ws,
                              stream=stream, hdiag=self.hdiag, **out)
        return QuantizedLayer(q=out["q"], g_idx=out["g_idx"], W_hat=W, perm=self.perm,
                              dead=self.dead, scale=out.get("scale"), zero=out.get("zero"),
                              super_scale=out.get("q4k_super_scale"),
                              super_min=out.get("q4k_super_min"),
                              sub_scale=out.get("q4k_sub_scale"),
                              sub_min=out.get("q4k_sub_min"))

    def pack_codes(self, q: torch.Tensor, packed: torch.Tensor | None = None, stream=None):
        bits = 4 if self.grid == "q4k" else self.bits
        if packed is None:
            packed = torch.empty((self.rows, self.cols * bits // 32), dtype=torch.int32,
                                 device=self.device)
        B.gptq_pack(q, bits, packed, stream=stream)
        return packed

    def pack_zeros(self, zero: torch.Tensor, packed: torch.Tensor | None = None, stream=None):
        """All zero points of the layer as one stream (rows * groups codes)."""
        n = zero.numel()
        if packed is None:
            packed = torch.empty(((n * self.bits + 31) // 32,), dtype=torch.int32,
                                 device=self.device)
        B.gptq_pack(zero, self.bits, packed, rows=1, cols=n, stream=stream)
        return packed
