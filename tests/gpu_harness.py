"""Drive one layer through the HIP path and through the oracle on the same
seeded inputs (test infrastructure)."""
from __future__ import annotations

import sys
from dataclasses import dataclass

import numpy as np

import oracle as O
from post_weight_quantization_layer_amd import inputs as I


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device_x(xs: np.ndarray, dev, pad_to: int = 8):
    """Storage-dtype chunk (uint16 bf16 bits or float32) -> device tensor with
    a row stride padded to a multiple of ``pad_to``; returns (tensor, n, ld)."""
    import torch
    d, n = xs.shape
    ld = (n + pad_to - 1) // pad_to * pad_to
    if xs.dtype == np.uint16:
        t = torch.zeros((d, ld), dtype=torch.bfloat16, device=dev)
        t[:, :n] = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        t = torch.zeros((d, ld), dtype=torch.float32, device=dev)
        t[:, :n] = torch.from_numpy(xs).to(dev)
    return t, n, ld


@dataclass
class GpuOut:
    H: np.ndarray
    hdiag: np.ndarray
    U: np.ndarray
    perm: np.ndarray
    dead: np.ndarray
    q: np.ndarray
    g_idx: np.ndarray
    W_hat: np.ndarray
    scale: np.ndarray | None = None
    zero: np.ndarray | None = None
    D: np.ndarray | None = None
    Dm: np.ndarray | None = None
    sc: np.ndarray | None = None
    mc: np.ndarray | None = None


def expected_factor(U: np.ndarray, H: np.ndarray, diag: np.ndarray, perm: np.ndarray,
                    percdamp: float, route: str) -> np.ndarray:
    """What gptq_prepare_hinv writes for a route, from the oracle: U itself
    (inverse route), or U inside the 128 x 128 diagonal blocks and, above
    each diagonal block B, R_{<B,B} U_BB with Hp = R R^T (Hessian route;
    R = T diag(R) from the oracle's unit factor T, diag(R) = 1 / diag(U))."""
    if route == "inverse":
        return U
    T = O.unit_upper_factor(O.damped_processing_hessian(H, diag, perm, percdamp))
    T /= np.diag(U)[None, :]          # R, in place
    d = U.shape[0]
    F = np.zeros_like(U)
    for b0 in range(0, d, 128):
        b1 = min(b0 + 128, d)
        F[b0:b1, b0:b1] = U[b0:b1, b0:b1]
        F[:b0, b0:b1] = T[:b0, b0:b1] @ U[b0:b1, b0:b1]
    return F


def gpu_layer(cfg: I.LayerConfig, W: np.ndarray, chunks, dev="cuda", keep_H=True,
              search=False, route="inverse") -> GpuOut:
    """chunks: iterable of storage-dtype X chunks (d x n_c)."""
    import torch
    from post_weight_quantization_layer_amd import binding as B
    from post_weight_quantization_layer_amd.layer import GptqLayer
    L = GptqLayer(W.shape[0], cfg.cols, bits=cfg.bits, group=cfg.group, block=cfg.block,
                  act_order=cfg.act_order, percdamp=cfg.percdamp, grid=cfg.grid, device=dev,
                  search=search, route=route)
    for xs in chunks:
        t, n, ld = to_device_x(xs, dev)
        B.gptq_hessian_accumulate(L.H, L.hdiag, t, n_tok=n, ld_x=ld, ws=L.ws)
        del t
    L.prepare()
    Wd = torch.from_numpy(np.ascontiguousarray(W, dtype=np.float32)).to(dev)
    res = L.quantize(Wd)
    torch.cuda.synchronize()
    out = GpuOut(H=L.H.cpu().numpy() if keep_H else None, hdiag=L.hdiag.cpu().numpy(),
                 U=L.U.cpu().numpy(), perm=L.perm.cpu().numpy().astype(np.int64),
                 dead=L.dead.cpu().numpy().astype(bool), q=res.q.cpu().numpy(),
                 g_idx=res.g_idx.cpu().numpy(), W_hat=res.W_hat.cpu().numpy())
    if cfg.grid == "affine":
        out.scale = res.scale.cpu().numpy()
        out.zero = res.zero.cpu().numpy()
    else:
        out.D = res.super_scale.cpu().numpy().view(np.float16)
        out.Dm = res.super_min.cpu().numpy().view(np.float16)
        out.sc = res.sub_scale.cpu().numpy()
        out.mc = res.sub_min.cpu().numpy()
    return out


def oracle_layer(cfg: I.LayerConfig, W: np.ndarray, chunks_f32, block=None, search=False):
    H = None
    diag = None
    for xc in chunks_f32:
        h = O.hessian([xc])
        dg = O.hessian_diag([xc])
        H = h if H is None else H + h
        diag = dg if diag is None else diag + dg
    res = O.quantize_layer(W, H, diag, bits=cfg.bits, group=cfg.group, block=block,
                           act_order=cfg.act_order, percdamp=cfg.percdamp, grid=cfg.grid,
                           search=search)
    return res, H, diag


def gpu_grid(g: GpuOut, grid: str) -> dict:
    """The GPU's grid outputs (processing order) in the form the tie-forced
    replay compares."""
    if grid == "affine":
        return {"scale": g.scale, "zero": g.zero}
    return {"D": g.D, "Dm": g.Dm, "sc": g.sc, "mc": g.mc}


def check_replay(cfg: I.LayerConfig, W: np.ndarray, o, g: GpuOut, diag=None, search=False,
                 max_frac: float = 1e-3, max_search_rows=None, tag: str = ""):
    """Tie-forced replay of the oracle's sweep against the GPU's decisions,
    asserted (see tests.parity.assert_replay); returns the report."""
    from tests.parity import assert_replay, replay_layer
    grid = gpu_grid(g, cfg.grid)
    rp = replay_layer(W, o, g.q, grid, grid_kind=cfg.grid, bits=cfg.bits, group=cfg.group,
                      diag=diag, search=search)
    log(f"[replay] {tag}: adopted {rp.forced} at ties ({rp.search_ties} search-tie "
        f"super-blocks), {len(rp.bad)} decisions off a tie")
    assert_replay(rp, g.q[:, o.perm], grid, cfg.grid, max_frac=max_frac,
                  max_search_rows=max_search_rows)
    return rp
