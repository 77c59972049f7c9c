"""HIP path at the workloads' full sizes, in the launch configuration the
benchmark times (32768-token chunks), against the oracle.

For every workload -- q_proj 4096x4096, down_proj 4096x11008 with 131072
tokens (the headline layer), up_proj 28672x8192 (int3), Q4K 14336x4096 --
the oracle builds the full float64 H (streamed over 8192-token chunks as the
GPU's inputs are generated) and the full U by the literal route.  The GPU
runs the route the benchmark takes for the layer (the Hessian-factor route
where it applies) and must match: H, and the route's factor (U, or U's
diagonal 128-blocks and the Hessian's unit factor above them), within 1e-4
relative (Frobenius), the activation energy
and the processing order exactly.  128 sampled rows of W are then swept by the
plain, unblocked oracle (rows are independent given U) and compared code by
code through the tie-forced replay, grid by grid, and by reconstruction error
(within 1 %, and below round-to-nearest on the same grid).  The share of
sampled codes that differ from the plain oracle's is logged and held below
MAX_RAW_FRAC; the replay requires every one of them to come from a tie.
"""
import numpy as np
import pytest

import oracle as O
from post_weight_quantization_layer_amd import inputs as I
from tests.gpu_harness import expected_factor, log
from tests.parity import assert_replay, classify_codes, rel_fro, replay_layer

pytestmark = pytest.mark.gpu

CHUNK = 32768       # tokens per accumulate call (as in the benchmark)
GEN = 8192          # tokens per host generation step
NSAMPLE_ROWS = 128
NRTN_ROWS = 32       # of those, rows also rounded to nearest (error comparison)
# Share of sampled codes that may differ from the plain oracle's.  Every
# difference must come from a tie (the replay below holds that strictly);
# a tie's cascade then carries on the order of 1-3 % of the rest of its row,
# so at 4096-11008 columns about one row in thirty differs in a few hundred
# codes and the differing share is near 1e-3 for the whole layer -- too near
# for a fixed sample to hold it below 1e-3 every time.
MAX_RAW_FRAC = 3e-3


def _run_gpu_stream(cfg, on_chunk=None, keep_x=False):
    """Generate X chunk by chunk, feed the GPU in CHUNK-token calls and hand
    every generated float32 chunk (d x GEN) to on_chunk.  Returns the layer
    object after prepare(), and X on the device when keep_x."""
    import torch
    from post_weight_quantization_layer_amd import binding as B
    from post_weight_quantization_layer_amd.layer import GptqLayer
    L = GptqLayer(cfg.rows, cfg.cols, bits=cfg.bits, group=cfg.group, block=cfg.block,
                  act_order=cfg.act_order, percdamp=cfg.percdamp, grid=cfg.grid, device="cuda",
                  route="auto")
    dev = torch.device("cuda")
    xall = torch.empty((cfg.cols, cfg.tokens if keep_x else CHUNK), dtype=torch.bfloat16,
                       device=dev)
    for c0 in range(0, cfg.tokens, CHUNK):
        n = min(CHUNK, cfg.tokens - c0)
        base = c0 if keep_x else 0
        for g0 in range(0, n, GEN):
            m = min(GEN, n - g0)
            xb = I.x_chunk_storage(cfg, c0 + g0, m)
            xall[:, base + g0:base + g0 + m].copy_(
                torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16))
            if on_chunk is not None:
                on_chunk(I.bf16_to_f32(xb))
        B.gptq_hessian_accumulate(L.H, L.hdiag, xall[:, base:base + n], n_tok=n,
                                  ld_x=xall.stride(0), ws=L.ws)
        log(f"[fullsize] {cfg.name}: accumulated {c0 + n}/{cfg.tokens} tokens")
    L.prepare()
    torch.cuda.synchronize()
    if keep_x:
        return L, xall
    del xall
    return L


def _quantize_gpu(cfg, L, W):
    import torch
    Wd = torch.from_numpy(W).cuda()
    res = L.quantize(Wd)
    torch.cuda.synchronize()
    return res


def _sample_rows(cfg):
    rng = np.random.default_rng(cfg.seed)
    return np.sort(rng.choice(cfg.rows, NSAMPLE_ROWS, replace=False))


FULL = ["q_proj_4096x4096_int4_g128",
        "down_proj_4096x11008_int4_g128_actorder",
        "up_proj_28672x8192_int3_g128_actorder",
        "q4k_14336x4096"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_with_full_oracle(name):
    cfg = I.CONFIGS[name]
    log(f"[fullsize] {name}: rows={cfg.rows} cols={cfg.cols} tokens={cfg.tokens}")
    G = np.zeros((cfg.cols, cfg.cols))
    energy = np.zeros(cfg.cols)

    def acc(xf):
        x = xf.astype(np.float64)
        G[...] += x @ x.T
        energy[...] += np.einsum("it,it->i", x, x)

    L = _run_gpu_stream(cfg, acc)
    H = 2.0 * G
    del G
    diag = 2.0 * energy
    # H and its activation energy
    Hg = L.H.cpu().numpy()
    iu = np.triu_indices(cfg.cols)
    errH = rel_fro(Hg[iu], H[iu])
    del Hg, iu
    log(f"[fullsize] {name}: H rel err {errH:.2e}")
    assert errH <= 1e-4
    assert rel_fro(L.hdiag.cpu().numpy(), diag) <= 1e-12
    # processing order and U
    perm = O.act_order_perm(diag) if cfg.act_order else np.arange(cfg.cols)
    np.testing.assert_array_equal(L.perm.cpu().numpy(), perm)
    Hp = O.damped_processing_hessian(H, diag, perm, cfg.percdamp)
    U = O.inverse_cholesky_upper(Hp)
    del Hp
    # the factor of the route the benchmark takes for this layer
    F = expected_factor(U, H, diag, perm, cfg.percdamp, L.route)
    errU = rel_fro(L.U.cpu().numpy(), F)
    del F
    log(f"[fullsize] {name}: {L.route} factor rel err {errU:.2e}")
    assert errU <= 1e-4
    # sweep: full GPU layer, oracle on sampled rows (rows are independent given U)
    W = I.weight(cfg)
    res = _quantize_gpu(cfg, L, W)
    rows = _sample_rows(cfg)
    Ws = W[rows].astype(np.float64)
    dead = O.dead_columns(diag)
    o = O.LayerResult(perm=perm, dead=dead, U=U, sweep=None, q=None, what=None, g_idx=None)
    Wp = Ws.copy()
    Wp[:, dead] = 0.0
    spec = O.GridSpec(cfg.grid, cfg.bits, O.Q4K_SUPER if cfg.grid == "q4k" else cfg.group)
    sw = O.gptq_sweep(Wp[:, perm], U, spec)
    what = np.empty_like(sw.what)
    what[:, perm] = sw.what
    q_gpu = res.q.cpu().numpy()[rows]
    rep = classify_codes(q_gpu[:, perm], sw, cfg.grid, cfg.group)
    log(f"[fullsize] {name}: codes {rep.mismatches}/{rep.n} differ in {rep.rows_with_mismatch} "
        f"rows ({rep.frac:.2e})")
    assert rep.frac <= MAX_RAW_FRAC
    if cfg.grid == "affine":
        grid = {"scale": res.scale.cpu().numpy()[rows], "zero": res.zero.cpu().numpy()[rows]}
    else:
        grid = {"D": res.super_scale.cpu().numpy()[rows].view(np.float16),
                "Dm": res.super_min.cpu().numpy()[rows].view(np.float16),
                "sc": res.sub_scale.cpu().numpy()[rows], "mc": res.sub_min.cpu().numpy()[rows]}
    rp = replay_layer(Ws, o, q_gpu, grid, grid_kind=cfg.grid, bits=cfg.bits, group=cfg.group)
    log(f"[fullsize] {name}: replay adopted {rp.forced} at ties, {len(rp.bad)} off a tie")
    assert_replay(rp, q_gpu[:, perm], grid, cfg.grid)
    w_hat = res.W_hat.cpu().numpy()[rows]
    e_gpu = O.reconstruction_error(Ws, w_hat, H)
    e_or = O.reconstruction_error(Ws, what, H)
    k = NRTN_ROWS
    r = O.rtn(Wp[:k, perm], spec)
    what_rtn = np.empty_like(r.what)
    what_rtn[:, perm] = r.what
    e_rtn = O.reconstruction_error(Ws[:k], what_rtn, H)
    e_gpu_k = O.reconstruction_error(Ws[:k], w_hat[:k], H)
    log(f"[fullsize] {name}: E_gpu/E_oracle = {e_gpu / e_or:.6f}, E_gptq/E_rtn = "
        f"{e_gpu_k / e_rtn:.4f} (first {k} rows)")
    assert abs(e_gpu - e_or) <= 0.01 * e_or
    assert e_gpu_k < e_rtn
    # the GPU's weights lie on its own grid (whole layer)
    perm_g = perm
    q_all = res.q.cpu().numpy()
    g_idx = res.g_idx.cpu().numpy()
    gsz = O.Q4K_SUB if cfg.grid == "q4k" else cfg.group
    np.testing.assert_array_equal(g_idx[perm_g], np.arange(cfg.cols) // gsz)
    if cfg.grid == "affine":
        s = res.scale.cpu().numpy()
        z = res.zero.cpu().numpy().astype(np.float32)
        assert int(q_all.max()) <= 2 ** cfg.bits - 1 and int(z.max()) <= 2 ** cfg.bits - 1
        np.testing.assert_array_equal(res.W_hat.cpu().numpy(),
                                      s[:, g_idx] * (q_all.astype(np.float32) - z[:, g_idx]))
