"""Edge cases of the HIP path: pack, not-positive-definite detection, dead
columns, determinism, empty and degenerate inputs."""
import numpy as np
import pytest

import oracle as O
from post_weight_quantization_layer_amd import inputs as I
from tests.gpu_harness import gpu_layer, log, oracle_layer
from tests.parity import assert_codes, classify_codes, rel_fro

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bits,rows,cols", [(2, 3, 48), (3, 5, 96), (4, 7, 40), (5, 2, 32),
                                            (6, 3, 16), (7, 4, 64), (8, 9, 12), (3, 1, 11008)])
def test_pack_matches_oracle(bits, rows, cols):
    import torch
    from post_weight_quantization_layer_amd import binding as B
    rng = np.random.Generator(np.random.Philox(key=bits * 1000 + cols))
    codes = rng.integers(0, 2 ** bits, size=(rows, cols)).astype(np.uint8)
    dev = torch.device("cuda")
    c = torch.from_numpy(codes).to(dev)
    out = torch.empty((rows, cols * bits // 32), dtype=torch.int32, device=dev)
    B.gptq_pack(c, bits, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got, O.pack(codes, bits))


def test_not_spd_is_reported():
    import torch
    from post_weight_quantization_layer_amd import binding as B
    d = 300
    dev = torch.device("cuda")
    H = torch.zeros((d, d), dtype=torch.float32, device=dev)
    idx = torch.arange(d, device=dev)
    H[idx, idx] = 1.0
    H[17, 17] = -5.0                        # indefinite, large enough to beat damping
    hdiag = torch.ones(d, dtype=torch.float64, device=dev)
    p = B.make_params(4, 100, 100, False, 0.0)
    U = torch.empty_like(H)
    perm = torch.empty(d, dtype=torch.int32, device=dev)
    dead = torch.empty(d, dtype=torch.uint8, device=dev)
    ws = torch.empty(B.gptq_workspace_bytes(8, d, p), dtype=torch.uint8, device=dev)
    with pytest.raises(B.NotSPDError):
        B.gptq_prepare_hinv(H, hdiag, p, U, perm, dead, ws)
    with pytest.raises(O.NotSPD):
        O.inverse_cholesky_upper(np.diag(np.where(np.arange(d) == 17, -5.0, 1.0)))
    # the same buffers work again afterwards
    H[17, 17] = 2.0
    B.gptq_prepare_hinv(H, hdiag, p, U, perm, dead, ws)
    torch.cuda.synchronize()
    u = U.cpu().numpy()
    expect = np.ones(d)
    expect[17] = 1 / np.sqrt(2.0)
    np.testing.assert_allclose(np.diag(u), expect, rtol=1e-6)
    assert np.all(u - np.diag(np.diag(u)) == 0)


def test_dead_column_and_diagonal_hessian():
    """A zero feature row: dead column, zero weights, processed last.  With
    disjoint feature supports H is diagonal and GPTQ equals round-to-nearest."""
    cfg = I.CONFIGS["q_proj_4096x4096_int4_g128"].with_(rows=70, cols=256, tokens=1024,
                                                       act_order=True)
    W = I.weight(cfg)
    X = np.zeros((256, 1024), np.float32)
    for i in range(256):
        if i != 37:
            X[i, 4 * i: 4 * i + 4] = 1.0 + (i % 7) / 8.0
    store = [I.bf16_bits(X)]
    g = gpu_layer(cfg, W, store)
    o, H, diag = oracle_layer(cfg, W.astype(np.float64), [X])
    assert g.dead[37] and g.dead.sum() == 1
    assert np.all(g.W_hat[:, 37] == 0)
    np.testing.assert_array_equal(g.perm, o.perm)
    np.testing.assert_array_equal(g.q, o.q)
    np.testing.assert_array_equal(g.W_hat, o.what)
    assert np.all(np.triu(g.U, 1) == 0)


def test_bitwise_deterministic():
    cfg = I.CONFIGS["down_proj_4096x11008_int4_g128_actorder"].with_(rows=96, cols=640,
                                                                    tokens=1500)
    W = I.weight(cfg)
    store = [I.x_chunk_storage(cfg, 0, 1500)]
    a = gpu_layer(cfg, W, store)
    b = gpu_layer(cfg, W, store)
    for f in ("H", "hdiag", "U", "q", "W_hat", "scale", "zero"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f), err_msg=f)


@pytest.mark.parametrize("block,group", [(32, 128), (64, 64), (128, 32), (16, 256)])
def test_block_group_combinations(block, group):
    """Blocks smaller than, equal to and larger than the group give the
    oracle's result (the method's result does not depend on B)."""
    cfg = I.CONFIGS["up_proj_28672x8192_int3_g128_actorder"].with_(
        rows=64, cols=512, tokens=1200, block=block, group=group)
    W = I.weight(cfg)
    store = [I.x_chunk_storage(cfg, 0, 1200)]
    f32 = [I.bf16_to_f32(store[0])]
    g = gpu_layer(cfg, W, store)
    o, H, diag = oracle_layer(cfg, W.astype(np.float64), f32)
    rep = classify_codes(g.q[:, o.perm], o.sweep, "affine", group)
    log(f"[edges] B={block} g={group}: {rep.mismatches} code mismatches")
    assert_codes(rep)
    assert rel_fro(g.U, o.U) <= 1e-4


@pytest.mark.parametrize("act", [False, True])
def test_odd_width_small_groups(act):
    """An odd number of columns (scalar W access path), groups of 5, blocks of 5."""
    cfg = I.CONFIGS["q_proj_4096x4096_int4_g128"].with_(rows=33, cols=125, tokens=700, group=5,
                                                       block=5, act_order=act)
    W = I.weight(cfg)
    store = [I.x_chunk_storage(cfg, 0, 700)]
    g = gpu_layer(cfg, W, store)
    o, H, diag = oracle_layer(cfg, W.astype(np.float64), [I.bf16_to_f32(store[0])])
    rep = classify_codes(g.q[:, o.perm], o.sweep, "affine", 5)
    assert_codes(rep)
    assert rel_fro(g.U, o.U) <= 1e-4
    e_gpu = O.reconstruction_error(W, g.W_hat, H)
    e_or = O.reconstruction_error(W, o.what, H)
    assert abs(e_gpu - e_or) <= 0.01 * e_or


@pytest.mark.parametrize("bits,group,block", [(2, 64, 64), (8, 128, 128), (3, 512, 128),
                                              (5, 32, 128)])
def test_bit_widths_and_per_channel(bits, group, block):
    """Affine grids of 2, 3, 5 and 8 bits; group = cols is one scale per row
    (per-channel)."""
    cfg = I.CONFIGS["down_proj_4096x11008_int4_g128_actorder"].with_(
        rows=48, cols=512, tokens=1500, bits=bits, group=group, block=block)
    W = I.weight(cfg)
    store = [I.x_chunk_storage(cfg, 0, 1500)]
    g = gpu_layer(cfg, W, store)
    o, H, diag = oracle_layer(cfg, W.astype(np.float64), [I.bf16_to_f32(store[0])])
    rep = classify_codes(g.q[:, o.perm], o.sweep, "affine", group)
    log(f"[edges] bits={bits} g={group} B={block}: {rep.mismatches} code mismatches")
    assert_codes(rep)
    assert int(g.q.max()) <= 2 ** bits - 1
    e_gpu = O.reconstruction_error(W, g.W_hat, H)
    e_or = O.reconstruction_error(W, o.what, H)
    assert abs(e_gpu - e_or) <= 0.01 * e_or


@pytest.mark.parametrize("bits,act", [(2, False), (3, True), (5, False), (6, True)])
def test_kquant_code_widths(bits, act):
    """Two-level grid with 2-, 3-, 5- and 6-bit codes (sub-block scale/min
    codes 4, 6, 6 and 8 bits wide): codes, super- and sub-block codes equal
    the oracle's away from tie cascades, dequantized weights on the GPU's own
    grid, reconstruction error within 1 %."""
    from tests.parity import cascade_mask
    cfg = I.CONFIGS["q4k_14336x4096"].with_(rows=64, cols=768, tokens=1500, bits=bits,
                                              act_order=act)
    W = I.weight(cfg)
    store = [I.x_chunk_storage(cfg, 0, 1500)]
    g = gpu_layer(cfg, W, store)
    o, H, diag = oracle_layer(cfg, W.astype(np.float64), [I.bf16_to_f32(store[0])])
    perm = o.perm
    qg_p = g.q[:, perm]
    rep = classify_codes(qg_p, o.sweep, "q4k", 256)
    log(f"[edges] k-quant bits={bits}: {rep.mismatches} code mismatches")
    assert_codes(rep)
    kmax = 2 ** O.kquant_sub_bits(bits) - 1
    assert int(g.q.max()) <= 2 ** bits - 1
    assert int(g.sc.max()) <= kmax and int(g.mc.max()) <= kmax
    casc = cascade_mask(qg_p, o.sweep, O.Q4K_SUPER)
    casc_sub = np.repeat(casc, 8, axis=1)
    np.testing.assert_array_equal(g.D[~casc], o.sweep.D[~casc])
    np.testing.assert_array_equal(g.Dm[~casc], o.sweep.Dm[~casc])
    np.testing.assert_array_equal(g.sc[~casc_sub], o.sweep.sc[~casc_sub])
    np.testing.assert_array_equal(g.mc[~casc_sub], o.sweep.mc[~casc_sub])
    S = np.repeat(np.repeat(g.D.astype(np.float32), 8, axis=1) * g.sc, 32, axis=1)
    M = np.repeat(np.repeat(g.Dm.astype(np.float32), 8, axis=1) * g.mc, 32, axis=1)
    np.testing.assert_array_equal(g.W_hat[:, perm], S * qg_p.astype(np.float32) - M)
    e_gpu = O.reconstruction_error(W, g.W_hat, H)
    e_or = O.reconstruction_error(W, o.what, H)
    assert abs(e_gpu - e_or) <= 0.01 * e_or


@pytest.mark.parametrize("bits,group,block,act", [(4, 128, 128, True), (3, 128, 64, True),
                                                  (4, 32, 128, False), (4, 256, 128, True)])
def test_weighted_grid_search(bits, group, block, act):
    """Importance-weighted grid choice: codes, scales and zero points as the
    oracle's away from tie cascades (search ties included), the GPU's weights
    on its own grid, reconstruction error within 1 % of the oracle's and
    below the min-max grid's."""
    from tests.parity import cascade_mask, near_half
    cfg = I.CONFIGS["down_proj_4096x11008_int4_g128_actorder"].with_(
        rows=96, cols=768, tokens=1800, bits=bits, group=group, block=block, act_order=act,
        x_kind="gauss", outlier_frac=0.01, outlier_scale=20.0)
    W = I.weight(cfg)
    store = [I.x_chunk_storage(cfg, 0, 1800)]
    f32 = [I.bf16_to_f32(store[0])]
    g = gpu_layer(cfg, W, store, search=True)
    o, H, diag = oracle_layer(cfg, W.astype(np.float64), f32, search=True)
    perm = o.perm
    qg_p = g.q[:, perm]
    rep = classify_codes(qg_p, o.sweep, "affine", group)
    casc = cascade_mask(qg_p, o.sweep, group)
    # a tie's cascade can move a later group's choice to another candidate,
    # so the share of differing codes is counted outside the cascades
    outside = (qg_p != o.sweep.q) & ~np.repeat(casc, group, axis=1)
    log(f"[edges] search bits={bits} g={group}: {rep.mismatches} code mismatches in "
        f"{rep.rows_with_mismatch} rows, {int(outside.sum())} outside tie cascades, "
        f"{int((o.sweep.sgap < 1e-9).sum())} search ties")
    assert not rep.unclassified, f"mismatches not at a tie: {rep.unclassified[:5]}"
    assert outside.sum() == 0
    assert rep.rows_with_mismatch <= max(1, qg_p.shape[0] // 50)
    rel = np.abs(g.scale - o.sweep.scale) / o.sweep.scale
    assert rel[~casc].max() <= 1e-3
    zdiff = (g.zero.astype(np.int64) != o.sweep.zero.astype(np.int64)) & ~casc
    assert np.all(near_half(o.sweep.zratio[zdiff], 1e-3))
    s = np.repeat(g.scale, group, axis=1)
    z = np.repeat(g.zero.astype(np.float32), group, axis=1)
    np.testing.assert_array_equal(g.W_hat[:, perm], s * (qg_p.astype(np.float32) - z))
    e_gpu = O.reconstruction_error(W, g.W_hat, H)
    e_or = O.reconstruction_error(W, o.what, H)
    assert abs(e_gpu - e_or) <= 0.01 * e_or
    base = gpu_layer(cfg, W, store)
    e_base = O.reconstruction_error(W, base.W_hat, H)
    log(f"[edges] search bits={bits} g={group}: E_search / E_minmax = {e_gpu / e_base:.3f}")
    assert e_gpu < e_base


@pytest.mark.parametrize("bits,act", [(4, True), (3, False)])
def test_weighted_search_two_level_grid(bits, act):
    """Importance-weighted (scale, min) of each sub-block of the two-level grid:
    codes and grid codes as the oracle's outside tie cascades (search ties
    included), weights on the GPU's own grid, reconstruction error within 1 %
    of the oracle's and below the min-max grids'."""
    from tests.parity import cascade_mask
    cfg = I.CONFIGS["q4k_14336x4096"].with_(rows=80, cols=768, tokens=1600, bits=bits,
                                              act_order=act, outlier_frac=0.01,
                                              outlier_scale=20.0)
    W = I.weight(cfg)
    store = [I.x_chunk_storage(cfg, 0, 1600)]
    f32 = [I.bf16_to_f32(store[0])]
    g = gpu_layer(cfg, W, store, search=True)
    o, H, diag = oracle_layer(cfg, W.astype(np.float64), f32, search=True)
    perm = o.perm
    qg_p = g.q[:, perm]
    rep = classify_codes(qg_p, o.sweep, "q4k", 256)
    casc = cascade_mask(qg_p, o.sweep, O.Q4K_SUPER)
    outside = (qg_p != o.sweep.q) & ~np.repeat(casc, O.Q4K_SUPER, axis=1)
    log(f"[edges] two-level search bits={bits}: {rep.mismatches} code mismatches in "
        f"{rep.rows_with_mismatch} rows, {int(outside.sum())} outside tie cascades")
    assert not rep.unclassified, f"mismatches not at a tie: {rep.unclassified[:5]}"
    assert outside.sum() == 0
    assert rep.rows_with_mismatch <= max(1, qg_p.shape[0] // 50)
    # super-scales within one fp16 step: the searched sub-block scales carry
    # the last-bit differences of the fp32 trailing updates, which can move
    # max_b s_b / kmax across an fp16 rounding boundary
    for a_, b_ in ((g.D, o.sweep.D), (g.Dm, o.sweep.Dm)):
        ga, ob = a_[~casc].astype(np.float32), b_[~casc].astype(np.float32)
        assert np.all(np.abs(ga - ob) <= 2.0 ** -10 * np.abs(ob))
    same = np.repeat((g.D == o.sweep.D) & (g.Dm == o.sweep.Dm) & ~casc, 8, axis=1)
    np.testing.assert_array_equal(g.sc[same], o.sweep.sc[same])
    np.testing.assert_array_equal(g.mc[same], o.sweep.mc[same])
    S = np.repeat(np.repeat(g.D.astype(np.float32), 8, axis=1) * g.sc, 32, axis=1)
    M = np.repeat(np.repeat(g.Dm.astype(np.float32), 8, axis=1) * g.mc, 32, axis=1)
    np.testing.assert_array_equal(g.W_hat[:, perm], S * qg_p.astype(np.float32) - M)
    e_gpu = O.reconstruction_error(W, g.W_hat, H)
    e_or = O.reconstruction_error(W, o.what, H)
    assert abs(e_gpu - e_or) <= 0.01 * e_or
    base = gpu_layer(cfg, W, store)
    assert e_gpu < O.reconstruction_error(W, base.W_hat, H)
