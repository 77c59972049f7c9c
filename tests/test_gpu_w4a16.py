"""W4A16 product on the GPU (through the C ABI) against the float64 oracle.

Bar: every output within the bound the arithmetic fixes (derived in
``tolerance``); bit-exact reproducibility between calls; group-structure
errors in g_idx reported by the prepare call."""
import numpy as np
import pytest

from oracle import w4a16_oracle as W
from post_weight_quantization_layer_amd import inputs as I
from tests.gpu_harness import log

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24   # unit roundoff of float32
U16 = 2.0 ** -11   # unit roundoff of float16


def tolerance(x_bits, L, rows=None):
    """|y - y64| <= u16 |y64| + (64 + K/128 + 16) u32 sum|x w^| + 2^-24.

    The kernel forms x * (q - z) exactly, sums at most 32 products inside an
    MFMA and chains 4 of them (a 128-column group or less), scales the sum
    once, adds it to the running total (at most K/128 groups), then adds the
    split-K partials (at most K/128): a summation tree of depth below
    64 + K/128 + 16, so the float32 error is below that many u32 times the sum
    of the magnitudes.  Rounding to float16 adds half an ulp (u16 relative,
    2^-25 absolute near zero)."""
    sel = slice(None) if rows is None else rows
    ref = W.w4a16_product(x_bits, L.codes[sel], L.g_idx, L.scale[sel], L.zero[sel])
    mag = W.w4a16_abs_product_sum(x_bits, L.codes[sel], L.g_idx, L.scale[sel], L.zero[sel])
    K = L.codes.shape[1]
    tol = U16 * np.abs(ref) + (64 + K / 128 + 16) * U32 * mag + 2.0 ** -24
    return ref, tol


def run(L, x_bits, calls=1):
    import torch
    from post_weight_quantization_layer_amd.w4a16 import W4A16Linear
    dev = torch.device("cuda")
    lin = W4A16Linear.from_codes(torch.from_numpy(L.codes).to(dev),
                                 torch.from_numpy(L.g_idx).to(dev),
                                 torch.from_numpy(L.scale).to(dev),
                                 torch.from_numpy(L.zero).to(dev), L.group)
    x = torch.from_numpy(x_bits.view(np.int16)).to(dev).view(torch.float16)
    outs = []
    for _ in range(calls):
        y = lin(x)
        torch.cuda.synchronize()
        outs.append(y.view(torch.int16).cpu().numpy().view(np.uint16))
    return outs, lin


def check(y_bits, x_bits, L, rows=None, name=""):
    y = y_bits.view(np.float16).astype(np.float64)
    if rows is not None:
        y = y[:, rows]
    ref, tol = tolerance(x_bits, L, rows)
    err = np.abs(y - ref)
    worst = float(np.max(err / tol))
    log(f"{name}: max |err|/tol = {worst:.3g}, max rel = "
        f"{float(np.max(err / np.maximum(np.abs(ref), 1e-30))):.3g}")
    bad = np.argwhere(err > tol)
    assert bad.size == 0, f"{name}: {len(bad)} outputs out of bound, first {bad[:5].tolist()}"


@pytest.mark.parametrize("rows,cols,group,act", [
    (80, 384, 128, False),
    (80, 384, 128, True),
    (48, 768, 256, True),
    (37, 320, 64, True),     # columns padded to 384, groups of 64
    (21, 352, 32, True),     # columns padded to 384, groups of 32
    (64, 4096, 128, False),  # many split-K partials
    (4200, 512, 128, True),  # more 16-row tiles than CUs: workgroups walk 1-2 tiles
    (9600, 256, 64, False),  # 600 tiles: up to 3 per workgroup
])
@pytest.mark.parametrize("batch", [1, 2, 3, 16, 17, 40, 64, 70])
def test_w4a16_matches_oracle(rows, cols, group, act, batch):
    name = f"w4a16 {rows}x{cols} g{group} act={act} batch={batch}"
    log(name)
    L = I.stored_int4_layer(rows, cols, group, act, seed=rows * 7 + cols + group)
    x = I.activations_f16(batch, cols, seed=batch + 100)
    (y,), lin = run(L, x)
    assert lin.layer.permuted == int(act)
    check(y, x, L, name=name)


@pytest.mark.parametrize("rows,cols,act,batch", [
    (4096, 11008, True, 1),
    (4096, 11008, True, 16),
    (4096, 4096, False, 64),
])
def test_w4a16_full_size(rows, cols, act, batch):
    name = f"w4a16 full {rows}x{cols} act={act} batch={batch}"
    log(name)
    L = I.stored_int4_layer(rows, cols, 128, act, seed=rows + cols)
    x = I.activations_f16(batch, cols, seed=batch)
    (y,), _ = run(L, x)
    check(y, x, L, name=name)


@pytest.mark.parametrize("rows,cols,act,batch", [
    (28672, 8192, True, 4),
    (14336, 4096, False, 32),
])
def test_w4a16_full_size_sampled_rows(rows, cols, act, batch):
    name = f"w4a16 full {rows}x{cols} act={act} batch={batch} (sampled rows)"
    log(name)
    L = I.stored_int4_layer(rows, cols, 128, act, seed=rows + cols)
    x = I.activations_f16(batch, cols, seed=batch)
    (y,), _ = run(L, x)
    pick = np.sort(np.random.default_rng(rows).choice(rows, 512, replace=False))
    pick[-1] = rows - 1
    check(y, x, L, rows=pick, name=name)


def test_w4a16_reproducible_across_calls():
    L = I.stored_int4_layer(4096, 11008, 128, True, seed=1)
    x = I.activations_f16(8, 11008, seed=2)
    outs, _ = run(L, x, calls=3)
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])


@pytest.mark.parametrize("how", ["moved", "out_of_range", "negative"])
def test_w4a16_prepare_rejects_bad_groups(how):
    import torch
    from post_weight_quantization_layer_amd import binding as B
    from post_weight_quantization_layer_amd.w4a16 import W4A16Linear
    L = I.stored_int4_layer(32, 256, 64, True, seed=4)
    g = L.g_idx.copy()
    c = int(np.nonzero(g == 0)[0][0])
    g[c] = {"moved": 1, "out_of_range": 4, "negative": -1}[how]
    dev = torch.device("cuda")
    with pytest.raises(B.GptqError, match="g_idx"):
        W4A16Linear.from_codes(torch.from_numpy(L.codes).to(dev), torch.from_numpy(g).to(dev),
                               torch.from_numpy(L.scale).to(dev),
                               torch.from_numpy(L.zero).to(dev), 64)
