"""Sequential calibration of a gated MLP block on the GPU (through the C ABI)
against the float64 oracle pipeline, on the same seeded inputs.

Every linear is held to the per-layer bar (H and U within 1e-4, codes
through the tie-forced replay, reconstruction error within 1 %) against the
oracle quantizing it from the SAME activations the GPU quantized it from:
gate and up from the block input, down from the GPU's own stored
activations.  Separately, those activations are compared with the oracle's
own pipeline (exact sums rounded to bf16): a stored activation can differ
where its sum lies within float32 error of a rounding boundary, so at most
0.1 % of them may differ, each by at most a few bf16 steps of its value (or
of 1 % of the activations' rms where a sum cancels to nearly zero; G, U and
A are each rounded).  The whole-pipeline reconstruction error of down is
also held within 1 % of the oracle pipeline's."""
import numpy as np
import pytest

import oracle as O
from oracle import calibration_oracle as C
from post_weight_quantization_layer_amd import inputs as I
from tests.gpu_harness import log
from tests.parity import assert_replay, replay_layer
from tests.parity import assert_codes, classify_codes, rel_fro

pytestmark = pytest.mark.gpu


def _cfgs(d, dff, bits, group, block, act):
    base = I.CONFIGS["down_proj_4096x11008_int4_g128_actorder"]
    kw = dict(bits=bits, group=group, block=block, act_order=act, w_dtype="f32")
    gate = base.with_(rows=dff, cols=d, seed=base.seed + 101, x_kind="gauss",
                      outlier_frac=0.01, outlier_scale=20.0, w_sigma=0.05, **kw)
    up = gate.with_(seed=base.seed + 102)
    down = base.with_(rows=d, cols=dff, seed=base.seed + 103, w_sigma=0.05, **kw)
    return gate, up, down


@pytest.mark.parametrize("d,dff,tokens,chunk,bits,group,block,act", [
    (256, 640, 3000, 1000, 4, 128, 128, True),
    (384, 512, 2100, 700, 3, 64, 64, False),
])
def test_gated_mlp_calibration_matches_oracle(d, dff, tokens, chunk, bits, group, block, act):
    import torch
    from post_weight_quantization_layer_amd.calibrate import GatedMLPCalibrator
    log(f"[calib] d={d} dff={dff} tokens={tokens} bits={bits} g={group} act={act}")
    cg, cu, cd = _cfgs(d, dff, bits, group, block, act)
    Wg, Wu, Wd = I.weight(cg), I.weight(cu), I.weight(cd)
    spans = I.token_chunks(cg.with_(tokens=tokens), chunk)
    store = [I.x_chunk_storage(cg.with_(tokens=tokens), t0, n) for t0, n in spans]
    x64 = [I.bf16_to_f32(s).astype(np.float64) for s in store]

    dev = torch.device("cuda")
    xs = []
    for s in store:
        ld = (s.shape[1] + 7) // 8 * 8
        t = torch.zeros((d, ld), dtype=torch.bfloat16, device=dev)
        t[:, :s.shape[1]] = torch.from_numpy(s.view(np.int16)).view(torch.bfloat16).to(dev)
        xs.append(t[:, :s.shape[1]])
    cal = GatedMLPCalibrator(d, dff, bits=bits, group=group, block=block, act_order=act,
                             device=dev)
    tg, tu, td = (torch.from_numpy(w).to(dev) for w in (Wg, Wu, Wd))
    res = cal.run(tg, tu, td, xs)
    torch.cuda.synchronize()
    o = C.calibrate_gated_mlp(Wg.astype(np.float64), Wu.astype(np.float64),
                              Wd.astype(np.float64), x64, bits=bits, group=group, block=None,
                              act_order=act, percdamp=0.01)

    def per_layer(name, W, H, diag, qres, orc, H_gpu, U_gpu):
        """The per-layer bar for one linear, oracle and GPU on the same inputs."""
        h_err = rel_fro(np.triu(H_gpu), np.triu(H))
        u_err = rel_fro(U_gpu, orc.U)
        qg = qres.q.cpu().numpy()
        rep = classify_codes(qg[:, orc.perm], orc.sweep, "affine", group)
        grid = {"scale": qres.scale.cpu().numpy(), "zero": qres.zero.cpu().numpy()}
        rp = replay_layer(W.astype(np.float64), orc, qg, grid, grid_kind="affine", bits=bits,
                          group=group)
        e_gpu = O.reconstruction_error(W, qres.W_hat.cpu().numpy(), H)
        e_or = O.reconstruction_error(W, orc.what, H)
        log(f"[calib] {name}: H rel {h_err:.2e}, U rel {u_err:.2e}, {rep.mismatches}/{rep.n} "
            f"codes differ, replay adopted {rp.forced}, {len(rp.bad)} off a tie, "
            f"E_gpu/E_oracle = {e_gpu / e_or:.5f}")
        assert h_err <= 1e-4 and u_err <= 1e-4, name
        assert_codes(rep)
        assert_replay(rp, qg[:, orc.perm], grid, "affine")
        assert abs(e_gpu - e_or) <= 0.01 * e_or, name

    # gate and up: the block input, identical on both sides
    U1 = cal.gate_up.U.cpu().numpy()
    H1g = cal.gate_up.H.cpu().numpy()
    per_layer("gate", Wg, o["H1"], o["d1"], res.gate, o["gate"], H1g, U1)
    per_layer("up", Wu, o["H1"], o["d1"], res.up, o["up"], H1g, U1)

    # down: the oracle quantizes it from the GPU's own stored activations
    a_chunks = [a.float().cpu().numpy().astype(np.float64) for a in res.activations]
    H2g = O.hessian(a_chunks)
    d2g = O.hessian_diag(a_chunks)
    orc_d = O.quantize_layer(Wd.astype(np.float64), H2g, d2g, bits=bits, group=group,
                             block=None, act_order=act, percdamp=0.01)
    assert rel_fro(cal.down.hdiag.cpu().numpy(), d2g) <= 1e-12
    per_layer("down", Wd, H2g, d2g, res.down, orc_d, cal.down.H.cpu().numpy(),
              cal.down.U.cpu().numpy())

    # the activations themselves against the oracle's pipeline
    a_gpu = np.concatenate(a_chunks, axis=1)
    a_or = np.concatenate(o["A"], axis=1)
    diff = a_gpu != a_or
    # a bf16 step of the value, or of a hundredth of the activations' rms
    # scale where float32 summation error dominates a sum that cancels to ~0
    scale = np.maximum(np.abs(a_or), 0.01 * np.sqrt(np.mean(a_or ** 2)))
    step = np.abs(a_gpu - a_or) / scale
    log(f"[calib] activations: {int(diff.sum())}/{diff.size} differ, "
        f"max |diff|/scale {step.max():.2e}")
    # G, U and A are each rounded to bf16: an activation may move by up to
    # three steps where G or U sat on a rounding boundary
    assert diff.mean() <= 1e-3
    assert np.all(step <= 2.0 ** -5)
    # and down's error over the oracle pipeline's own inputs
    e_gpu = O.reconstruction_error(Wd, res.down.W_hat.cpu().numpy(), o["H2"])
    e_or = O.reconstruction_error(Wd, o["down"].what, o["H2"])
    log(f"[calib] down over the oracle pipeline's inputs: E_gpu/E_oracle = {e_gpu / e_or:.5f}")
    assert abs(e_gpu - e_or) <= 0.01 * e_or
