"""The tie-forced replay used by the GPU parity tests, checked on the CPU.

A "GPU result" is made here by the oracle itself, with decisions changed on
purpose through its decision hook: a genuine tie taken the other way (the
replay must adopt it and then agree everywhere), and a code changed off a tie
right after such a tie (a compensation bug hiding in a tie's cascade: the
first-difference classifier accepts it, the replay must not)."""
import numpy as np
import pytest

import oracle as O
from post_weight_quantization_layer_amd import inputs as I
from tests.parity import _other_side, assert_replay, classify_codes, replay_ties


def _layer(grid="affine", bits=4, group=32, rows=24, cols=256, tokens=600, act=False):
    base = "q4k_14336x4096" if grid == "q4k" else "q_proj_4096x4096_int4_g128"
    cfg = I.CONFIGS[base].with_(rows=rows, cols=cols, tokens=tokens, bits=bits,
                                group=(256 if grid == "q4k" else group), act_order=act)
    W = I.weight(cfg).astype(np.float64)
    X = I.x_chunk(cfg, 0, tokens)
    H = O.hessian([X])
    diag = O.hessian_diag([X])
    o = O.quantize_layer(W, H, diag, bits=bits, group=cfg.group, block=None, act_order=act,
                         percdamp=0.01, grid=grid)
    Wp = W[:, o.perm]
    spec = O.GridSpec(grid=grid, bits=bits, group=cfg.group)
    return Wp, o, spec


def _grid(sw, grid):
    if grid == "affine":
        return {"scale": sw.scale, "zero": sw.zero}
    return {"D": sw.D, "Dm": sw.Dm, "sc": sw.sc, "mc": sw.mc}


class _Flip:
    """Take the other rounding of chosen (column, row) code decisions."""

    def __init__(self, at):
        self.at = at   # {(j, r): "tie" | "off"}

    def __call__(self, name, j, pre, val):
        if name != "code":
            return val
        val = np.array(val, np.float32)
        for (jj, r), kind in self.at.items():
            if jj == j:
                val[r] += _other_side(pre[r]) if kind == "tie" else 1.0 if val[r] < 7 else -1.0
        return val


@pytest.mark.parametrize("grid", ["affine", "q4k"])
def test_replay_of_the_oracle_itself_adopts_nothing(grid):
    Wp, o, spec = _layer(grid)
    sw = o.sweep
    rep = replay_ties(Wp, o.U, spec, sw.q, _grid(sw, grid))
    assert rep.forced_total == 0 and not rep.bad
    assert_replay(rep, sw.q, _grid(sw, grid), grid)


def _closest_tie(sw, row, lo=8):
    """Column of ``row`` (past the first ``lo``) whose pre-rounding value is
    nearest a half-integer, and that distance."""
    frac = np.abs(sw.ratio[row, lo:].astype(np.float64) % 1.0 - 0.5)
    frac[~np.isfinite(frac)] = 1.0
    j = int(np.argmin(frac)) + lo
    return j, float(frac[j - lo])


@pytest.mark.parametrize("grid", ["affine", "q4k"])
def test_replay_adopts_a_tie_and_its_cascade(grid):
    Wp, o, spec = _layer(grid)
    row = 5
    j, dist = _closest_tie(o.sweep, row)
    other = O.gptq_sweep(Wp, o.U, spec, None, decide=_Flip({(j, row): "tie"}))
    assert (other.q[row] != o.sweep.q[row]).any()
    tau = dist * 1.01 + 1e-9
    rep = replay_ties(Wp, o.U, spec, other.q, _grid(other, grid), tau=tau)
    assert not rep.bad
    assert rep.forced.get("code", 0) >= 1
    assert_replay(rep, other.q, _grid(other, grid), grid, max_frac=1.0)


def test_replay_catches_an_error_inside_a_tie_cascade():
    """A code changed off a tie, later in the row than a genuine tie: the
    first-difference classifier calls it cascade; the replay reports it."""
    Wp, o, spec = _layer("affine")
    row = 3
    j, dist = _closest_tie(o.sweep, row)
    # a later column of the same row whose value is far from any tie
    fr = np.abs(o.sweep.ratio[row].astype(np.float64) % 1.0 - 0.5)
    later = [k for k in range(j + 3, Wp.shape[1]) if fr[k] > 0.3
             and 0 < o.sweep.q[row, k] < 15]
    k = later[0]
    bad = O.gptq_sweep(Wp, o.U, spec, None, decide=_Flip({(j, row): "tie", (k, row): "off"}))
    tau = dist * 1.01 + 1e-9
    cls = classify_codes(bad.q, o.sweep, "affine", spec.group, tau=tau)
    assert not cls.unclassified          # the old classifier cannot see it
    rep = replay_ties(Wp, o.U, spec, bad.q, _grid(bad, "affine"), tau=tau)
    assert any(b[0] == "code" and b[1] == k and b[2] == row for b in rep.bad), rep.bad[:3]
    with pytest.raises(AssertionError):
        assert_replay(rep, bad.q, _grid(bad, "affine"), "affine", max_frac=1.0)


def test_replay_adopts_a_zero_point_tie():
    """The zero point of a group taken the other way at a (forced) tie."""
    Wp, o, spec = _layer("affine")
    row = 7
    frac = np.abs(o.sweep.zratio[row].astype(np.float64) % 1.0 - 0.5)
    gi = int(np.argmin(frac))
    j0 = gi * spec.group

    def flip_zero(name, j, pre, val):
        if name == "zero" and j == j0:
            val = np.array(val, np.float32)
            val[row] += _other_side(pre[row])
        return val

    other = O.gptq_sweep(Wp, o.U, spec, None, decide=flip_zero)
    rep = replay_ties(Wp, o.U, spec, other.q, _grid(other, "affine"),
                      tau=float(frac[gi]) * 1.01 + 1e-9)
    assert not rep.bad and rep.forced.get("zero", 0) == 1
    assert_replay(rep, other.q, _grid(other, "affine"), "affine", max_frac=1.0)


def test_replay_rejects_a_wrong_super_scale():
    """An fp16 super-scale one step off where the value is not at a rounding
    midpoint is reported."""
    Wp, o, spec = _layer("q4k")
    row, sb = 2, 0

    def bump_d(name, j, pre, val):
        if name == "D" and j == sb * O.Q4K_SUPER:
            val = np.array(val, np.float16)
            val[row] = np.nextafter(val[row], np.float16(np.inf))
        return val

    other = O.gptq_sweep(Wp, o.U, spec, None, decide=bump_d)
    rep = replay_ties(Wp, o.U, spec, other.q, _grid(other, "q4k"))
    assert any(b[0] == "D" for b in rep.bad)
