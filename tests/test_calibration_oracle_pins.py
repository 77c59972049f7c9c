"""Pins of the sequential calibration oracle (CPU only)."""
import numpy as np
import pytest

import oracle as O
from oracle import calibration_oracle as C


def test_round_bf16_known_values():
    # exactly representable values pass through; halfway cases go to even
    assert C.round_bf16(np.array([1.0, -2.5, 0.0]))[0] == 1.0
    one_ulp = 2.0 ** -7                                  # bf16 spacing in [1, 2)
    x = np.array([1.0 + one_ulp / 2, 1.0 + 3 * one_ulp / 2, 1.0 + one_ulp / 4])
    np.testing.assert_array_equal(C.round_bf16(x), [1.0, 1.0 + 2 * one_ulp, 1.0])
    # silu(1) * 1 = 0.7310585786... -> bf16 0.73046875 (1 + 59/128) / 2
    assert C.silu_mul(np.array([1.0]), np.array([1.0]))[0] == 0.73046875
    assert C.silu_mul(np.array([0.0]), np.array([5.0]))[0] == 0.0


def test_linear_forward_orientation_exact_case():
    """Small dyadic weights and integer inputs: every product and sum is exact
    and representable, so the outputs are known exactly (rows of W^ times
    columns of X)."""
    W = np.array([[1.0, 0.5, -2.0], [0.0, 0.25, 1.0]])
    X = np.array([[1.0, 2.0, 3.0, 4.0], [4.0, 0.0, -4.0, 8.0], [1.0, 1.0, 0.0, -1.0]])
    Y = C.linear_forward(W, X)
    np.testing.assert_array_equal(Y, [[1.0, 0.0, 1.0, 10.0], [2.0, 1.0, -1.0, 1.0]])


def _chunks(rng, d, n, nc):
    X = C.round_bf16(rng.standard_normal((d, n)))
    return [X[:, i:i + n // nc] for i in range(0, n, n // nc)]


def test_gate_and_up_are_plain_gptq_on_the_block_input():
    rng = np.random.default_rng(1)
    d, dff = 64, 96
    Xc = _chunks(rng, d, 600, 3)
    Wg, Wu, Wd = (rng.standard_normal(s) * 0.02 for s in ((dff, d), (dff, d), (d, dff)))
    out = C.calibrate_gated_mlp(Wg, Wu, Wd, Xc, bits=4, group=32, block=32, act_order=True,
                                percdamp=0.01)
    X = np.concatenate(Xc, axis=1)
    H = O.hessian([X])
    diag = O.hessian_diag([X])
    np.testing.assert_allclose(out["H1"], H, rtol=1e-12, atol=1e-12)
    ref = O.quantize_layer(Wg, H, diag, bits=4, group=32, block=32, act_order=True,
                           percdamp=0.01)
    np.testing.assert_array_equal(out["gate"].q, ref.q)


def test_down_reads_the_outputs_of_the_updated_weights():
    """The down linear's Hessian is built from activations of the quantized
    gate and up (loops over tokens), not of the original weights."""
    rng = np.random.default_rng(2)
    d, dff, n = 32, 48, 200
    Xc = _chunks(rng, d, n, 2)
    Wg, Wu, Wd = (rng.standard_normal(s) * 0.05 for s in ((dff, d), (dff, d), (d, dff)))
    out = C.calibrate_gated_mlp(Wg, Wu, Wd, Xc, bits=3, group=16, block=16, act_order=False,
                                percdamp=0.01)
    X = np.concatenate(Xc, axis=1)
    Gq, Uq = out["gate"].what.astype(np.float64), out["up"].what.astype(np.float64)
    A = np.zeros((dff, n))
    for t in range(n):
        for i in range(dff):
            g = C.round_bf16(np.array([Gq[i] @ X[:, t]]))[0]
            u = C.round_bf16(np.array([Uq[i] @ X[:, t]]))[0]
            A[i, t] = C.round_bf16(np.array([g / (1 + np.exp(-g)) * u]))[0]
    np.testing.assert_array_equal(np.concatenate(out["A"], axis=1), A)
    np.testing.assert_allclose(out["H2"], 2 * A @ A.T, rtol=1e-12, atol=1e-15)
    A0 = C.silu_mul(C.linear_forward(Wg, X), C.linear_forward(Wu, X))
    assert not np.allclose(A0, A)             # the original weights give other inputs


def test_each_linear_beats_round_to_nearest_on_its_own_inputs():
    rng = np.random.default_rng(3)
    d, dff = 64, 128
    Xc = _chunks(rng, d, 900, 3)
    Wg, Wu, Wd = (rng.standard_normal(s) * 0.02 for s in ((dff, d), (dff, d), (d, dff)))
    out = C.calibrate_gated_mlp(Wg, Wu, Wd, Xc, bits=4, group=32, block=32, act_order=True,
                                percdamp=0.01)
    for name, W, H in (("gate", Wg, out["H1"]), ("up", Wu, out["H1"]), ("down", Wd, out["H2"])):
        res = out[name]
        rtn = O.rtn(np.asarray(W)[:, res.perm], O.GridSpec("affine", 4, 32))
        e_rtn = O.reconstruction_error(np.asarray(W)[:, res.perm], rtn.what,
                                       H[np.ix_(res.perm, res.perm)])
        assert O.reconstruction_error(W, res.what, H) <= e_rtn, name
