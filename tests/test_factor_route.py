"""The compensation carried by the Hessian's own factor (CPU, float64).

The HIP path can take the compensation between blocks from the factor of
the damped Hessian itself instead of U, the Cholesky factor of Hp^-1
("GPTQ", section Komponenty).  With Hp = R R^T (R upper, so U = R^-1), the
pages' errors satisfy W - W^ = E U, hence E = (W - W^) R.  Writing o for the
weights before any compensation, the compensated weights of a block B at its
turn, with every earlier column fixed, are

    c_B = o_B + (o - w^)_{<B} R_{<B,B} U_BB,

U_BB being U's diagonal block of B (the inverse of R's).  So the lazy
updates can hand each block its compensated weights directly through
M = R_{<B,B} U_BB, with the error w^_j - o_j, and the pages' rule runs
inside the block on U_BB.  Only U's diagonal blocks are inverted, which a
blocked Cholesky forms anyway; no inverse of the whole factor is needed.

This file checks that formulation in float64 against the oracle, which
follows the pages' route: the same codes (decisions in float32 on both
sides, on values that agree to about 1e-13) and the same W^.
"""
import numpy as np
import pytest

import oracle as O


def hessian_route_factor(U, T, block):
    """F: U's diagonal blocks, and M = R_{<B,B} U_BB above them (R = T diag(R),
    diag(R) = 1 / diag(U)); zero below."""
    d = U.shape[0]
    R = T / np.diag(U)[None, :]
    F = np.zeros((d, d))
    for b0 in range(0, d, block):
        b1 = min(b0 + block, d)
        F[b0:b1, b0:b1] = U[b0:b1, b0:b1]
        F[:b0, b0:b1] = R[:b0, b0:b1] @ U[b0:b1, b0:b1]
    return F


def sweep_hessian_factor(Wp, F, spec, block):
    """Blocked sweep over Wp (processing order): between blocks the updates
    go through F's blocks above the diagonal with the error w^ - o; inside a
    block the pages' rule runs on F's diagonal block (U_BB)."""
    o = np.array(Wp, dtype=np.float64)
    W = o.copy()
    r, d = W.shape
    Q = np.zeros((r, d))
    What = np.zeros((r, d))
    span = spec.span
    for i1 in range(0, d, block):
        i2 = min(i1 + block, d)
        E = np.zeros((r, i2 - i1))
        for j in range(i1, i2):
            if j % span == 0:
                v = W[:, j:j + span].astype(np.float32)
                if spec.grid == "affine":
                    s, zp, _ = O.affine_params(v, spec.bits)
                else:
                    _, _, _, _, S, M = O.q4k_params(v, spec.bits)
            if spec.grid == "affine":
                q, wq = O.affine_quantize(W[:, j].astype(np.float32), s, zp, spec.bits)
            else:
                b = (j % span) // O.Q4K_SUB
                q, wq = O.q4k_quantize(W[:, j].astype(np.float32), S[:, b], M[:, b], spec.bits)
            wq = wq.astype(np.float64)
            e = (W[:, j] - wq) / F[j, j]
            W[:, j + 1:i2] -= np.outer(e, F[j, j + 1:i2])
            E[:, j - i1] = wq - o[:, j]
            Q[:, j], What[:, j] = q, wq
            W[:, j] = wq
        if i2 < d:
            W[:, i2:] -= E @ F[i1:i2, i2:]
    return Q, What


@pytest.mark.parametrize("grid,bits,group,block,act", [
    ("affine", 4, 16, 16, False),
    ("affine", 3, 32, 64, True),
    ("affine", 2, 64, 64, True),
    ("affine", 8, 16, 32, False),
    ("affine", 4, 128, 128, True),
    ("q4k", 4, 256, 256, False),
])
def test_unit_factor_sweep_equals_oracle(grid, bits, group, block, act):
    rng = np.random.default_rng(bits * 31 + block)
    r, d = 10, 256
    X = rng.standard_normal((d, 700))
    X[rng.choice(d, 4, replace=False)] *= 15
    W = rng.standard_normal((r, d)) * 0.02
    H, diag = O.hessian([X]), O.hessian_diag([X])
    res = O.quantize_layer(W, H, diag, bits=bits, group=group, block=None,
                           act_order=act, percdamp=0.01, grid=grid)
    Hp = O.damped_processing_hessian(H, diag, res.perm, 0.01)
    F = hessian_route_factor(res.U, O.unit_upper_factor(Hp), block)
    spec = O.GridSpec(grid, bits, group)
    Q, What = sweep_hessian_factor(W[:, res.perm], F, spec, block)
    np.testing.assert_array_equal(Q, res.sweep.q)
    np.testing.assert_allclose(What, res.sweep.what, rtol=0, atol=1e-7)


def test_unit_factor_dead_column():
    """A feature that never fires: its weights are zeroed before the sweep
    on both routes, and H_ii := 1."""
    rng = np.random.default_rng(3)
    r, d = 6, 64
    X = rng.standard_normal((d, 300))
    X[5] = 0.0
    W = rng.standard_normal((r, d)) * 0.02
    H, diag = O.hessian([X]), O.hessian_diag([X])
    res = O.quantize_layer(W, H, diag, bits=4, group=16, block=None, act_order=True,
                           percdamp=0.01)
    Hp = O.damped_processing_hessian(H, diag, res.perm, 0.01)
    Wd = W.copy()
    Wd[:, res.dead] = 0.0
    F = hessian_route_factor(res.U, O.unit_upper_factor(Hp), 16)
    Q, What = sweep_hessian_factor(Wd[:, res.perm], F, O.GridSpec("affine", 4, 16), 16)
    np.testing.assert_array_equal(Q, res.sweep.q)
    np.testing.assert_allclose(What, res.sweep.what, rtol=0, atol=1e-7)
