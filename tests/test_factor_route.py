"""The compensation carried by the Hessian's own factor (CPU, float64).

The HIP path can take the compensation between blocks from T, the unit upper
factor with Hp = T D T^T, instead of U, the Cholesky factor of Hp^-1
("GPTQ", section Komponenty).  With R = U^-1 (so T = R diag(R)^-1) the
pages' errors satisfy W - W^ = E U, hence E = (W - W^) R.  Writing o for the
weights before any compensation, the weight a column k has when its turn
comes is

    w_k = o_k + sum_{j<k} (o_j - w^_j) T_jk,

so between blocks the later columns take y -= (w^_j - o_j) T_jk.  Inside a
block a group's grid is chosen from the compensated weights of all its
columns with the earlier columns fixed -- for the block B starting at i1,
c = o_B + z U_BB with z_j = (y_j - o_j) R_jj -- and the pages' rule then runs
on U_BB, the inverse factor's diagonal block, from c.  Only U's diagonal
blocks are needed, which a blocked Cholesky forms anyway.

This file checks that formulation in float64 against the oracle, which
follows the pages' route: the same codes (decisions in float32 on both
sides, on values that agree to about 1e-13) and the same W^.
"""
import numpy as np
import pytest

import oracle as O


def sweep_hessian_factor(Wp, U, T, spec, block):
    """Blocked sweep over Wp (processing order): T between blocks, U's
    diagonal blocks inside them."""
    o = np.array(Wp, dtype=np.float64)
    Y = o.copy()
    r, d = Y.shape
    Q = np.zeros((r, d))
    What = np.zeros((r, d))
    span = spec.span
    Rd = 1.0 / np.diag(U)          # R_jj
    for i1 in range(0, d, block):
        i2 = min(i1 + block, d)
        Ub = U[i1:i2, i1:i2]
        z = (Y[:, i1:i2] - o[:, i1:i2]) * Rd[None, i1:i2]
        C = o[:, i1:i2] + z @ Ub
        E = np.zeros((r, i2 - i1))
        for j in range(i1, i2):
            jj = j - i1
            if j % span == 0:
                v = C[:, jj:jj + span].astype(np.float32)
                if spec.grid == "affine":
                    s, zp, _ = O.affine_params(v, spec.bits)
                else:
                    _, _, _, _, S, M = O.q4k_params(v, spec.bits)
            if spec.grid == "affine":
                q, wq = O.affine_quantize(C[:, jj].astype(np.float32), s, zp, spec.bits)
            else:
                b = (j % span) // O.Q4K_SUB
                q, wq = O.q4k_quantize(C[:, jj].astype(np.float32), S[:, b], M[:, b], spec.bits)
            wq = wq.astype(np.float64)
            e = (C[:, jj] - wq) / Ub[jj, jj]
            C[:, jj + 1:] -= np.outer(e, Ub[jj, jj + 1:])
            E[:, jj] = wq - o[:, j]
            Q[:, j], What[:, j] = q, wq
        if i2 < d:
            Y[:, i2:] -= E @ T[i1:i2, i2:]
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
    T = O.unit_upper_factor(Hp)
    spec = O.GridSpec(grid, bits, group)
    Q, What = sweep_hessian_factor(W[:, res.perm], res.U, T, spec, block)
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
    Q, What = sweep_hessian_factor(Wd[:, res.perm], res.U, O.unit_upper_factor(Hp),
                                   O.GridSpec("affine", 4, 16), 16)
    np.testing.assert_array_equal(Q, res.sweep.q)
    np.testing.assert_allclose(What, res.sweep.what, rtol=0, atol=1e-7)
