"""Pins of the oracle's R form of the factor (oracle.gptq_oracle.r_form) and of the identity the library's
second quantize route rests on.

Lesson "GPTQ's error-compensation loop": every column's residual over the pivot is the row's error, and the
later columns take off error * U[j][k]; summed over the loop, the start minus the quantized values of a row is
its errors times U (W0 - Q = E U, U upper with a positive diagonal). With R = U^-1 this gives E = D R,
D = W0 - Q. The checks below tie R to the definition (R R^T = H), to U computed another way (the inverse
and its Cholesky factor), and the identity to the oracle's own loop.
"""
import numpy as np
import pytest

from oracle import gptq_oracle as O


def _spd(d, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((3 * d + 5, d)) @ (np.eye(d) + 0.3 * rng.standard_normal((d, d)))
    S, colsq, n = O.hessian_from_x(X)
    H_p, perm, dead, lam = O.prepare(S, colsq, n, 0.01, True)
    return H_p


@pytest.mark.parametrize("d", [1, 5, 64, 130, 256, 320])
def test_r_form_is_the_reversed_factor_and_u_inverse(d):
    H = _spd(d, 100 + d)
    M = O.r_form(H)
    R = np.triu(M)
    # the definition: upper, positive diagonal, R R^T = H
    assert np.all(np.diag(R) > 0)
    assert np.linalg.norm(R @ R.T - H) <= 1e-12 * np.linalg.norm(H)
    # R is U^-1 for U from the inverse and its Cholesky factor
    U = O.upper_factor_of_inverse(H)
    assert np.linalg.norm(R @ U - np.eye(d)) <= 1e-10 * np.sqrt(d) * np.linalg.cond(R)
    # the strictly lower parts of the 128 x 128 diagonal blocks are U's diagonal blocks, reversed
    for b in range(0, d, 128):
        p = min(128, d - b)
        lower = np.tril(M[b:b + p, b:b + p], -1)
        want = np.tril(U[b:b + p, b:b + p][::-1, ::-1], -1)
        assert np.allclose(lower, want, rtol=1e-9, atol=1e-12 * np.abs(U).max())
    # nothing else below the diagonal
    outside = np.tril(M, -1).copy()
    for b in range(0, d, 128):
        outside[b:b + 128, b:b + 128] = 0.0
    assert np.all(outside == 0.0)


def test_r_form_panel_layout_by_hand():
    """A 3 x 3 case with a 2-column block, worked by hand: H = R R^T for a chosen R, U = R^-1."""
    R = np.array([[2.0, 1.0, -1.0], [0.0, 4.0, 2.0], [0.0, 0.0, 1.0]])
    H = R @ R.T
    M = O.r_form(H, panel=2)
    assert np.allclose(np.triu(M), R, atol=1e-14)
    # U = R^-1: U[0][1] = -1/8; block [0, 2) stores J U_00 J, i.e. U[0][1] at (1, 0); block [2, 3) is 1 x 1
    U = np.linalg.inv(R)
    assert U[0, 1] == pytest.approx(-0.125)
    assert M[1, 0] == pytest.approx(-0.125)
    assert M[2, 0] == 0.0 and M[2, 1] == 0.0


@pytest.mark.parametrize("group", [0, 8])
def test_loop_errors_are_d_times_r(group):
    """E = (W0 - Q) R on the oracle's own loop: the identity behind the R-form route."""
    rng = np.random.default_rng(7 + group)
    d, out = 40, 6
    H = _spd(d, 11)
    U = O.upper_factor_of_inverse(H)
    R = np.triu(O.r_form(H))
    W0 = 0.1 * rng.standard_normal((out, d))
    codes, scales, errs, loss = O.compensation_loop(W0, U, 4, group)
    g = (np.arange(d) // group) if group else np.zeros(d, dtype=int)
    Q = codes * scales[:, g]
    D = W0 - Q
    assert np.allclose(D, errs @ U, rtol=0, atol=1e-12 * np.abs(W0).max())
    assert np.allclose(errs, D @ R, rtol=0, atol=1e-9 * np.abs(errs).max())
    # a planted mistake (the diagonal dropped from U) breaks the identity
    assert not np.allclose(D, errs @ np.triu(U, 1), rtol=0, atol=1e-6 * np.abs(W0).max())
