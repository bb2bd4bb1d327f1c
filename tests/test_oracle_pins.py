"""Pins for the CPU oracle: checks against what the pages and the mathematics fix, not against the
oracle's own formulas. Each test names the passage it follows. CPU only.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

from oracle import gptq_oracle as O
import synthetic as syn

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_problem(seed, out, d, n, relu=False, dead=()):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, d))
    if relu:
        X = np.maximum(X, 0.0)
    X[:, list(dead)] = 0.0
    # mild correlation between inputs so that compensation matters
    X = X @ (np.eye(d) + 0.3 * rng.standard_normal((d, d)) / np.sqrt(d))
    X[:, list(dead)] = 0.0
    W = 0.1 * rng.standard_normal((out, d))
    return W, X


# ------------------------------------------------------------------------------------------------
# Hand-worked example (tests/golden/two_column_hand.json)
# ------------------------------------------------------------------------------------------------
def test_golden_two_column_hand():
    g = json.load(open(os.path.join(HERE, "golden", "two_column_hand.json")))
    W, X = np.array(g["W"]), np.array(g["X"])
    r = O.gptq_oracle(W, X, bits=g["bits"], group=g["group"], damp=g["damp"])
    np.testing.assert_allclose(r["H_p"], g["H"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(r["U"], g["U"], rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(r["codes"], g["codes"])
    np.testing.assert_allclose(r["scales"][:, 0], g["scales"], rtol=1e-15)
    np.testing.assert_allclose(r["loss"], g["loss"], rtol=1e-12)
    # the updated column 1 just before it is rounded: q1 + err1 * U11
    upd = r["codes"][:, 1] * r["scales"][:, 0] + r["errs"][:, 1] * r["U"][1, 1]
    np.testing.assert_allclose(upd, g["column1_after_update"], rtol=1e-12)
    codes_rtn, _ = O.rtn(W, g["bits"])
    np.testing.assert_array_equal(codes_rtn, g["rtn_codes"])


# ------------------------------------------------------------------------------------------------
# P-1: Hessian accumulation
# ------------------------------------------------------------------------------------------------
def test_hessian_brute_force_and_chunking():
    """[guide] 'The idea': H = 2 X^T X / n; S checked entry by entry as a plain sum over rows."""
    rng = np.random.default_rng(7)
    X = rng.standard_normal((37, 6))
    S, colsq, n = O.hessian_from_x(X)
    assert n == 37
    for i in range(6):
        for j in range(6):
            ref = sum(X[k, i] * X[k, j] for k in range(37))
            assert abs(S[i, j] - ref) <= 1e-12 * (1 + abs(ref))
        assert abs(colsq[i] - sum(X[k, i] ** 2 for k in range(37))) <= 1e-12 * colsq[i]
    # streaming over several calls equals one call; chunk size larger than the hessian chunk
    Xb = rng.standard_normal((5000, 12))
    S1, c1, n1 = O.hessian_from_x(Xb)
    S2, c2 = np.zeros((12, 12)), np.zeros(12)
    n2 = O.accumulate(S2, c2, Xb[:1234]) + O.accumulate(S2, c2, Xb[1234:])
    assert n1 == n2 == 5000
    np.testing.assert_allclose(S1, S2, rtol=1e-13)
    np.testing.assert_allclose(c1, np.diag(S1), rtol=1e-13)
    # H from prepare with damp=0 and no dead inputs is exactly 2 S / n (symmetric)
    H, perm, dead, lam = O.prepare(S1, c1, n1, 0.0, False)
    assert lam == 0.0 and not dead.any()
    np.testing.assert_allclose(H, 2.0 * Xb.T @ Xb / 5000, rtol=1e-12)
    assert np.array_equal(H, H.T)


def test_flattened_3d_inputs_count_tokens():
    """[handbook] compute_hessian flattens (samples, seq, hidden) to (tokens, hidden)."""
    rng = np.random.default_rng(3)
    X3 = rng.standard_normal((4, 9, 5))
    S, colsq, n = O.hessian_from_x(X3.reshape(-1, 5))
    assert n == 36
    np.testing.assert_allclose(S, np.einsum("abi,abj->ij", X3, X3), rtol=1e-13)


# ------------------------------------------------------------------------------------------------
# P-2, P-16: dead inputs, damping
# ------------------------------------------------------------------------------------------------
def test_damping_and_dead_hand_values():
    """[guide] Damping: add 0.01 * mean(diag H); dead inputs (zero diagonal) get H_ii = 1 first."""
    X = np.array([[1.0, 0.0, 2.0], [3.0, 0.0, -1.0]])  # column 1 never fires
    S, colsq, n = O.hessian_from_x(X)
    H, perm, dead, lam = O.prepare(S, colsq, n, 0.01, False)
    # 2 X^T X / 2 = X^T X = [[10, 0, -1], [0, 0, 0], [-1, 0, 5]]; dead fix -> H11 = 1; mean diag = 16/3
    assert dead.tolist() == [False, True, False]
    assert lam == pytest.approx(0.01 * 16.0 / 3.0, rel=1e-15)
    ref = np.array([[10.0, 0, -1], [0, 1, 0], [-1, 0, 5]]) + lam * np.eye(3)
    np.testing.assert_allclose(H, ref, rtol=1e-15)
    r = O.gptq_oracle(np.array([[0.3, 0.9, -0.2]]), X, bits=3)
    assert r["codes"][0, 1] == 0 and r["Q"][0, 1] == 0.0


def test_all_dead_inputs():
    """P-2: all inputs dead -> H = (1 + damp) I, U = I / sqrt(1 + damp), every code 0."""
    X = np.zeros((16, 5))
    W = np.random.default_rng(1).standard_normal((3, 5))
    r = O.gptq_oracle(W, X, bits=4, damp=0.01)
    np.testing.assert_allclose(r["H_p"], 1.01 * np.eye(5), rtol=1e-15)
    np.testing.assert_allclose(r["U"], np.eye(5) / np.sqrt(1.01), rtol=1e-15)
    assert (r["codes"] == 0).all() and (r["Q"] == 0).all()


def test_not_spd_without_damping():
    """P-16: with damp = 0 a rank-deficient X (duplicated column) has no Cholesky factor."""
    rng = np.random.default_rng(5)
    X = rng.standard_normal((20, 4))
    X[:, 3] = X[:, 1]
    with pytest.raises(np.linalg.LinAlgError):
        O.gptq_oracle(rng.standard_normal((2, 4)), X, damp=0.0)
    # any positive damping with one live input makes it positive definite
    O.gptq_oracle(rng.standard_normal((2, 4)), X, damp=1e-3)


# ------------------------------------------------------------------------------------------------
# P-3, P-4: U
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("d", [1, 2, 7, 64, 300])
def test_u_factor_properties_and_reverse_closed_form(d):
    """[guide] trick 2: U upper with U^T U = H^-1 (unique with a positive diagonal). Independently,
    H = V V^T with V = U^-1 upper, so J V J is the (lower) Cholesky factor of J H J (J reverses
    the index order) and U = J chol(J H J)^-1 J without forming H^-1."""
    W, X = rand_problem(d, 2, d, 3 * d + 5)
    S, colsq, n = O.hessian_from_x(X)
    H, _, _, _ = O.prepare(S, colsq, n, 0.01, False)
    U = O.upper_factor_of_inverse(H)
    assert np.array_equal(U, np.triu(U)) and (np.diag(U) > 0).all()
    Hinv = np.linalg.inv(H)
    assert np.linalg.norm(U.T @ U - Hinv) <= 1e-10 * np.linalg.norm(Hinv)
    J = np.eye(d)[::-1]
    Lr = np.linalg.cholesky(J @ H @ J)
    U2 = J @ scipy.linalg.solve_triangular(Lr, np.eye(d), lower=True) @ J
    assert np.linalg.norm(U - U2) <= 1e-10 * np.linalg.norm(U)


def test_u_rows_are_eliminated_inverse_rows():
    """[guide] trick 2: row j of U equals row j of H_F^-1 (F = {j..d-1}) over sqrt(H_F^-1[j, j]),
    with H_F^-1 from successive Gaussian elimination ('Remove j and repeat')."""
    W, X = rand_problem(11, 1, 6, 40)
    S, colsq, n = O.hessian_from_x(X)
    H, _, _, _ = O.prepare(S, colsq, n, 0.01, False)
    U = O.upper_factor_of_inverse(H)
    Hinv = np.linalg.inv(H)
    for j in range(6):
        np.testing.assert_allclose(U[j, j:], Hinv[j, j:] / np.sqrt(Hinv[j, j]), rtol=1e-10, atol=1e-14)
        Hinv = Hinv - np.outer(Hinv[:, j], Hinv[j, :]) / Hinv[j, j]


# ------------------------------------------------------------------------------------------------
# P-5, P-6: the loop against the OBS form
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(40))
def test_cholesky_form_equals_obs_elimination(seed):
    """P-5: [guide] 'How it works': the OBS step plus Gaussian elimination of H^-1 gives the same codes
    and the same trajectory as the Cholesky-form update, for in <= 8."""
    rng = np.random.default_rng(1000 + seed)
    d = int(rng.integers(1, 9))
    out = int(rng.integers(1, 5))
    bits = int(rng.integers(2, 5))
    group = int(rng.choice([0, 1, 2, 3, d]))
    W, X = rand_problem(seed, out, d, d + int(rng.integers(1, 20)), relu=bool(seed % 3 == 0))
    r = O.gptq_oracle(W, X, bits=bits, group=group, damp=0.01)
    codes_obs, traj = O.obs_elimination_loop(r["W0"], r["H_p"], bits, group)
    np.testing.assert_array_equal(r["codes_q"], codes_obs)
    # replay the Cholesky form and compare the not-yet-rounded columns before each step
    Wc = r["W0"].copy()
    for j in range(d):
        np.testing.assert_allclose(Wc[:, j:], traj[j][:, j:], rtol=1e-9, atol=1e-12)
        if group and j % group == 0:
            sc = O.row_scales(Wc[:, j:j + group], O.qmax_for(bits))
        elif j == 0:
            sc = O.row_scales(Wc, O.qmax_for(bits))
        q = r["codes_q"][:, j] * sc
        e = (Wc[:, j] - q) / r["U"][j, j]
        Wc[:, j + 1:] -= np.outer(e, r["U"][j, j + 1:])


def test_each_step_is_the_constrained_least_squares_solve():
    """P-6: [guide] OBS steps 1-4: the update minimises 1/2 delta H delta^T over the remaining
    coordinates subject to delta_j = -e, and the objective rises by e^2 / (2 H_F^-1[j, j])."""
    W, X = rand_problem(21, 1, 7, 30)
    r = O.gptq_oracle(W, X, bits=3)
    H, U, d = r["H_p"], r["U"], 7
    for j in range(d):
        e = 0.37 * (j + 1)  # any forced change
        F = np.arange(j, d)
        HF = H[np.ix_(F, F)]
        m = len(F)
        K = np.zeros((m + 1, m + 1))
        K[:m, :m] = HF
        K[m, 0] = K[0, m] = 1.0
        rhs = np.zeros(m + 1)
        rhs[m] = -e
        delta = np.linalg.solve(K, rhs)[:m]
        np.testing.assert_allclose(delta[1:], -(e / U[j, j]) * U[j, j + 1:], rtol=1e-9, atol=1e-12)
        rise = 0.5 * delta @ HF @ delta
        assert rise == pytest.approx(e * e / (2.0 * U[j, j] ** 2), rel=1e-9)


def _exact_gptq(W, X, bits, group, damp):
    """Exact rational arithmetic: H, damping, dead fix, explicit H^-1 by Gauss-Jordan, the OBS step
    and elimination. Round-half-even on exact values. Brute force for tiny inputs only."""
    n, d = X.shape
    Xf = [[Fraction(float(v)) for v in row] for row in X]
    S = [[sum(Xf[k][i] * Xf[k][j] for k in range(n)) for j in range(d)] for i in range(d)]
    H = [[2 * S[i][j] / n for j in range(d)] for i in range(d)]
    dead = [S[i][i] == 0 for i in range(d)]
    for i in range(d):
        if dead[i]:
            H[i][i] = Fraction(1)
    lam = Fraction(damp) * sum(H[i][i] for i in range(d)) / d
    for i in range(d):
        H[i][i] += lam
    A = [row[:] + [Fraction(int(i == j)) for j in range(d)] for i, row in enumerate(H)]
    for c in range(d):
        p = max(range(c, d), key=lambda r: abs(A[r][c]))
        A[c], A[p] = A[p], A[c]
        piv = A[c][c]
        A[c] = [v / piv for v in A[c]]
        for r in range(d):
            if r != c and A[r][c] != 0:
                f = A[r][c]
                A[r] = [a - f * b for a, b in zip(A[r], A[c])]
    Hinv = [row[d:] for row in A]
    qmax = 2 ** (bits - 1) - 1
    floor = Fraction(1e-12)
    codes = []
    for wrow in W:
        w = [Fraction(0) if dead[i] else Fraction(float(v)) for i, v in enumerate(wrow)]
        Hi = [row[:] for row in Hinv]
        s = max(max(abs(v) for v in w), floor) / qmax
        crow = []
        for j in range(d):
            if group and j % group == 0:
                s = max(max(abs(v) for v in w[j:j + group]), floor) / qmax
            c = min(max(round(w[j] / s), -qmax), qmax)
            crow.append(c)
            e = w[j] - c * s
            f = e / Hi[j][j]
            w = [w[k] - f * Hi[j][k] for k in range(d)]
            Hi = [[Hi[a][b] - Hi[a][j] * Hi[j][b] / Hi[j][j] for b in range(d)] for a in range(d)]
        codes.append(crow)
    return np.array(codes, dtype=np.int64), np.array(dead)


@pytest.mark.parametrize("seed", range(12))
def test_loop_matches_exact_rational_obs(seed):
    """P-5 in exact arithmetic: codes of the fp64 Cholesky-form oracle equal those of an exact
    rational OBS/elimination run (no square roots, no rounding until the grid decision)."""
    rng = np.random.default_rng(77 + seed)
    d = int(rng.integers(1, 6))
    out = int(rng.integers(1, 4))
    bits = int(rng.integers(2, 5))
    group = int(rng.choice([0, 1, 2, d]))
    W, X = rand_problem(500 + seed, out, d, d + 3, dead=(0,) if (seed % 4 == 1 and d > 1) else ())
    r = O.gptq_oracle(W, X, bits=bits, group=group, damp=0.01)
    ex_codes, ex_dead = _exact_gptq(W, X, bits, group, 0.01)
    np.testing.assert_array_equal(r["dead"], ex_dead)
    np.testing.assert_array_equal(r["codes_q"], ex_codes)


@pytest.mark.parametrize("seed", range(4))
def test_group_scales_from_updated_weights_exact(seed):
    """[guide] 'The code, line by line': at each group boundary the scale comes from the already-updated
    weights W[:, j:j+group]. Exact rational OBS run with several groups per row."""
    W, X = rand_problem(900 + seed, 3, 6, 9)
    X[:, 1] += 2.0 * X[:, 0]  # strong coupling so that updates move the next group's maximum
    r = O.gptq_oracle(W, X, bits=2, group=2, damp=0.01)
    ex_codes, _ = _exact_gptq(W, X, 2, 2, 0.01)
    np.testing.assert_array_equal(r["codes_q"], ex_codes)
    codes_obs, traj = O.obs_elimination_loop(r["W0"], r["H_p"], 2, 2)
    for g0 in range(0, 6, 2):
        ref = np.maximum(np.abs(traj[g0][:, g0:g0 + 2]).max(1), 1e-12) / 1
        np.testing.assert_allclose(r["scales"][:, g0 // 2], ref, rtol=1e-9)


# ------------------------------------------------------------------------------------------------
# P-7, P-9, P-10: special cases that reduce to RTN
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("bits", [3, 4])
def test_heavy_damping_is_rtn(bits):
    """P-7: [guide] 'When it breaks': heavy damping makes H ~ multiple of I, and GPTQ turns into RTN."""
    c = syn.config_by_name("tiny")
    W = O.to_f64(syn.gen_w(c), c.dtype)
    X = O.to_f64(syn.gen_x(c), c.dtype)
    r = O.gptq_oracle(W, X, bits=bits, damp=1e6)
    codes_rtn, Q_rtn = O.rtn(W, bits)
    np.testing.assert_array_equal(r["codes"], codes_rtn)


def test_orthogonal_inputs_and_single_input_are_rtn():
    """P-9: diagonal H gives U[j, j+1:] = 0, so nothing is pushed and GPTQ equals RTN; same for in=1."""
    rng = np.random.default_rng(9)
    Qm, _ = np.linalg.qr(rng.standard_normal((64, 8)))
    X = Qm * rng.uniform(0.5, 3.0, 8)  # orthogonal columns with different norms
    W = rng.standard_normal((5, 8))
    r = O.gptq_oracle(W, X, bits=3)
    assert np.abs(np.triu(r["U"], 1)).max() < 1e-12
    np.testing.assert_array_equal(r["codes"], O.rtn(W, 3)[0])
    r1 = O.gptq_oracle(W[:, :1], X[:, :1], bits=3)
    np.testing.assert_array_equal(r1["codes"], O.rtn(W[:, :1], 3)[0])


def test_group_sizes_special_cases():
    """P-10: group = in is one group = the per-row scale; group = 1 rounds every weight exactly to
    +-qmax (scale from the weight itself), so no error is pushed."""
    W, X = rand_problem(4, 6, 10, 40)
    a = O.gptq_oracle(W, X, bits=4, group=0)
    b = O.gptq_oracle(W, X, bits=4, group=10)
    np.testing.assert_array_equal(a["codes"], b["codes"])
    c = O.gptq_oracle(W, X, bits=3, group=1)
    assert set(np.unique(np.abs(c["codes"]))) <= {0, 3}
    assert np.abs(c["errs"]).max() < 1e-12
    np.testing.assert_allclose(c["Q"], W, rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------------------------------------------
# P-8, P-15: the loss identity, clipping
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("group,act", [(0, False), (4, False), (4, True)])
def test_loss_identity(group, act):
    """P-8: per row, sum_j err_j^2 = (q - w0) H_p (q - w0)^T, because q - w0 = -err U and
    U H_p U^T = I ([guide] trick 2). Holds for any rounding decisions, clipping and groups."""
    W, X = rand_problem(8, 9, 16, 60, relu=True, dead=(3,))
    r = O.gptq_oracle(W, X, bits=3, group=group, act_order=act)
    Qq = r["Q"][:, r["perm"]]
    D = Qq - r["W0"]
    quad = np.einsum("ri,ij,rj->r", D, r["H_p"], D)
    np.testing.assert_allclose(r["loss"], quad, rtol=1e-10)


def test_clipping_propagates_clipped_error():
    """P-15: [guide] 'When it breaks': compensation can push a weight past the row scale; its code is
    clipped to +-qmax and the clipped error is what propagates (err uses the clipped q)."""
    rng = np.random.default_rng(12)
    base = rng.standard_normal((256, 2))
    X = np.column_stack([base[:, 0], 0.5 * base[:, 0] + 0.05 * base[:, 1]])  # H10 / H11 ~ 2
    W = np.array([[0.45, 1.0], [-0.45, -1.0]])  # column 1 holds the row max; column 0 rounds to 0
    r = O.gptq_oracle(W, X, bits=2, damp=0.0)
    assert (np.abs(r["codes"][:, 1]) == 1).all()
    # the update pushed column 1 beyond the grid: w/scale > qmax + 0.5 before clipping
    pre = r["codes"][:, 1] * r["scales"][:, 0] + r["errs"][:, 1] * r["U"][1, 1]
    assert (np.abs(pre / r["scales"][:, 0]) > 1.5).all()
    Qq = r["Q"][:, r["perm"]]
    D = Qq - r["W0"]
    np.testing.assert_allclose(r["loss"], np.einsum("ri,ij,rj->r", D, r["H_p"], D), rtol=1e-10)


# ------------------------------------------------------------------------------------------------
# P-11, P-14: invariances
# ------------------------------------------------------------------------------------------------
def test_power_of_two_scaling_and_row_independence():
    """P-11: scaling X or W by 2^k changes H, U and scales exactly by powers of two, so the codes are
    bitwise identical; rows are independent ([guide] 'How it works': rows share one H)."""
    W, X = rand_problem(31, 12, 20, 80)
    a = O.gptq_oracle(W, X, bits=4, group=5)
    b = O.gptq_oracle(W * 8.0, X * 0.25, bits=4, group=5)
    np.testing.assert_array_equal(a["codes"], b["codes"])
    np.testing.assert_array_equal(a["scales"] * 8.0, b["scales"])
    rows = np.array([7, 2, 11])
    c = O.gptq_oracle(W[rows], X, bits=4, group=5)
    np.testing.assert_array_equal(a["codes"][rows], c["codes"])


def test_duplicated_calibration_set_same_h():
    """P-14: stacking X twice leaves H = 2 X^T X / n unchanged, and so the codes."""
    W, X = rand_problem(41, 5, 12, 50)
    a = O.gptq_oracle(W, X, bits=3)
    b = O.gptq_oracle(W, np.vstack([X, X]), bits=3)
    np.testing.assert_allclose(a["H_p"], b["H_p"], rtol=1e-13)
    np.testing.assert_array_equal(a["codes"], b["codes"])


def test_act_order_equals_explicitly_permuted_problem():
    """[guide] act_order: quantize columns in decreasing diag(X^T X) with U recomputed for that order,
    then restore the original order. Same as running the plain loop on (W[:, perm], X[:, perm])."""
    W, X = rand_problem(51, 6, 14, 70, relu=True, dead=(2, 9))
    X[:, 5] *= 4.0
    r = O.gptq_oracle(W, X, bits=3, group=4, act_order=True)
    perm = r["perm"]
    colsq = (X ** 2).sum(0)
    assert all(colsq[perm[k]] >= colsq[perm[k + 1]] for k in range(13))
    assert perm[0] == 5 and set(perm[-2:]) == {2, 9}  # dead inputs sort last
    p = O.gptq_oracle(W[:, perm], X[:, perm], bits=3, group=4, act_order=False)
    np.testing.assert_array_equal(r["codes"][:, perm], p["codes"])
    np.testing.assert_array_equal(r["g_idx"][perm], np.arange(14) // 4)
    np.testing.assert_allclose(r["Q"][:, perm], p["Q"], rtol=1e-12, atol=0)


def test_act_order_ties_break_by_index():
    colsq = np.array([1.0, 3.0, 1.0, 3.0, 0.0, 2.0])
    assert O.activation_order(colsq).tolist() == [1, 3, 5, 0, 2, 4]


# ------------------------------------------------------------------------------------------------
# P-12, P-13: end to end on the two small workloads
# ------------------------------------------------------------------------------------------------
def test_output_error_gram_form_equals_direct():
    W, X = rand_problem(61, 7, 9, 33)
    r = O.gptq_oracle(W, X, bits=3)
    direct = np.sum((X @ W.T - X @ r["Q"].T) ** 2)
    assert O.output_error(W, r["Q"], r["S"]) == pytest.approx(direct, rel=1e-11)


@pytest.mark.parametrize("name,bits,act", [("tiny", 4, False), ("tiny", 3, False), ("teacher", 3, False),
                                           ("teacher", 2, False), ("teacher", 3, True), ("teacher", 2, True)])
def test_output_error_well_below_rtn(name, bits, act):
    """P-12: [lesson] acceptance check: on X, GPTQ's output error must be clearly lower than that of
    round-to-nearest. The ratio should be near mean(1/U_jj^2) / mean(H_jj) (the variance of x_j left after regressing on the
    inputs not yet quantized, relative to its total variance)."""
    c = syn.config_by_name(name)
    W = O.to_f64(syn.gen_w(c), c.dtype)
    X = O.to_f64(syn.gen_x(c), c.dtype)
    r = O.gptq_oracle(W, X, bits=bits, damp=c.damp, act_order=act)
    _, Q_rtn = O.rtn(W, bits, dead=r["dead"])
    e_g = O.relative_output_error(W, r["Q"], r["S"])
    e_r = O.relative_output_error(W, Q_rtn, r["S"])
    assert e_g < 0.8 * e_r
    live = ~r["dead"][r["perm"]]
    pred = np.mean(1.0 / np.diag(r["U"])[live] ** 2) / np.mean(np.diag(r["H_p"])[live])
    assert abs(e_g / e_r - pred) < 0.15


def test_outputs_consistent():
    """P-13: Q = codes * scales[:, g_idx]; codes in [-qmax, qmax]; dead columns have code 0."""
    c = syn.config_by_name("teacher")
    W = O.to_f64(syn.gen_w(c), c.dtype)
    X = O.to_f64(syn.gen_x(c), c.dtype)
    r = O.gptq_oracle(W, X, bits=3, group=32, act_order=True)
    assert np.abs(r["codes"]).max() <= 3
    assert (r["codes"][:, r["dead"]] == 0).all() and r["dead"].sum() == 13
    np.testing.assert_array_equal(r["Q"], r["codes"] * r["scales"][:, r["g_idx"]])
    assert r["scales"].shape == (256, 8)


def test_forced_replay_accepts_own_codes_and_flags_wrong_ones():
    """The comparison helper: the oracle's own codes are within 0.5 of the unrounded value; a code
    moved by one step is not."""
    W, X = rand_problem(71, 8, 24, 90)
    r = O.gptq_oracle(W, X, bits=4, group=8)
    dist, scales = O.forced_replay(r["W0"], r["U"], 4, 8, r["codes_q"])
    assert dist.max() <= 0.5 + 1e-9
    np.testing.assert_array_equal(scales, r["scales"])
    bad = r["codes_q"].copy()
    bad[3, 10] += 1 if bad[3, 10] < 7 else -1
    dist2, _ = O.forced_replay(r["W0"], r["U"], 4, 8, bad)
    assert dist2[3, 10] > 0.5


# ------------------------------------------------------------------------------------------------
# Inputs
# ------------------------------------------------------------------------------------------------
def test_bf16_encoding_matches_torch_and_is_deterministic():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ours = syn.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    c = syn.config_by_name("down")
    x1 = syn.gen_x(c, 4000, 4100)
    x2 = syn.gen_x(c, 4000, 4100, threads=1)
    np.testing.assert_array_equal(x1, x2)
    assert (syn.gen_x(c, 0, 64)[:, syn.workloads.dead_channels(c)] == 0).all()


def test_bf16_decoding_matches_torch_for_every_pattern():
    """to_f64's bf16 branch against torch's own bf16 -> fp32 widening, for all 65536 bit patterns
    (zeros, subnormals, normals, infinities; NaN patterns must decode to NaN)."""
    torch = pytest.importorskip("torch")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # NaN patterns widen with a warning
        ours = O.to_f64(bits, "bf16")
        ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 127  # exponent all ones, mantissa != 0, either sign
    np.testing.assert_array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint64), ref[~nan].view(np.uint64))  # bitwise, -0.0 included


def test_prepare_reads_the_lower_triangle_of_s():
    """S's lower triangle is authoritative (the library writes only that half): whatever the strictly
    upper half holds, H is built from the lower half mirrored."""
    W, X = rand_problem(81, 3, 9, 40)
    S, colsq, n = O.hessian_from_x(X)
    junk = S.copy()
    junk[np.triu_indices(9, 1)] = np.random.default_rng(2).standard_normal(36) * 1e3
    a = O.prepare(S, colsq, n, 0.01, False)[0]
    b = O.prepare(junk, colsq, n, 0.01, False)[0]
    assert np.array_equal(a, b) and np.array_equal(b, b.T)


# ------------------------------------------------------------------------------------------------
# Noise floor (the oracle against itself with an fp32-accumulated Hessian, or with U in fp32)
# ------------------------------------------------------------------------------------------------
def test_fp32_segment_hessian_is_exact_on_integer_data():
    """Integer-valued X whose segment sums stay below 2^24: every fp32 product and partial sum inside a
    segment is exact, so the fp32-segment S must equal the fp64 S bit for bit (and colsq is the same
    fp64 sum). The totals over all 64 segments pass 2^24, so summing the segments in fp32 would not be
    exact: the segments must be combined in fp64."""
    rng = np.random.default_rng(23)
    X = rng.integers(-31, 32, size=(64 * 2048 + 5, 12)).astype(np.float64)  # |segment sum| <= 2048*961 < 2^24
    S64, c64, n64 = O.hessian_from_x(X)
    S32, c32, n32 = O.hessian_from_x(X, fp32_segments=True)
    assert n64 == n32 == X.shape[0]
    assert np.diag(S64).min() > 2.0 ** 24
    assert np.array_equal(S64, S32) and np.array_equal(c64, c32)


def test_fp32_segment_hessian_error_is_fp32_sized():
    """On N(0,1) data the fp32-segment S differs from the fp64 S, and every entry stays inside the
    floating-point dot-product bound for m = 2048 fp32 terms per segment,
    |dS_ij| <= gamma_m sum_k |x_ki x_kj|, gamma_m = m u / (1 - m u), u = 2^-24 (plus fp64 rounding).
    Its typical relative size is near 1e-7 (a few fp32 ulps)."""
    rng = np.random.default_rng(29)
    X = rng.standard_normal((3 * 2048 + 111, 16)).astype(np.float32).astype(np.float64)
    S64, _, _ = O.hessian_from_x(X)
    S32, _, _ = O.hessian_from_x(X, fp32_segments=True)
    A = np.abs(X).T @ np.abs(X)
    u, m = 2.0 ** -24, 2048
    gamma = m * u / (1 - m * u)
    dS = np.abs(S32 - S64)
    assert (dS <= gamma * A + 1e-12 * A).all()
    rel = dS / np.sqrt(np.outer(np.diag(S64), np.diag(S64)))
    assert 1e-9 < np.median(rel[np.tril_indices(16)]) < 1e-5
    assert rel.max() > 0.0


def test_fp32_segment_hessian_rejects_wider_inputs():
    with pytest.raises(ValueError):
        O.hessian_from_x(np.full((4, 2), 0.1), fp32_segments=True)


def test_u_rounded_to_fp32_is_within_half_an_fp32_ulp():
    W, X = rand_problem(83, 4, 20, 60)
    S, colsq, n = O.hessian_from_x(X)
    r64 = O.gptq_oracle(W, hessian=(S, colsq, n))
    r32 = O.gptq_oracle(W, hessian=(S, colsq, n), u_round=np.float32)
    nz = r64["U"] != 0
    assert np.all(np.abs(r32["U"][nz] - r64["U"][nz]) <= 2.0 ** -24 * np.abs(r64["U"][nz]))
    assert np.array_equal(r32["U"][~nz], r64["U"][~nz])
    assert np.array_equal(r32["U"].astype(np.float32).astype(np.float64), r32["U"])


def test_noise_floor_is_zero_when_the_fp32_sums_are_exact():
    """The floor measures the oracle against itself: with integer data the fp32-segment mode reproduces
    the fp64 run exactly (no drift), while the fp32-U mode still perturbs U."""
    rng = np.random.default_rng(31)
    X = rng.integers(-3, 4, size=(3000, 32)).astype(np.float64)
    X = X @ (np.eye(32, dtype=np.int64) + np.eye(32, k=1, dtype=np.int64))  # correlated, still integral
    W = 0.05 * rng.standard_normal((40, 32))
    S64, colsq, n = O.hessian_from_x(X)
    S32, _, _ = O.hessian_from_x(X, fp32_segments=True)
    fl = O.noise_floor(W, S64, S32, colsq, n, 3, 8, 0.01, True)
    assert fl["fp32_segment_S"] == dict(f=0.0, mismatches=0, q_rel=0.0, out_rel=0.0)
    ref = O.gptq_oracle(W, X, bits=3, group=8, act_order=True)
    assert np.array_equal(fl["ref"]["codes"], ref["codes"])
    assert fl["fp32_U"]["f"] <= 0.01


def test_fp32_chain_model_equals_scalar_loop_and_is_exact_on_integers():
    """The plain fp32 accumulation model against a brute-force loop of numpy float32 scalars: per chain,
    run = float32(run + exact sum of the group's 16 products), chains summed in fp64. Bitwise on a tiny
    block with ragged chains and groups; exact on integer data (no rounding happens at all)."""
    rng = np.random.default_rng(37)
    X = rng.standard_normal((101, 3)).astype(np.float32).astype(np.float64)
    got = O.fp32_chain_block(X, X, chain_rows=48, group_rows=16)
    want = np.zeros((3, 3))
    for i in range(3):
        for j in range(3):
            total = 0.0
            for c0 in range(0, 101, 48):
                run = np.float32(0.0)
                for g0 in range(c0, min(101, c0 + 48), 16):
                    exact = sum(Fraction(float(X[k, i])) * Fraction(float(X[k, j])) for k in range(g0, min(101, c0 + 48, g0 + 16)))
                    run = np.float32(float(Fraction(float(run)) + exact))  # one rounding of the exact step
                total += float(run)
            want[i, j] = total
    assert np.array_equal(got, want)
    Xi = rng.integers(-9, 10, size=(3000, 20)).astype(np.float64)
    S64, c64, _ = O.hessian_from_x(Xi)
    S, c = np.zeros((20, 20)), np.zeros(20)
    O.accumulate_fp32_chains(S, c, Xi, chain_rows=1024, tile=8)
    low = np.tril_indices(20)
    assert np.array_equal(S[low], S64[low]) and np.array_equal(c, c64)
    assert np.all(S[np.triu_indices(20, 1)] == 0.0)


def test_fp32_chain_model_error_is_within_the_sequential_bound():
    """Each step rounds once to fp32, so |S_chain - S| <= u * sum over steps of |running value| (u = 2^-24,
    plus the fp64 sums); on N(0,1) data the error is not zero and grows with the chain length."""
    rng = np.random.default_rng(41)
    X = rng.standard_normal((4096, 8)).astype(np.float32).astype(np.float64)
    S64 = X.T @ X
    errs = {}
    for chain in (256, 4096):
        Sc = O.fp32_chain_block(X, X, chain_rows=chain)
        bound = np.zeros((8, 8))
        for c0 in range(0, 4096, chain):
            part = np.cumsum(np.einsum("ki,kj->kij", X[c0:c0 + chain], X[c0:c0 + chain]).reshape(-1, 16, 8, 8).sum(1), axis=0)
            bound += np.abs(part).sum(0)
        dS = np.abs(Sc - S64)
        assert (dS <= 2.0 ** -24 * bound * (1 + 1e-6) + 1e-12).all()
        assert dS.max() > 0
        errs[chain] = np.median(dS / np.sqrt(np.outer(np.diag(S64), np.diag(S64))))
    assert errs[4096] > errs[256]
