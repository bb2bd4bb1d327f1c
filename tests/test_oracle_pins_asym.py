"""Pins for the oracle's asymmetric grid (min/max plus a zero point), CPU only.

The quantizer is the handbook's ("quantize_weight", "dequantize_weight" and the group parameters of
"gptq_quantize_row"); the guide's "Simplifications" names it the paper's default. The loop around it is
the one the symmetric pins already fix. These pins fix the grid itself by closed forms and hand values,
the loop by an exact rational run, and the limits where GPTQ must equal round-to-nearest.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import gptq_oracle as O
import synthetic as syn
from tests.test_oracle_pins import rand_problem


# ------------------------------------------------------------------------------------------------
# The grid: hand values and closed forms
# ------------------------------------------------------------------------------------------------
def test_grid_hand_values():
    """Three rows worked by hand at 2 bits (levels 0..3).
    [-1.5, 0, 3]: scale 4.5/3 = 1.5, zero round(1.5/1.5) = 1; codes round(w/1.5 + 1) = 0, 1, 3.
    [2.5, 2.5, 2.5]: max = min, so scale 1; zero clip(round(-2.5)) = 0; round(2.5) ties to even = 2.
    [1, 2, 4]: scale 1, zero clip(round(-1)) = 0; 4 saturates at 3 (all-positive group)."""
    B = np.array([[-1.5, 0.0, 3.0], [2.5, 2.5, 2.5], [1.0, 2.0, 4.0]])
    s, z = O.asym_params(B, 2)
    np.testing.assert_array_equal(s, [1.5, 1.0, 1.0])
    np.testing.assert_array_equal(z, [1.0, 0.0, 0.0])
    c = O.asym_code(B, s[:, None], z[:, None], 2)
    np.testing.assert_array_equal(c, [[0, 1, 3], [2, 2, 2], [1, 2, 3]])
    np.testing.assert_array_equal(O.asym_value(c, s[:, None], z[:, None]), [[-1.5, 0, 3], [2, 2, 2], [1, 2, 3]])


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_grid_end_points_and_half_step_bound(bits):
    """When -min/scale is an integer (zero not clipped), min maps to code 0, max to 2^bits - 1, and every
    weight in [min, max] comes back within scale/2."""
    rng = np.random.default_rng(bits)
    L = 2 ** bits - 1
    for _ in range(20):
        scale = rng.uniform(0.01, 2.0)
        z = int(rng.integers(1, L))
        lo, hi = -z * scale, (L - z) * scale
        w = np.concatenate([[lo, hi], rng.uniform(lo, hi, 50)])[None, :]
        s, zz = O.asym_params(w, bits)
        assert abs(s[0] - scale) <= 1e-12 * scale and zz[0] == z
        c = O.asym_code(w, s[:, None], zz[:, None], bits)
        assert c[0, 0] == 0 and c[0, 1] == L
        assert np.abs(w - O.asym_value(c, s[:, None], zz[:, None])).max() <= 0.5 * s[0] * (1 + 1e-9)


def test_levels_and_bits():
    assert [O.asym_levels(b) for b in (2, 3, 4, 8)] == [3, 7, 15, 255]
    with pytest.raises(ValueError):
        O.asym_levels(1)


# ------------------------------------------------------------------------------------------------
# The loop: exact rational run, limits, identities
# ------------------------------------------------------------------------------------------------
def _exact_asym(W, X, bits, group, damp):
    """Exact rational GPTQ with the asymmetric grid: H, dead fix, damping, H^-1 by Gauss-Jordan, then
    per row the OBS step and elimination, rounding half to even on exact values."""
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
    L = 2 ** bits - 1

    def params(vals):
        lo, hi = min(vals), max(vals)
        s = (hi - lo) / L if hi > lo else Fraction(1)
        return s, min(max(round(-lo / s), 0), L)

    codes = []
    for wrow in W:
        w = [Fraction(0) if dead[i] else Fraction(float(v)) for i, v in enumerate(wrow)]
        Hi = [row[:] for row in Hinv]
        s, z = params(w)
        crow = []
        for j in range(d):
            if group and j % group == 0:
                s, z = params(w[j:j + group])
            c = min(max(round(w[j] / s + z), 0), L)
            crow.append(c)
            e = w[j] - s * (c - z)
            f = e / Hi[j][j]
            w = [w[k] - f * Hi[j][k] for k in range(d)]
            Hi = [[Hi[a][b] - Hi[a][j] * Hi[j][b] / Hi[j][j] for b in range(d)] for a in range(d)]
        codes.append(crow)
    return np.array(codes, dtype=np.int64), np.array(dead)


@pytest.mark.parametrize("seed", range(12))
def test_loop_matches_exact_rational_obs_asym(seed):
    """The fp64 Cholesky-form loop with the asymmetric grid makes the codes of an exact rational
    OBS/elimination run (per-row and grouped parameters, dead inputs)."""
    rng = np.random.default_rng(311 + seed)
    d = int(rng.integers(1, 6))
    out = int(rng.integers(1, 4))
    bits = int(rng.integers(2, 5))
    group = int(rng.choice([0, 1, 2, d]))
    W, X = rand_problem(900 + seed, out, d, d + 3, dead=(0,) if (seed % 4 == 1 and d > 1) else ())
    r = O.gptq_oracle_asym(W, X, bits=bits, group=group, damp=0.01)
    ex_codes, ex_dead = _exact_asym(W, X, bits, group, 0.01)
    np.testing.assert_array_equal(r["dead"], ex_dead)
    np.testing.assert_array_equal(r["codes_q"], ex_codes)


@pytest.mark.parametrize("seed", range(4))
def test_group_params_from_updated_weights_exact_asym(seed):
    """With groups, each group's (scale, zero) comes from its weights as the earlier steps have updated
    them (the handbook's per-column loop; the guide's "The code, line by line" for the scale). Exact
    rational run with three groups per row and strongly coupled inputs, so that the updates move each
    later group's min and max."""
    W, X = rand_problem(940 + seed, 3, 6, 9)
    X[:, 1] += 2.0 * X[:, 0]
    X[:, 3] -= 1.5 * X[:, 2]
    r = O.gptq_oracle_asym(W, X, bits=2, group=2, damp=0.01)
    ex_codes, _ = _exact_asym(W, X, 2, 2, 0.01)
    np.testing.assert_array_equal(r["codes_q"], ex_codes)


@pytest.mark.parametrize("bits,group", [(3, 0), (4, 0), (3, 32)])
def test_heavy_damping_is_rtn_asym(bits, group):
    """Heavy damping makes H a multiple of I: nothing is pushed and the asymmetric GPTQ codes are the
    asymmetric round-to-nearest codes (parameters from the starting weights in both)."""
    c = syn.config_by_name("teacher")
    W = O.to_f64(syn.gen_w(c), c.dtype)
    X = O.to_f64(syn.gen_x(c), c.dtype)
    r = O.gptq_oracle_asym(W, X, bits=bits, group=group, damp=1e6)
    codes_rtn, Q_rtn = O.rtn_asym(W, bits, group, dead=r["dead"])
    np.testing.assert_array_equal(r["codes"], codes_rtn)


def test_orthogonal_inputs_are_rtn_asym():
    """Diagonal H gives U[j, j+1:] = 0: no error moves and GPTQ equals RTN on the same grid."""
    rng = np.random.default_rng(19)
    Qm, _ = np.linalg.qr(rng.standard_normal((64, 8)))
    X = Qm * rng.uniform(0.5, 3.0, 8)
    W = rng.standard_normal((5, 8))
    for group in (0, 4):
        r = O.gptq_oracle_asym(W, X, bits=3, group=group)
        np.testing.assert_array_equal(r["codes"], O.rtn_asym(W, 3, group)[0])


@pytest.mark.parametrize("group,act", [(0, False), (4, False), (4, True)])
def test_loss_identity_asym(group, act):
    """sum_j err_j^2 = (q - w0) H_p (q - w0)^T holds for any rounding rule, this grid included."""
    W, X = rand_problem(28, 9, 16, 60, relu=True, dead=(3,))
    r = O.gptq_oracle_asym(W, X, bits=3, group=group, act_order=act)
    D = r["Q"][:, r["perm"]] - r["W0"]
    quad = np.einsum("ri,ij,rj->r", D, r["H_p"], D)
    np.testing.assert_allclose(r["loss"], quad, rtol=1e-10)


def test_outputs_consistent_asym():
    """Codes in 0..2^b-1, zeros integral and inside the levels, Q = scale (code - zero) through g_idx,
    the loop's own codes replay with distance <= 0.5 and a moved code is flagged."""
    W, X = rand_problem(31, 6, 12, 50, relu=True, dead=(5,))
    r = O.gptq_oracle_asym(W, X, bits=3, group=4, act_order=True)
    assert r["codes"].min() >= 0 and r["codes"].max() <= 7
    assert np.array_equal(r["zeros"], np.round(r["zeros"])) and r["zeros"].min() >= 0 and r["zeros"].max() <= 7
    Q = r["scales"][:, r["g_idx"]] * (r["codes"] - r["zeros"][:, r["g_idx"]])
    np.testing.assert_array_equal(Q, r["Q"])
    dist = O.forced_replay_asym(r["W0"], r["U"], 3, 4, r["codes_q"])
    assert dist.max() <= 0.5 + 1e-12
    bad = r["codes_q"].copy()
    bad[2, 5] = (bad[2, 5] + 2) % 8
    assert O.forced_replay_asym(r["W0"], r["U"], 3, 4, bad).max() > 0.5


@pytest.mark.parametrize("bits", [2, 3])
def test_output_error_below_rtn_asym(bits):
    """On the 256-input teacher-like layer the asymmetric GPTQ output error is well below RTN's on the
    same grid (the pages' headline claim for the method, here for the paper's default quantizer)."""
    c = syn.config_by_name("teacher")
    W = O.to_f64(syn.gen_w(c), c.dtype)
    X = O.to_f64(syn.gen_x(c), c.dtype)
    r = O.gptq_oracle_asym(W, X, bits=bits)
    _, Q_rtn = O.rtn_asym(W, bits, dead=r["dead"])
    e_g = O.relative_output_error(W, r["Q"], r["S"])
    e_r = O.relative_output_error(W, Q_rtn, r["S"])
    assert e_g < 0.8 * e_r, (e_g, e_r)
