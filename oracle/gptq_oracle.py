"""CPU oracle for GPTQ per-layer quantization (numpy, fp64). TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke entry and the benchmark's CPU-baseline leg may import this module.
The GPU library never calls it, and this module imports nothing from the GPU package.

Sources (three web pages on GPTQ):
  [lesson]   "GPTQ's error-compensation loop" (Lesson 10 of 10), herodthegreater.github.io/pigeon/school/gptq_loop/
  [handbook] "GPTQ > Implementation with AutoGPTQ", mbrenndoerfer.com/writing/gptq-4bit-weight-quantization-llm-guide/
  [guide]    "GPTQ", herodthegreater.github.io/pigeon/guide/gptq/

What is computed. GPTQ is a greedy, sequential rounding rule, so the oracle carries out its steps in the
pages' order; where a step has a closed definition (X^T X, the factor U) the oracle evaluates that
definition directly.
  1. the curvature of the layer's squared output error, H = 2 X^T X / n    ([guide] "The idea")
  2. inputs that never fire (zero diagonal) are "dead": H_ii = 1, their weights are zeroed
                                                                          ([guide] "The code, line by line")
  3. damping: damp * mean(diag H) is added to every diagonal entry       ([guide] "How it works", Damping)
  4. optional act_order: inputs taken in decreasing diag(X^T X)          ([guide] "The code, line by line")
  5. U, the upper-triangular factor with positive diagonal and U^T U = H^-1
                                                                          ([guide] "GPTQ's two tricks", trick 2)
  6. every row of W is swept once over the positions j = 0..in-1 (rows are independent and share U,
     [guide] "How it works"). At position j the current weight is snapped to the grid; the residual,
     divided by the pivot U[j, j], is the row's step error, and the not-yet-quantized positions
     absorb step error times U[j, j+1:]. This is the optimal-brain-surgeon update with the inverse
     Hessian of the remaining positions expressed through U ([guide] trick 2; [lesson] statement).
     The grid is fitted once per row to the starting weights, or, with groups, afresh at each group's
     first position to that group's weights as updated so far ([guide] "The code, line by line").
     Snapping clips to the grid, so the clipped residual is what is pushed on ([guide] "When it breaks").
  7. codes go back to the original column order; g_idx maps a column to its group ([guide] "When it breaks")
  8. the same sweep on the asymmetric grid (levels 0..2^b-1 with a zero point)
     ([guide] "Simplifications"; [handbook] quantize_weight, dequantize_weight, gptq_quantize_row)
  9. storage and use: packed codes, Q from codes and grid parameters, the layer-wise driver
     ([guide] "When it breaks", "How it works" apply_layerwise; [handbook] int4 storage)
 10. the noise floor: the oracle re-run with its Hessian summed in fp32 (per 2048-row segment by a BLAS
     product, or as plain sequential fp32 chains), and with U rounded to fp32, measured against itself
     (how far an fp32-accumulated Hessian alone moves the result; the calibration set is 128 segments of
     2048 tokens, [guide] "How it works").

Readings where the pages leave a detail open (each is also listed with the build's design notes):
  * qmax for b bits is 2^(b-1) - 1 (the lesson's starter code; "2-bit" = ternary {-s, 0, s} in the guide).
  * rounding is to nearest with ties to even (numpy's rule); dead = colsq == 0 exactly, decided in fp64.
  * H[dead, dead] = 1 touches only the diagonal (numpy pairs the two boolean index arrays).
  * damping uses the mean diagonal after the dead fix; the normalisation is 2/n (not the handbook's 2).
  * S's lower triangle is the authoritative copy: H[i][j] = H[j][i] = 2/n S[max(i,j)][min(i,j)].
  * act_order key is diag(X^T X) before the dead fix; ties are broken by the lower original index.
  * U for the permuted problem equals the factor of P^T H P (dead fix and damping commute with P).
  * g_idx[perm[j]] = j // group: groups are formed in quantization order.
  * Output error of a quantized layer is ||X (W - Q)^T||_F^2, relative to ||X W^T||_F^2 ([guide] simulations).
  * Asymmetric grid: min/max over the weights themselves (0 is not forced into the range); the zero point
    is clipped to the levels, so a group of all-positive (or all-negative) weights saturates at one end,
    as the handbook's formulas do. Per-row mode takes (scale, zero) from the starting weights, groups
    from the current weights at the group start (the handbook's per-column loop does the latter).
  * Packed layout (the pages fix none): per row a little-endian bit stream of b-bit codes in 32-bit
    words, symmetric codes offset by 2^(b-1). The driver's F is float32; an MLP layer is affine + ReLU
    (no ReLU on the output layer); layer outputs are the exact values rounded once to fp32.
  * Noise floor: "fp32 accumulation" is modelled two ways. (a) One single-precision BLAS product per
    2048-row segment (the order of its sums is the library's), segments summed in fp64. (b) The plainest
    form: a sequential fp32 running sum over a chain of rows, taking 16 rows at a time with one rounding
    per step, chains summed in fp64. colsq stays fp64 in both.
"""
from __future__ import annotations

import numpy as np

HESSIAN_CHUNK_ROWS = 2048
SCALE_FLOOR = 1e-12  # [guide] "The code, line by line": per-row scale floor


# ---------------------------------------------------------------------------------------------
# Input decoding (the oracle reads the same stored bits as the GPU, widened exactly to fp64)
# ---------------------------------------------------------------------------------------------
def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 array or bf16 bit patterns (uint16) -> fp64, exactly: a bf16 value is the upper half of the
    fp32 value with the same bits, so shifting the pattern up 16 bits gives that fp32 value."""
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------------------------
# Step 1: Hessian accumulation
# ---------------------------------------------------------------------------------------------
def accumulate(S: np.ndarray, colsq: np.ndarray, X64: np.ndarray) -> int:
    """S += X^T X and colsq += sum of squares per column, in fp64; returns the rows added.

    [guide] "The idea": H = 2 X^T X / n over the n calibration inputs (rows of X). The handbook's
    compute_hessian flattens (samples, seq, hidden) inputs to (tokens, hidden) first, so n counts tokens.
    The sum is taken over 2048-row chunks; colsq is the diagonal of X^T X kept on its own (it is the
    act_order key and the exact dead test).
    """
    n = X64.shape[0]
    for r0 in range(0, n, HESSIAN_CHUNK_ROWS):
        blk = X64[r0:r0 + HESSIAN_CHUNK_ROWS]
        S += blk.T @ blk
        colsq += np.einsum("ki,ki->i", blk, blk)
    return n


def accumulate_fp32_segments(S: np.ndarray, colsq: np.ndarray, X64: np.ndarray,
                             seg_rows: int = HESSIAN_CHUNK_ROWS) -> int:
    """The noise-floor variant of accumulate: each segment's X^T X is one single-precision product
    (fp32 sums), then added to S in fp64. The inputs must be fp32-representable (bf16 or fp32 data),
    so only the sums are rounded differently. colsq is kept in fp64 as in accumulate."""
    n = X64.shape[0]
    for r0 in range(0, n, seg_rows):
        blk = X64[r0:r0 + seg_rows]
        b32 = blk.astype(np.float32)
        if not np.array_equal(b32.astype(np.float64), blk):
            raise ValueError("inputs are not fp32-representable")
        S += (b32.T @ b32).astype(np.float64)
        colsq += np.einsum("ki,ki->i", blk, blk)
    return n


def fp32_chain_block(XI: np.ndarray, XJ: np.ndarray, chain_rows: int = 4096, group_rows: int = 16) -> np.ndarray:
    """One block XI^T XJ under the plainest fp32 accumulation (the second noise-floor model): within each
    chain of `chain_rows` rows, an fp32 running sum takes one group of `group_rows` rows at a time, each
    step rounded to fp32 (the running value plus the group's sum of products, formed in fp64, where the
    products of fp32-representable inputs and their short sums are exact); the chains' sums are added in
    fp64. XI, XJ: the same rows, fp32-representable values widened to fp64."""
    out = np.zeros((XI.shape[1], XJ.shape[1]))
    step = np.empty_like(out)
    run = np.empty(out.shape, dtype=np.float32)
    for c0 in range(0, XI.shape[0], chain_rows):
        run.fill(0.0)
        for g0 in range(c0, min(XI.shape[0], c0 + chain_rows), group_rows):
            np.matmul(XI[g0:g0 + group_rows].T, XJ[g0:g0 + group_rows], out=step)
            np.add(step, run, out=step)
            np.copyto(run, step, casting="same_kind")
        out += run
    return out


def accumulate_fp32_chains(S: np.ndarray, colsq: np.ndarray, X64: np.ndarray, chain_rows: int = 4096,
                           group_rows: int = 16, tile: int = 256) -> int:
    """S (lower triangle) += X^T X under fp32_chain_block, tile by tile (the tiling only keeps a tile of
    the running sum in cache; every entry sees the same operations). colsq += column sums of squares in
    fp64. The inputs must be fp32-representable. The strictly upper triangle of S is left as it was."""
    n, d = X64.shape
    if not np.array_equal(X64.astype(np.float32).astype(np.float64), X64):
        raise ValueError("inputs are not fp32-representable")
    for i0 in range(0, d, tile):
        for j0 in range(0, i0 + 1, tile):
            blk = fp32_chain_block(X64[:, i0:i0 + tile], X64[:, j0:j0 + tile], chain_rows, group_rows)
            dst = S[i0:i0 + tile, j0:j0 + tile]
            if i0 == j0:
                low = np.tril(np.ones(blk.shape, dtype=bool))
                dst[low] += blk[low]
            else:
                dst += blk
    colsq += np.einsum("ki,ki->i", X64, X64)
    return n


def hessian_from_x(X64: np.ndarray, fp32_segments: bool = False):
    d = X64.shape[1]
    S = np.zeros((d, d))
    colsq = np.zeros(d)
    n = (accumulate_fp32_segments if fp32_segments else accumulate)(S, colsq, X64)
    return S, colsq, n


# ---------------------------------------------------------------------------------------------
# Step 2-4: H, dead inputs, damping, column order
# ---------------------------------------------------------------------------------------------
def activation_order(colsq: np.ndarray) -> np.ndarray:
    """Columns by decreasing diag(X^T X); equal keys keep increasing index ([guide] act_order)."""
    return np.argsort(-colsq, kind="stable")


def prepare(S: np.ndarray, colsq: np.ndarray, n: int, damp: float, act_order: bool):
    """Returns (H_p, perm, dead, lam): the damped Hessian in quantization order and its metadata.

    [guide] "The code, line by line", _hessian_inverse_chol: H = 2 X^T X / n; inputs whose diagonal
    is zero are dead and get H_ii = 1; then 0.01 * mean(diag H) is added to the diagonal.
    [guide] act_order: perm sorts by decreasing diag(X^T X), and U is recomputed for the permuted
    inputs, i.e. for P^T H P. S's lower triangle is read (its upper triangle may be stale).
    """
    if n < 1:
        raise ValueError("n must be >= 1")
    d = S.shape[0]
    lower = np.tril(S)
    H = (2.0 / n) * (lower + np.tril(S, -1).T)
    dead = colsq == 0.0
    idx = np.flatnonzero(dead)
    H[idx, idx] = 1.0
    lam = damp * np.mean(np.diag(H))
    H[np.arange(d), np.arange(d)] += lam
    perm = activation_order(colsq) if act_order else np.arange(d)
    H_p = H[np.ix_(perm, perm)]
    return H_p, perm, dead, lam


# ---------------------------------------------------------------------------------------------
# Step 5: U, the upper Cholesky factor of H^-1
# ---------------------------------------------------------------------------------------------
def upper_factor_of_inverse(H_p: np.ndarray) -> np.ndarray:
    """The definition ([guide] trick 2): U upper-triangular with a positive diagonal and U^T U = H^-1.

    H^-1 is formed, its lower Cholesky factor L (H^-1 = L L^T) taken, and U = L^T. U is unique, so any
    other route to it (the tests use one without an explicit inverse) must agree. Raises
    numpy.linalg.LinAlgError when H is not positive definite.
    """
    Hinv = np.linalg.inv(H_p)
    L = np.linalg.cholesky(Hinv)
    return np.ascontiguousarray(L.T)


def r_form(H_p: np.ndarray, panel: int = 128) -> np.ndarray:
    """The factor in the form the second quantize route of the library reads (a layout, not a step of the
    pages): R = U^-1, upper-triangular with R R^T = H (so J R J is the lower Cholesky factor of J H J, J the
    index reversal), in the upper triangle, diagonal included; and for each run of `panel` columns
    [b, b + p) the strictly lower part of that diagonal block holding J U_bb J, U_bb = R_bb^-1 being U's
    diagonal block. Written from the definitions with numpy's Cholesky factor and inverse.
    """
    d = H_p.shape[0]
    rev = np.arange(d)[::-1]
    R = np.linalg.cholesky(H_p[np.ix_(rev, rev)])[np.ix_(rev, rev)]
    M = np.triu(R)
    for b in range(0, d, panel):
        p = min(panel, d - b)
        U_bb = np.linalg.inv(R[b:b + p, b:b + p])
        M[b:b + p, b:b + p] += np.tril(U_bb[::-1, ::-1], -1)
    return M


# ---------------------------------------------------------------------------------------------
# Grids: fitting a grid to a run of weights, snapping a weight to it, and the snapped value
# ---------------------------------------------------------------------------------------------
def qmax_for(bits: int) -> int:
    """Largest code of the symmetric grid {-qmax..qmax}: 2^(bits-1) - 1 ([lesson] starter code)."""
    if bits < 2:
        raise ValueError("bits must be >= 2")
    return 2 ** (bits - 1) - 1


def row_scales(Wblock: np.ndarray, qmax: int) -> np.ndarray:
    """Symmetric grid step of each row of a block of columns: max(max|w|, 1e-12) / qmax
    ([guide] "The code, line by line"). Reduces over the last axis (a 1-D run gives a scalar)."""
    if Wblock.shape[-1] == 0:
        return np.full(Wblock.shape[:-1], SCALE_FLOOR / qmax)
    return np.maximum(np.abs(Wblock).max(axis=-1), SCALE_FLOOR) / qmax


def sym_code(w, scale, qmax: int):
    """Nearest grid point, ties to even, clipped to -qmax..qmax."""
    return np.minimum(np.maximum(np.rint(w / scale), -qmax), qmax)


def sym_value(c, scale):
    return c * scale


# [guide] "Simplifications": the paper's default quantizer is asymmetric, min/max plus a zero point.
# [handbook] "quantize_weight" / "dequantize_weight" and the group parameters in "gptq_quantize_row" give
# the formulas: levels 0 .. 2^bits - 1; over a group's current weights, scale = (max - min) / (2^bits - 1)
# when max > min and 1 otherwise; zero = round(-min / scale) clipped to the levels; a weight's code is
# round(w / scale + zero) clipped to the levels, and its value is scale * (code - zero). Python's round
# rounds half to even, as numpy's does.
def asym_levels(bits: int) -> int:
    """Largest code of the asymmetric grid {0..2^bits - 1}."""
    if bits < 2:
        raise ValueError("bits must be >= 2")
    return 2 ** bits - 1


def asym_params(Wblock: np.ndarray, bits: int):
    """Per-row (scale, zero) of a block of columns ([handbook] group parameters); last axis reduced."""
    levels = asym_levels(bits)
    wmin = Wblock.min(axis=-1)
    wmax = Wblock.max(axis=-1)
    scale = np.where(wmax > wmin, (wmax - wmin) / levels, 1.0)
    zero = np.minimum(np.maximum(np.rint(-wmin / scale), 0), levels)
    return scale, zero


def asym_code(w, scale, zero, bits: int):
    """round(w / scale + zero) clipped to 0 .. 2^bits - 1 ([handbook] quantize_weight)."""
    return np.minimum(np.maximum(np.rint(w / scale + zero), 0), asym_levels(bits))


def asym_value(c, scale, zero):
    """scale * (code - zero) ([handbook] dequantize_weight)."""
    return scale * (c - zero)


class SymmetricGrid:
    """Codes -qmax..qmax, value code * scale. Parameters of a run of weights: (scale, 0)."""
    asymmetric = False

    def __init__(self, bits: int):
        self.bits = bits
        self.top = qmax_for(bits)

    def fit(self, run):
        return row_scales(run, self.top), 0.0

    def snap(self, w, p):
        return sym_code(w, p[0], self.top)

    def value(self, c, p):
        return sym_value(c, p[0])

    def offset(self, w, c, p):
        """How far code c is from the unrounded (clipped) position of w on the grid; <= 0.5 for a code
        that rounding could have produced."""
        return np.abs(np.minimum(np.maximum(w / p[0], -self.top), self.top) - c)


class AsymmetricGrid:
    """Codes 0..2^b-1, value scale * (code - zero). Parameters of a run of weights: (scale, zero)."""
    asymmetric = True

    def __init__(self, bits: int):
        self.bits = bits
        self.top = asym_levels(bits)

    def fit(self, run):
        return asym_params(run, self.bits)

    def snap(self, w, p):
        return asym_code(w, p[0], p[1], self.bits)

    def value(self, c, p):
        return asym_value(c, p[0], p[1])

    def offset(self, w, c, p):
        return np.abs(np.minimum(np.maximum(w / p[0] + p[1], 0), self.top) - c)


# ---------------------------------------------------------------------------------------------
# Step 6: the error-compensation sweep of one row
# ---------------------------------------------------------------------------------------------
def _grid_source(w_now: np.ndarray, w_start: np.ndarray, j: int, group: int):
    """The weights that set the grid from position j on, or None to keep the current grid.

    Per-row grid: the whole starting row, fitted once at j = 0. Groups: at the first position of each
    group, that group's weights as every earlier step has left them ([guide] "The code, line by line").
    """
    if group:
        return w_now[j:j + group] if j % group == 0 else None
    return w_start if j == 0 else None


def _step_error(residual, pivot):
    """The step error: the snapped weight's residual over the pivot U[j, j]. In OBS terms the
    compensation of the remaining positions is -(residual / H_F^-1[j, j]) H_F^-1[j, :], and with
    H_F^-1[j, :] = U[j, j] U[j, :] this is -(residual / U[j, j]) U[j, :] ([guide] trick 2)."""
    return residual / pivot


def _propagate(w: np.ndarray, j: int, eps, U: np.ndarray) -> None:
    """The positions after j absorb the compensation: w[k] -= eps * U[j, k] for k > j."""
    w[j + 1:] -= eps * U[j, j + 1:]


def sweep_row(w_start: np.ndarray, U: np.ndarray, grid, group: int = 0, forced=None):
    """One row of the layer through positions j = 0..d-1 (quantization order).

    w_start: the row's starting weights (dead inputs zeroed, in quantization order).
    forced:  None to snap each weight to the nearest grid point, or the codes to take instead (a replay
             of another run's decisions).
    Returns (codes int64[d], grid parameters of each group in order, step errors float[d], offsets) where
    offsets[j] is grid.offset of the weight at step j and its code (None unless forced).
    """
    w = np.array(w_start, dtype=np.float64, copy=True)
    d = w.shape[0]
    codes = np.zeros(d, dtype=np.int64)
    eps = np.zeros(d)
    offsets = None if forced is None else np.zeros(d)
    fits = []
    p = None
    for j in range(d):
        src = _grid_source(w, w_start, j, group)
        if src is not None:
            p = grid.fit(src)
            fits.append(p)
        x = w[j]
        c = grid.snap(x, p) if forced is None else float(forced[j])
        if offsets is not None:
            offsets[j] = grid.offset(x, c, p)
        e = _step_error(x - grid.value(c, p), U[j, j])
        codes[j] = int(c)
        eps[j] = e
        _propagate(w, j, e, U)
    return codes, fits, eps, offsets


def sweep_layer(W0: np.ndarray, U: np.ndarray, grid, group: int = 0, forced_codes_q=None):
    """sweep_row for every row. Returns codes (out x d), params (out x G x 2), errs (out x d), loss
    (per row, sum of step errors squared) and offsets (out x d, or None)."""
    out, d = W0.shape
    n_groups = -(-d // group) if group else 1
    codes = np.zeros((out, d), dtype=np.int64)
    params = np.zeros((out, n_groups, 2))
    errs = np.zeros((out, d))
    offsets = None if forced_codes_q is None else np.zeros((out, d))
    for r in range(out):
        forced = None if forced_codes_q is None else forced_codes_q[r]
        c, fits, e, off = sweep_row(W0[r], U, grid, group, forced)
        codes[r], errs[r] = c, e
        params[r] = np.array([[float(a), float(b)] for a, b in fits])
        if off is not None:
            offsets[r] = off
    loss = np.einsum("rj,rj->r", errs, errs)
    return codes, params, errs, loss, offsets


def start_weights(W64: np.ndarray, perm: np.ndarray, dead: np.ndarray) -> np.ndarray:
    """Working copy: dead input columns zeroed, then columns in quantization order ([guide] source)."""
    W0 = np.array(W64, dtype=np.float64, copy=True)
    W0[:, dead] = 0.0
    return W0[:, perm]


def compensation_loop(W0: np.ndarray, U: np.ndarray, bits: int, group: int = 0):
    """The sweep on the symmetric grid for all rows. Returns codes (int64, quantization order), scales
    (out x G, G = ceil(in/group) or 1), errs (the step error of every position) and loss (per row)."""
    codes, params, errs, loss, _ = sweep_layer(W0, U, SymmetricGrid(bits), group)
    return codes, params[:, :, 0].copy(), errs, loss


def compensation_loop_asym(W0: np.ndarray, U: np.ndarray, bits: int, group: int = 0):
    """The sweep on the asymmetric grid. Returns codes (0..2^bits-1), scales, zeros (out x G), errs, loss."""
    codes, params, errs, loss, _ = sweep_layer(W0, U, AsymmetricGrid(bits), group)
    return codes, params[:, :, 0].copy(), params[:, :, 1].copy(), errs, loss


def forced_replay(W0: np.ndarray, U: np.ndarray, bits: int, group: int, forced_codes_q: np.ndarray):
    """Replay the sweep taking the given codes (quantization order) instead of snapping.

    Returns (offsets, scales): offsets[r, j] = |clip(w/scale, -qmax, qmax) - c| at each step, which is
    <= 0.5 for a code that rounding could have chosen (up to the precision of the run that produced
    it); scales as the replay fitted them.
    """
    _, params, _, _, offsets = sweep_layer(W0, U, SymmetricGrid(bits), group, forced_codes_q)
    return offsets, params[:, :, 0].copy()


def forced_replay_asym(W0: np.ndarray, U: np.ndarray, bits: int, group: int, forced_codes_q: np.ndarray):
    """forced_replay on the asymmetric grid: offsets |clip(w / scale + zero, 0, levels) - c|."""
    return sweep_layer(W0, U, AsymmetricGrid(bits), group, forced_codes_q)[4]


# ---------------------------------------------------------------------------------------------
# Step 7: outputs in the original column order
# ---------------------------------------------------------------------------------------------
def group_index(perm: np.ndarray, group: int) -> np.ndarray:
    """g_idx[original column] = group of its quantization position ([guide] "When it breaks")."""
    d = perm.shape[0]
    g_idx = np.zeros(d, dtype=np.int64)
    if group:
        g_idx[perm] = np.arange(d) // group
    return g_idx


def finalize(codes_q: np.ndarray, scales: np.ndarray, perm: np.ndarray, group: int):
    """codes in original order, g_idx, and the dequantized Q = codes * scales[:, g_idx]."""
    codes = np.empty_like(codes_q)
    codes[:, perm] = codes_q
    g_idx = group_index(perm, group)
    Q = codes * scales[:, g_idx]
    return codes, g_idx, Q


def finalize_asym(codes_q: np.ndarray, scales: np.ndarray, zeros: np.ndarray, perm: np.ndarray, group: int):
    """codes in original order, g_idx, and Q = scales[:, g_idx] * (codes - zeros[:, g_idx])."""
    codes = np.empty_like(codes_q)
    codes[:, perm] = codes_q
    g_idx = group_index(perm, group)
    Q = asym_value(codes, scales[:, g_idx], zeros[:, g_idx])
    return codes, g_idx, Q


def _factor(H_p: np.ndarray, u_round):
    U = upper_factor_of_inverse(H_p)
    if u_round is not None:
        U = U.astype(u_round).astype(np.float64)
    return U


def gptq_oracle(W64: np.ndarray, X64: np.ndarray | None = None, bits: int = 4, group: int = 0,
                damp: float = 0.01, act_order: bool = False, hessian=None, u_round=None) -> dict:
    """The whole per-layer path. Defaults follow the guide's gptq() signature (bits=4, no groups,
    damp=0.01, no act_order). Pass hessian=(S, colsq, n) to skip step 1; u_round=np.float32 rounds U
    to that precision before the sweep (the noise floor's second mode)."""
    if hessian is None:
        S, colsq, n = hessian_from_x(X64)
    else:
        S, colsq, n = hessian
    H_p, perm, dead, lam = prepare(S, colsq, n, damp, act_order)
    U = _factor(H_p, u_round)
    W0 = start_weights(W64, perm, dead)
    codes_q, scales, errs, loss = compensation_loop(W0, U, bits, group)
    codes, g_idx, Q = finalize(codes_q, scales, perm, group)
    return dict(S=S, colsq=colsq, n=n, H_p=H_p, perm=perm, dead=dead, lam=lam, U=U, W0=W0,
                codes_q=codes_q, codes=codes, scales=scales, g_idx=g_idx, Q=Q, errs=errs, loss=loss)


def gptq_oracle_asym(W64: np.ndarray, X64: np.ndarray | None = None, bits: int = 4, group: int = 0,
                     damp: float = 0.01, act_order: bool = False, hessian=None, u_round=None) -> dict:
    """gptq_oracle with the asymmetric grid; the dict also holds `zeros`."""
    if hessian is None:
        S, colsq, n = hessian_from_x(X64)
    else:
        S, colsq, n = hessian
    H_p, perm, dead, lam = prepare(S, colsq, n, damp, act_order)
    U = _factor(H_p, u_round)
    W0 = start_weights(W64, perm, dead)
    codes_q, scales, zeros, errs, loss = compensation_loop_asym(W0, U, bits, group)
    codes, g_idx, Q = finalize_asym(codes_q, scales, zeros, perm, group)
    return dict(S=S, colsq=colsq, n=n, H_p=H_p, perm=perm, dead=dead, lam=lam, U=U, W0=W0,
                codes_q=codes_q, codes=codes, scales=scales, zeros=zeros, g_idx=g_idx, Q=Q, errs=errs,
                loss=loss)


# ---------------------------------------------------------------------------------------------
# Round-to-nearest, the comparison point ("plain rounding" in the lesson's acceptance test)
# ---------------------------------------------------------------------------------------------
def _rtn(W64, grid, group, dead, perm):
    d = W64.shape[1]
    perm = np.arange(d) if perm is None else perm
    dead = np.zeros(d, dtype=bool) if dead is None else dead
    W0 = start_weights(W64, perm, dead)
    codes_q = np.zeros(W0.shape, dtype=np.int64)
    Qq = np.zeros(W0.shape)
    step = group if group else d
    for g0 in range(0, d, step):
        run = W0[:, g0:g0 + step]
        p = tuple(np.broadcast_to(np.asarray(v, dtype=np.float64), (W0.shape[0],))[:, None] for v in grid.fit(run))
        c = grid.snap(run, p)
        codes_q[:, g0:g0 + step] = c.astype(np.int64)
        Qq[:, g0:g0 + step] = grid.value(c, p)
    codes = np.empty_like(codes_q)
    Q = np.empty_like(Qq)
    codes[:, perm] = codes_q
    Q[:, perm] = Qq
    return codes, Q


def rtn(W64: np.ndarray, bits: int, group: int = 0, dead: np.ndarray | None = None,
        perm: np.ndarray | None = None):
    """Same grid, fitted to the starting (dead-zeroed) weights of each row or group, no compensation.

    Groups are contiguous in the given column order (identity by default). Returns (codes, Q) in the
    original column order.
    """
    return _rtn(W64, SymmetricGrid(bits), group, dead, perm)


def rtn_asym(W64: np.ndarray, bits: int, group: int = 0, dead: np.ndarray | None = None,
             perm: np.ndarray | None = None):
    """Asymmetric round-to-nearest: (scale, zero) from the starting weights, no compensation."""
    return _rtn(W64, AsymmetricGrid(bits), group, dead, perm)


# ---------------------------------------------------------------------------------------------
# Step 10: the noise floor of an fp32-accumulated Hessian
# ---------------------------------------------------------------------------------------------
def quantize_rows(W_rows64: np.ndarray, S: np.ndarray, colsq: np.ndarray, n: int, bits: int, group: int,
                  damp: float, act_order: bool, u_round=None, asymmetric: bool = False) -> dict:
    """The oracle's path from a given S for a subset of W's rows (rows are independent given U)."""
    run = gptq_oracle_asym if asymmetric else gptq_oracle
    return run(W_rows64, bits=bits, group=group, damp=damp, act_order=act_order, hessian=(S, colsq, n),
               u_round=u_round)


def drift(ref: dict, alt: dict, W_rows64: np.ndarray, S: np.ndarray) -> dict:
    """How far `alt` lies from `ref`: the fraction of codes that differ, the relative Frobenius
    difference of the dequantized Q, and the relative change of the layer output error (through S)."""
    e_ref = output_error(W_rows64, ref["Q"], S)
    e_alt = output_error(W_rows64, alt["Q"], S)
    return dict(f=float(np.mean(ref["codes"] != alt["codes"])),
                mismatches=int(np.sum(ref["codes"] != alt["codes"])),
                q_rel=float(np.linalg.norm(alt["Q"] - ref["Q"]) / max(np.linalg.norm(ref["Q"]), 1e-300)),
                out_rel=float(abs(e_alt - e_ref) / max(e_ref, 1e-300)))


def noise_floor(W_rows64: np.ndarray, S64: np.ndarray, S32seg: np.ndarray, colsq: np.ndarray, n: int,
                bits: int, group: int, damp: float, act_order: bool, asymmetric: bool = False) -> dict:
    """The oracle measured against itself under the two perturbations an fp32 Hessian path brings:
    S summed in fp32 within 2048-row segments (S32seg, from accumulate_fp32_segments) and U rounded to
    fp32. Returns the fp64 reference run and, per mode, its drift from that run."""
    ref = quantize_rows(W_rows64, S64, colsq, n, bits, group, damp, act_order, asymmetric=asymmetric)
    via_s = quantize_rows(W_rows64, S32seg, colsq, n, bits, group, damp, act_order, asymmetric=asymmetric)
    via_u = quantize_rows(W_rows64, S64, colsq, n, bits, group, damp, act_order, u_round=np.float32,
                          asymmetric=asymmetric)
    return dict(ref=ref, fp32_segment_S=drift(ref, via_s, W_rows64, S64),
                fp32_U=drift(ref, via_u, W_rows64, S64))


# ---------------------------------------------------------------------------------------------
# Step 9: storage of the codes and their consumer ([guide] "When it breaks": integer codes with
# per-group scales, g_idx for act_order groups; [handbook] "int4" storage of 4-bit codes)
# ---------------------------------------------------------------------------------------------
def stored_code_offset(bits: int, asymmetric: bool) -> int:
    """Symmetric codes -qmax..qmax are stored as code + 2^(bits-1) (non-negative, below 2^bits); asymmetric
    codes 0..2^bits-1 are stored as they are. (The pages do not fix a packed layout; this is the reading.)"""
    return 0 if asymmetric else 2 ** (bits - 1)


def pack_rows(codes: np.ndarray, bits: int, asymmetric: bool = False) -> np.ndarray:
    """One little-endian bit stream per row: stored code j occupies stream bits [bits*j, bits*(j+1)), and
    stream bit k is bit k % 32 of 32-bit word k // 32. Unused high bits of the last word are 0."""
    if not 2 <= bits <= 8:
        raise ValueError("bits must be in 2..8")
    v = np.asarray(codes, dtype=np.int64) + stored_code_offset(bits, asymmetric)
    if v.size and (v.min() < 0 or v.max() >= 2 ** bits):
        raise ValueError("code outside the stored range")
    out, d = v.shape
    words = np.zeros((out, (d * bits + 31) // 32), dtype=np.int64)
    for j in range(d):
        bit = j * bits
        w, sh = bit // 32, bit % 32
        words[:, w] |= (v[:, j] << sh) & 0xFFFFFFFF
        if sh + bits > 32:  # the code straddles into the next word
            words[:, w + 1] |= v[:, j] >> (32 - sh)
    return words.astype(np.uint32)


def unpack_rows(words: np.ndarray, d: int, bits: int, asymmetric: bool = False) -> np.ndarray:
    """Inverse of pack_rows: (out x words) uint32 -> codes (out x d, int64)."""
    w64 = np.asarray(words, dtype=np.uint32).astype(np.int64)
    codes = np.zeros((w64.shape[0], d), dtype=np.int64)
    for j in range(d):
        bit = j * bits
        w, sh = bit // 32, bit % 32
        v = w64[:, w] >> sh
        if sh + bits > 32:
            v = v | (w64[:, w + 1] << (32 - sh))
        codes[:, j] = v & (2 ** bits - 1)
    return codes - stored_code_offset(bits, asymmetric)


def dequantize(codes: np.ndarray, scales: np.ndarray, g_idx: np.ndarray, zeros: np.ndarray | None = None):
    """Q[r, c] = scales[r, g] * (codes[r, c] - zeros[r, g]) with g = g_idx[c] (zero 0 on the symmetric
    grid), in fp64."""
    g = np.asarray(g_idx, dtype=np.int64)
    c = np.asarray(codes, dtype=np.float64)
    if zeros is not None:
        c = c - np.asarray(zeros, dtype=np.float64)[:, g]
    return np.asarray(scales, dtype=np.float64)[:, g] * c


def linear_forward(h: np.ndarray, Wl: np.ndarray, b: np.ndarray | None, relu: bool) -> np.ndarray:
    """One MLP layer, h W^T + b, then ReLU on hidden layers, exact in fp64 and rounded once to fp32.

    [guide] apply_layerwise (its source, in "Source code") stores layer weights and outputs in a float
    type it calls F and never defines, with a layer_forward it does not define either. Readings: F is
    float32; a layer is affine (weights and a bias) followed by ReLU, except the output layer, which has
    no activation; the fp32 result is the exact value rounded to nearest."""
    y = np.asarray(h, dtype=np.float64) @ np.asarray(Wl, dtype=np.float64).T
    if b is not None:
        y = y + np.asarray(b, dtype=np.float64)[None, :]
    if relu:
        y = np.maximum(y, 0.0)
    return y.astype(np.float32).astype(np.float64)


def apply_layerwise(weights, biases, X64: np.ndarray, quantize, skip_last: bool = False):
    """[guide] "How it works", apply_layerwise: quantize the layers in order, each one calibrated on the
    outputs of the layers before it AFTER those were quantized (the inputs it will see in use).

    weights[i]: out_i x in_i (in_0 = X's width); biases[i]: out_i or None; quantize(W64, h64) -> dict
    with "Q" (e.g. a partial of gptq_oracle). The quantized weights are kept in float32, as the driver
    stores them. Returns (results, inputs, h): results[i] is quantize's dict (None for a skipped last
    layer), inputs[i] the fp64 array layer i was calibrated on, h the network's output."""
    h = np.asarray(X64, dtype=np.float64)
    results, inputs = [], []
    L = len(weights)
    for i in range(L):
        last = i == L - 1
        W64 = np.asarray(weights[i], dtype=np.float64)
        inputs.append(h)
        if skip_last and last:
            results.append(None)
            Wl = W64
        else:
            r = quantize(W64, h)
            results.append(r)
            Wl = r["Q"].astype(np.float32)
        h = linear_forward(h.astype(np.float32), Wl, biases[i], relu=not last)
    return results, inputs, h


# ---------------------------------------------------------------------------------------------
# Output error ([guide] "What the simulations show": ||h W - h Wq||^2 / ||h W||^2)
# ---------------------------------------------------------------------------------------------
def output_error(W64: np.ndarray, Q: np.ndarray, S: np.ndarray) -> float:
    """||X (W - Q)^T||_F^2 through the Gram matrix S = X^T X (no n x out product needed)."""
    D = np.asarray(W64, dtype=np.float64) - Q
    return float(np.sum((D @ S) * D))


def relative_output_error(W64: np.ndarray, Q: np.ndarray, S: np.ndarray) -> float:
    W64 = np.asarray(W64, dtype=np.float64)
    return output_error(W64, Q, S) / float(np.sum((W64 @ S) * W64))


# ---------------------------------------------------------------------------------------------
# The OBS form of the same sweep (for cross-checks on tiny inputs)
# ---------------------------------------------------------------------------------------------
def obs_elimination_loop(W0: np.ndarray, H_p: np.ndarray, bits: int, group: int = 0):
    """The sweep written with the explicit inverse Hessian instead of its Cholesky factor.

    [guide] "How it works", OBS step: forcing coordinate j to quant(w_j) with e = w_j - quant(w_j)
    changes the row by delta = -(e / Hinv[j, j]) * Hinv[j, :]. "Remove j and repeat": the inverse
    Hessian of the remaining coordinates is one Gaussian-elimination step,
    Hinv <- Hinv - Hinv[:, j] Hinv[j, :] / Hinv[j, j]. Returns (codes, trajectory) where trajectory[j]
    is the row block just before column j is rounded.
    """
    qmax = qmax_for(bits)
    W = np.array(W0, dtype=np.float64, copy=True)
    out, d = W.shape
    Hinv = np.linalg.inv(H_p)
    codes = np.zeros((out, d), dtype=np.int64)
    traj = np.zeros((d, out, d))
    scale = row_scales(W, qmax)
    for j in range(d):
        if group and j % group == 0:
            scale = row_scales(W[:, j:j + group], qmax)
        traj[j] = W
        w = W[:, j]
        c = sym_code(w, scale, qmax)
        codes[:, j] = c.astype(np.int64)
        e = w - c * scale
        W = W - np.outer(e / Hinv[j, j], Hinv[j, :])
        W[:, j] = c * scale  # coordinate j is now fixed at its grid value
        Hinv = Hinv - np.outer(Hinv[:, j], Hinv[j, :]) / Hinv[j, j]
    return codes, traj
