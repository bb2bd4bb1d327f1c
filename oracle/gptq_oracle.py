"""CPU oracle for GPTQ per-layer quantization (numpy, fp64). TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke entry and the benchmark's CPU-baseline leg may import this module.
The GPU library never calls it, and this module imports nothing from the GPU package.

Sources (three web pages on GPTQ):
  [lesson]   "GPTQ's error-compensation loop" (Lesson 10 of 10), herodthegreater.github.io/pigeon/school/gptq_loop/
  [handbook] "GPTQ > Implementation with AutoGPTQ", mbrenndoerfer.com/writing/gptq-4bit-weight-quantization-llm-guide/
  [guide]    "GPTQ", herodthegreater.github.io/pigeon/guide/gptq/

What is computed (the method is a greedy sequential rounding heuristic, so the oracle follows its steps):
  1. Hessian of the layer's squared output error, H = 2 X^T X / n    ([guide] "The idea"; [lesson] intro)
  2. dead inputs (zero diagonal) get H_ii = 1 and zero weights       ([guide] "The code, line by line")
  3. damping: H += damp * mean(diag H) * I                            ([guide] "How it works", Damping)
  4. optional act_order: columns by decreasing diag(X^T X)            ([guide] "The code, line by line")
  5. U = upper Cholesky factor of H^-1, H^-1 = U^T U                  ([guide] "GPTQ's two tricks", trick 2)
  6. for each column j, for all rows at once: round to the symmetric grid, err = (w - q) / U[j, j],
     subtract outer(err, U[j, j+1:]) from the columns to the right   ([lesson] steps 1-4; [guide] trick 2)
     with per-row scales from the starting weights, or per-group scales from the updated weights at each
     group boundary                                                  ([guide] "The code, line by line")
  7. codes back to the original column order, g_idx for act_order+groups ([guide] "When it breaks")
  8. the same loop on the asymmetric grid: levels 0..2^b-1, (scale, zero) from min/max of the row or group
     ([guide] "Simplifications": the paper's default; [handbook] quantize_weight, gptq_quantize_row)
  9. storage and use: codes packed into 32-bit words, Q from codes, scales (zeros) and g_idx, and the
     layer-wise driver that calibrates each layer on the already-quantized layers' outputs
     ([guide] "When it breaks", "How it works" apply_layerwise; [handbook] int4 storage)

Readings where the pages leave a detail open (each is also listed with the build's design notes):
  * qmax for b bits is 2^(b-1) - 1 (the lesson's starter code; "2-bit" = ternary {-s, 0, s} in the guide).
  * round() ties go to even (numpy's rule); dead = colsq == 0 exactly, decided in fp64.
  * H[dead, dead] = 1 touches only the diagonal (numpy pairs the two boolean index arrays).
  * damping uses the mean diagonal after the dead fix; the normalisation is 2/n (not the handbook's 2).
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
"""
from __future__ import annotations

import numpy as np

HESSIAN_CHUNK_ROWS = 2048
SCALE_FLOOR = 1e-12  # [guide] "The code, line by line": per-row scale floor


# ---------------------------------------------------------------------------------------------
# Input decoding (the oracle reads the same stored bits as the GPU, widened exactly to fp64)
# ---------------------------------------------------------------------------------------------
def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 array or bf16 bit patterns (uint16) -> fp64, exactly."""
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    raise ValueError(dtype)


def qmax_for(bits: int) -> int:
    """Largest code of the symmetric grid {-qmax..qmax}: 2^(bits-1) - 1 ([lesson] starter code)."""
    if bits < 2:
        raise ValueError("bits must be >= 2")
    return 2 ** (bits - 1) - 1


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


def hessian_from_x(X64: np.ndarray):
    d = X64.shape[1]
    S = np.zeros((d, d))
    colsq = np.zeros(d)
    n = accumulate(S, colsq, X64)
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
    inputs, i.e. for P^T H P.
    """
    if n < 1:
        raise ValueError("n must be >= 1")
    d = S.shape[0]
    H = (2.0 / n) * S
    H = 0.5 * (H + H.T)  # S is symmetric up to summation order; use one value for (i, j) and (j, i)
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
    """U upper-triangular with positive diagonal and U^T U = H^-1 ([guide] trick 2, [lesson] intro).

    numpy's cholesky returns the lower factor L of H^-1 (H^-1 = L L^T); U = L^T. Raises
    numpy.linalg.LinAlgError when H is not positive definite.
    """
    return np.linalg.cholesky(np.linalg.inv(H_p)).T


# ---------------------------------------------------------------------------------------------
# Step 6: the column-by-column error-compensation loop
# ---------------------------------------------------------------------------------------------
def row_scales(Wblock: np.ndarray, qmax: int) -> np.ndarray:
    """Per-row scale max(max|w|, 1e-12) / qmax ([guide] "The code, line by line")."""
    if Wblock.shape[1] == 0:
        return np.full(Wblock.shape[0], SCALE_FLOOR / qmax)
    return np.maximum(np.abs(Wblock).max(axis=1), SCALE_FLOOR) / qmax


def start_weights(W64: np.ndarray, perm: np.ndarray, dead: np.ndarray) -> np.ndarray:
    """Working copy: dead input columns zeroed, then columns in quantization order ([guide] source)."""
    W0 = np.array(W64, dtype=np.float64, copy=True)
    W0[:, dead] = 0.0
    return W0[:, perm]


def compensation_loop(W0: np.ndarray, U: np.ndarray, bits: int, group: int = 0):
    """Quantize columns j = 0..in-1 of every row in turn, pushing each column's error right.

    [lesson] statement: q = round_to_grid(W[:, j]); err = (W[:, j] - q) / U[j, j];
    W[:, j+1:] -= outer(err, U[j, j+1:]). [guide] trick 2 derives this update from the OBS step.
    Scales: one per row from the starting weights; with groups, at each column j that starts a group,
    new scales from the *current* weights of columns [j, j + group) ([guide] "The code, line by line").
    Codes are clip(round(w / scale), -qmax, qmax), so compensation that pushes a weight past the
    scale is clipped and the clipped error is what propagates ([guide] "When it breaks").

    Returns codes (int64, quantization order), scales (out x G, G = ceil(in/group) or 1),
    errs (out x in, the err of every step) and loss (per row, sum of err^2).
    """
    qmax = qmax_for(bits)
    W = np.array(W0, dtype=np.float64, copy=True)
    out, d = W.shape
    n_groups = -(-d // group) if group else 1
    codes = np.zeros((out, d), dtype=np.int64)
    scales = np.zeros((out, n_groups))
    errs = np.zeros((out, d))
    scale = row_scales(W, qmax)
    if not group:
        scales[:, 0] = scale
    for j in range(d):
        if group and j % group == 0:
            scale = row_scales(W[:, j:j + group], qmax)
            scales[:, j // group] = scale
        w = W[:, j]
        c = np.clip(np.round(w / scale), -qmax, qmax)
        q = c * scale
        e = (w - q) / U[j, j]
        codes[:, j] = c.astype(np.int64)
        errs[:, j] = e
        if j + 1 < d:
            W[:, j + 1:] -= np.outer(e, U[j, j + 1:])
    loss = np.einsum("rj,rj->r", errs, errs)
    return codes, scales, errs, loss


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


def gptq_oracle(W64: np.ndarray, X64: np.ndarray | None = None, bits: int = 4, group: int = 0,
                damp: float = 0.01, act_order: bool = False, hessian=None) -> dict:
    """The whole per-layer path. Defaults follow the guide's gptq() signature (bits=4, no groups,
    damp=0.01, no act_order). Pass hessian=(S, colsq, n) to skip step 1."""
    if hessian is None:
        S, colsq, n = hessian_from_x(X64)
    else:
        S, colsq, n = hessian
    H_p, perm, dead, lam = prepare(S, colsq, n, damp, act_order)
    U = upper_factor_of_inverse(H_p)
    W0 = start_weights(W64, perm, dead)
    codes_q, scales, errs, loss = compensation_loop(W0, U, bits, group)
    codes, g_idx, Q = finalize(codes_q, scales, perm, group)
    return dict(S=S, colsq=colsq, n=n, H_p=H_p, perm=perm, dead=dead, lam=lam, U=U, W0=W0,
                codes_q=codes_q, codes=codes, scales=scales, g_idx=g_idx, Q=Q, errs=errs, loss=loss)


# ---------------------------------------------------------------------------------------------
# Round-to-nearest, the comparison point ("plain rounding" in the lesson's acceptance test)
# ---------------------------------------------------------------------------------------------
def rtn(W64: np.ndarray, bits: int, group: int = 0, dead: np.ndarray | None = None,
        perm: np.ndarray | None = None):
    """Same grid, scales from the starting (dead-zeroed) weights, no compensation.

    Groups are contiguous in the given column order (identity by default). Returns (codes, Q) in the
    original column order.
    """
    d = W64.shape[1]
    perm = np.arange(d) if perm is None else perm
    dead = np.zeros(d, dtype=bool) if dead is None else dead
    qmax = qmax_for(bits)
    W0 = start_weights(W64, perm, dead)
    codes_q = np.zeros(W0.shape, dtype=np.int64)
    Qq = np.zeros(W0.shape)
    for g0 in range(0, d, group if group else d):
        g1 = min(d, g0 + group) if group else d
        s = row_scales(W0[:, g0:g1], qmax)[:, None]
        c = np.clip(np.round(W0[:, g0:g1] / s), -qmax, qmax)
        codes_q[:, g0:g1] = c.astype(np.int64)
        Qq[:, g0:g1] = c * s
    codes = np.empty_like(codes_q)
    Q = np.empty_like(Qq)
    codes[:, perm] = codes_q
    Q[:, perm] = Qq
    return codes, Q


# ---------------------------------------------------------------------------------------------
# The asymmetric grid (min/max plus a zero point)
# ---------------------------------------------------------------------------------------------
# [guide] "Simplifications": the paper's default quantizer is asymmetric, min/max plus a zero point.
# [handbook] "quantize_weight" / "dequantize_weight" and the group parameters in "gptq_quantize_row" give
# the formulas: levels 0 .. 2^bits - 1; over a group's current weights, scale = (max - min) / (2^bits - 1)
# when max > min and 1 otherwise; zero = round(-min / scale) clipped to the levels; a weight's code is
# round(w / scale + zero) clipped to the levels, and its value is scale * (code - zero). Python's round
# rounds half to even, as numpy's does. The error-compensation loop around the quantizer is the same.
def asym_levels(bits: int) -> int:
    """Largest code of the asymmetric grid {0..2^bits - 1}."""
    if bits < 2:
        raise ValueError("bits must be >= 2")
    return 2 ** bits - 1


def asym_params(Wblock: np.ndarray, bits: int):
    """Per-row (scale, zero) of a block of columns ([handbook] group parameters)."""
    levels = asym_levels(bits)
    wmin = Wblock.min(axis=1)
    wmax = Wblock.max(axis=1)
    scale = np.where(wmax > wmin, (wmax - wmin) / levels, 1.0)
    zero = np.clip(np.round(-wmin / scale), 0, levels)
    return scale, zero


def asym_code(w: np.ndarray, scale: np.ndarray, zero: np.ndarray, bits: int) -> np.ndarray:
    """round(w / scale + zero) clipped to 0 .. 2^bits - 1 ([handbook] quantize_weight)."""
    return np.clip(np.round(w / scale + zero), 0, asym_levels(bits))


def asym_value(c: np.ndarray, scale: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """scale * (code - zero) ([handbook] dequantize_weight)."""
    return scale * (c - zero)


def compensation_loop_asym(W0: np.ndarray, U: np.ndarray, bits: int, group: int = 0):
    """The loop of compensation_loop with the asymmetric grid: (scale, zero) per row from the starting
    weights, or, with groups, from the current weights of columns [j, j + group) at each group start.

    Returns codes (int64, 0..2^bits-1, quantization order), scales and zeros (out x G), errs, loss.
    """
    W = np.array(W0, dtype=np.float64, copy=True)
    out, d = W.shape
    n_groups = -(-d // group) if group else 1
    codes = np.zeros((out, d), dtype=np.int64)
    scales = np.zeros((out, n_groups))
    zeros = np.zeros((out, n_groups))
    errs = np.zeros((out, d))
    scale, zero = asym_params(W, bits)
    if not group:
        scales[:, 0], zeros[:, 0] = scale, zero
    for j in range(d):
        if group and j % group == 0:
            scale, zero = asym_params(W[:, j:j + group], bits)
            scales[:, j // group], zeros[:, j // group] = scale, zero
        w = W[:, j]
        c = asym_code(w, scale, zero, bits)
        q = asym_value(c, scale, zero)
        e = (w - q) / U[j, j]
        codes[:, j] = c.astype(np.int64)
        errs[:, j] = e
        if j + 1 < d:
            W[:, j + 1:] -= np.outer(e, U[j, j + 1:])
    loss = np.einsum("rj,rj->r", errs, errs)
    return codes, scales, zeros, errs, loss


def finalize_asym(codes_q: np.ndarray, scales: np.ndarray, zeros: np.ndarray, perm: np.ndarray, group: int):
    """codes in original order, g_idx, and Q = scales[:, g_idx] * (codes - zeros[:, g_idx])."""
    codes = np.empty_like(codes_q)
    codes[:, perm] = codes_q
    g_idx = group_index(perm, group)
    Q = asym_value(codes, scales[:, g_idx], zeros[:, g_idx])
    return codes, g_idx, Q


def gptq_oracle_asym(W64: np.ndarray, X64: np.ndarray | None = None, bits: int = 4, group: int = 0,
                     damp: float = 0.01, act_order: bool = False, hessian=None) -> dict:
    """gptq_oracle with the asymmetric grid; the dict also holds `zeros`."""
    if hessian is None:
        S, colsq, n = hessian_from_x(X64)
    else:
        S, colsq, n = hessian
    H_p, perm, dead, lam = prepare(S, colsq, n, damp, act_order)
    U = upper_factor_of_inverse(H_p)
    W0 = start_weights(W64, perm, dead)
    codes_q, scales, zeros, errs, loss = compensation_loop_asym(W0, U, bits, group)
    codes, g_idx, Q = finalize_asym(codes_q, scales, zeros, perm, group)
    return dict(S=S, colsq=colsq, n=n, H_p=H_p, perm=perm, dead=dead, lam=lam, U=U, W0=W0,
                codes_q=codes_q, codes=codes, scales=scales, zeros=zeros, g_idx=g_idx, Q=Q, errs=errs,
                loss=loss)


def rtn_asym(W64: np.ndarray, bits: int, group: int = 0, dead: np.ndarray | None = None,
             perm: np.ndarray | None = None):
    """Asymmetric round-to-nearest: (scale, zero) from the starting weights, no compensation."""
    d = W64.shape[1]
    perm = np.arange(d) if perm is None else perm
    dead = np.zeros(d, dtype=bool) if dead is None else dead
    W0 = start_weights(W64, perm, dead)
    codes_q = np.zeros(W0.shape, dtype=np.int64)
    Qq = np.zeros(W0.shape)
    for g0 in range(0, d, group if group else d):
        g1 = min(d, g0 + group) if group else d
        s, z = asym_params(W0[:, g0:g1], bits)
        c = asym_code(W0[:, g0:g1], s[:, None], z[:, None], bits)
        codes_q[:, g0:g1] = c.astype(np.int64)
        Qq[:, g0:g1] = asym_value(c, s[:, None], z[:, None])
    codes = np.empty_like(codes_q)
    Q = np.empty_like(Qq)
    codes[:, perm] = codes_q
    Q[:, perm] = Qq
    return codes, Q


def forced_replay_asym(W0: np.ndarray, U: np.ndarray, bits: int, group: int, forced_codes_q: np.ndarray):
    """forced_replay with the asymmetric grid: dist = |clip(w / scale + zero, 0, levels) - c|."""
    levels = asym_levels(bits)
    W = np.array(W0, dtype=np.float64, copy=True)
    out, d = W.shape
    dist = np.zeros((out, d))
    scale, zero = asym_params(W, bits)
    for j in range(d):
        if group and j % group == 0:
            scale, zero = asym_params(W[:, j:j + group], bits)
        w = W[:, j]
        c = forced_codes_q[:, j].astype(np.float64)
        dist[:, j] = np.abs(np.clip(w / scale + zero, 0, levels) - c)
        e = (w - asym_value(c, scale, zero)) / U[j, j]
        if j + 1 < d:
            W[:, j + 1:] -= np.outer(e, U[j, j + 1:])
    return dist


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
    return float(np.einsum("ri,ij,rj->", D, S, D))


def relative_output_error(W64: np.ndarray, Q: np.ndarray, S: np.ndarray) -> float:
    W64 = np.asarray(W64, dtype=np.float64)
    return output_error(W64, Q, S) / float(np.einsum("ri,ij,rj->", W64, S, W64))


# ---------------------------------------------------------------------------------------------
# Comparison helper: forced replay ("mismatches only at round-half boundaries")
# ---------------------------------------------------------------------------------------------
def forced_replay(W0: np.ndarray, U: np.ndarray, bits: int, group: int, forced_codes_q: np.ndarray):
    """Run the loop but take the given codes (quantization order) instead of rounding.

    Returns, per entry, how far the forced code is from the clipped unrounded value,
    |clip(w/scale, -qmax, qmax) - c|; a code that a correct loop could have chosen has this <= 0.5
    (up to the precision of the run that produced it). Also returns the replayed Q and scales.
    """
    qmax = qmax_for(bits)
    W = np.array(W0, dtype=np.float64, copy=True)
    out, d = W.shape
    dist = np.zeros((out, d))
    n_groups = -(-d // group) if group else 1
    scales = np.zeros((out, n_groups))
    scale = row_scales(W, qmax)
    if not group:
        scales[:, 0] = scale
    for j in range(d):
        if group and j % group == 0:
            scale = row_scales(W[:, j:j + group], qmax)
            scales[:, j // group] = scale
        w = W[:, j]
        c = forced_codes_q[:, j].astype(np.float64)
        dist[:, j] = np.abs(np.clip(w / scale, -qmax, qmax) - c)
        e = (w - c * scale) / U[j, j]
        if j + 1 < d:
            W[:, j + 1:] -= np.outer(e, U[j, j + 1:])
    return dist, scales


# ---------------------------------------------------------------------------------------------
# The OBS form of the same loop (for cross-checks on tiny inputs)
# ---------------------------------------------------------------------------------------------
def obs_elimination_loop(W0: np.ndarray, H_p: np.ndarray, bits: int, group: int = 0):
    """The loop written with the explicit inverse Hessian instead of its Cholesky factor.

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
        c = np.clip(np.round(w / scale), -qmax, qmax)
        codes[:, j] = c.astype(np.int64)
        e = w - c * scale
        W = W - np.outer(e / Hinv[j, j], Hinv[j, :])
        W[:, j] = c * scale  # coordinate j is now fixed at its grid value
        Hinv = Hinv - np.outer(Hinv[:, j], Hinv[j, :]) / Hinv[j, j]
    return codes, traj
