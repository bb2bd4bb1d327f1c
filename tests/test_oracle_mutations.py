"""Plant plausible mistakes in the CPU oracle and check that the pins catch each one.

Every mutation is a small edit of one oracle step (a sign, an index, a dropped term, a transposed
operand, a wrong order of two steps). The pins in test_oracle_pins.py must fail for every one of them;
otherwise a pin is missing. CPU only; the mutations live only inside this test.
"""
import numpy as np
import pytest

from oracle import gptq_oracle as O
import tests.test_oracle_pins as P


# Mistakes in the steps of the sweep: each replaces one of the oracle's step functions.
def _propagate_sign(w, j, eps, U):
    w[j + 1:] += eps * U[j, j + 1:]


def _propagate_transposed(w, j, eps, U):
    w[j + 1:] -= eps * U[j + 1:, j]


def _propagate_off_by_one(w, j, eps, U):
    w[j + 1:] -= eps * U[j, j:-1]


def _step_error_undivided(residual, pivot):
    return residual


def _sym_code_unclipped(w, scale, qmax):
    return np.rint(w / scale)


def _sym_code_floor(w, scale, qmax):
    return np.minimum(np.maximum(np.floor(w / scale), -qmax), qmax)


def _grid_from_start(w_now, w_start, j, group):
    if group:
        return w_start[j:j + group] if j % group == 0 else None
    return w_start if j == 0 else None


def _grid_never_refit(w_now, w_start, j, group):
    return w_start if j == 0 else None


def _grid_refit_every_step(w_now, w_start, j, group):
    return w_now[j:j + group] if group else (w_start if j == 0 else None)


def _asym_code_unclipped(w, scale, zero, bits):
    return np.rint(w / scale + zero)


SWEEP_MUTATIONS = {
    "sign": ("_propagate", _propagate_sign),
    "transposed_u": ("_propagate", _propagate_transposed),
    "off_by_one": ("_propagate", _propagate_off_by_one),
    "no_divide": ("_step_error", _step_error_undivided),
    "unclipped": ("sym_code", _sym_code_unclipped),
    "floor_not_round": ("sym_code", _sym_code_floor),
    "group_from_original": ("_grid_source", _grid_from_start),
    "groups_ignored": ("_grid_source", _grid_never_refit),
    "refit_every_step": ("_grid_source", _grid_refit_every_step),
}


def _sweep_factory(kind):
    return SWEEP_MUTATIONS[kind][1]


def _prepare_factory(kind):
    def prepare(S, colsq, n, damp, act_order):
        d = S.shape[0]
        Sym = np.tril(S) + np.tril(S, -1).T
        H = (2.0 / n) * Sym if kind != "no_two" else (1.0 / n) * Sym
        dead = colsq == 0.0
        idx = np.flatnonzero(dead)
        if kind == "damp_before_dead":
            lam = damp * np.mean(np.diag(H))
            H[idx, idx] = 1.0
        else:
            H[idx, idx] = 1.0
            lam = damp * np.mean(np.diag(H))
        if kind == "absolute_damp":
            lam = damp
        H[np.arange(d), np.arange(d)] += lam
        if act_order:
            perm = np.argsort(colsq, kind="stable") if kind == "ascending" else O.activation_order(colsq)
        else:
            perm = np.arange(d)
        H_p = H[np.ix_(perm, perm)]
        return H_p, perm, dead, lam
    return prepare


def _factor_factory(kind):
    def factor(H_p):
        if kind == "lower":
            return np.linalg.cholesky(np.linalg.inv(H_p))
        if kind == "chol_of_h":
            return np.linalg.cholesky(H_p).T
        if kind == "inverse_of_chol":
            return np.linalg.inv(np.linalg.cholesky(H_p)).T
        raise ValueError(kind)
    return factor


PINS = [
    (P.test_golden_two_column_hand, ()),
    (P.test_hessian_brute_force_and_chunking, ()),
    (P.test_damping_and_dead_hand_values, ()),
    (P.test_all_dead_inputs, ()),
    (P.test_u_factor_properties_and_reverse_closed_form, (7,)),
    (P.test_u_rows_are_eliminated_inverse_rows, ()),
    (P.test_cholesky_form_equals_obs_elimination, (3,)),
    (P.test_cholesky_form_equals_obs_elimination, (5,)),
    (P.test_loop_matches_exact_rational_obs, (0,)),
    (P.test_loop_matches_exact_rational_obs, (4,)),
    (P.test_each_step_is_the_constrained_least_squares_solve, ()),
    (P.test_group_scales_from_updated_weights_exact, (0,)),
    (P.test_group_scales_from_updated_weights_exact, (1,)),
    (P.test_loss_identity, (4, True)),
    (P.test_clipping_propagates_clipped_error, ()),
    (P.test_group_sizes_special_cases, ()),
    (P.test_act_order_equals_explicitly_permuted_problem, ()),
    (P.test_output_error_well_below_rtn, ("teacher", 3, False)),
]

MUTATIONS = [
    (SWEEP_MUTATIONS[k][0], _sweep_factory, k) for k in SWEEP_MUTATIONS
] + [
    ("prepare", _prepare_factory, k) for k in ["no_two", "damp_before_dead", "absolute_damp", "ascending"]
] + [
    ("upper_factor_of_inverse", _factor_factory, k) for k in ["lower", "chol_of_h", "inverse_of_chol"]
]


@pytest.mark.parametrize("name,factory,kind", MUTATIONS, ids=[f"{m[0]}-{m[2]}" for m in MUTATIONS])
def test_pins_catch_planted_mistake(monkeypatch, name, factory, kind):
    monkeypatch.setattr(O, name, factory(kind))
    caught = []
    for fn, args in PINS:
        try:
            fn(*args)
        except (AssertionError, np.linalg.LinAlgError, FloatingPointError, ValueError, IndexError):
            caught.append(fn.__name__)
    assert caught, f"no pin caught mutation {name}:{kind}"


# ------------------------------------------------------------------------------------------------
# The asymmetric grid: mistakes in its parameters, its rounding or its loop
# ------------------------------------------------------------------------------------------------
import tests.test_oracle_pins_asym as PA  # noqa: E402


def _asym_params_factory(kind):
    def params(Wblock, bits):
        levels = 2 ** bits - 1
        if kind == "symmetric_levels":
            levels = 2 ** (bits - 1) - 1
        wmin = Wblock.min(axis=-1)
        wmax = Wblock.max(axis=-1)
        if kind == "levels_off_by_one":
            scale = np.where(wmax > wmin, (wmax - wmin) / (levels + 1), 1.0)
        else:
            scale = np.where(wmax > wmin, (wmax - wmin) / levels, 1.0)
        if kind == "zero_sign":
            zero = np.clip(np.round(wmin / scale), 0, levels)
        elif kind == "zero_unclipped":
            zero = np.round(-wmin / scale)
        else:
            zero = np.clip(np.round(-wmin / scale), 0, levels)
        return scale, zero
    return params


def _asym_value_factory(kind):
    def value(c, scale, zero):
        if kind == "no_zero_shift":
            return scale * c
        raise ValueError(kind)
    return value


ASYM_SWEEP_MUTATIONS = {
    "group_from_original": ("_grid_source", _grid_from_start),
    "error_before_clip": ("asym_code", _asym_code_unclipped),
    "no_divide": ("_step_error", _step_error_undivided),
}


def _asym_sweep_factory(kind):
    return ASYM_SWEEP_MUTATIONS[kind][1]


PINS_ASYM = [
    (PA.test_grid_hand_values, ()),
    (PA.test_grid_end_points_and_half_step_bound, (3,)),
    (PA.test_loop_matches_exact_rational_obs_asym, (0,)),
    (PA.test_loop_matches_exact_rational_obs_asym, (2,)),
    (PA.test_loop_matches_exact_rational_obs_asym, (5,)),
    (PA.test_group_params_from_updated_weights_exact_asym, (0,)),
    (PA.test_group_params_from_updated_weights_exact_asym, (1,)),
    (PA.test_heavy_damping_is_rtn_asym, (3, 32)),
    (PA.test_loss_identity_asym, (4, True)),
    (PA.test_outputs_consistent_asym, ()),
    (PA.test_output_error_below_rtn_asym, (3,)),
]

MUTATIONS_ASYM = [
    ("asym_params", _asym_params_factory, k) for k in
    ["symmetric_levels", "levels_off_by_one", "zero_sign", "zero_unclipped"]
] + [
    ("asym_value", _asym_value_factory, "no_zero_shift"),
] + [
    (ASYM_SWEEP_MUTATIONS[k][0], _asym_sweep_factory, k) for k in ASYM_SWEEP_MUTATIONS
]


@pytest.mark.parametrize("name,factory,kind", MUTATIONS_ASYM, ids=[f"{m[0]}-{m[2]}" for m in MUTATIONS_ASYM])
def test_asym_pins_catch_planted_mistake(monkeypatch, name, factory, kind):
    monkeypatch.setattr(O, name, factory(kind))
    caught = []
    for fn, args in PINS_ASYM:
        try:
            fn(*args)
        except (AssertionError, np.linalg.LinAlgError, FloatingPointError, ValueError, IndexError):
            caught.append(fn.__name__)
    assert caught, f"no pin caught mutation {name}:{kind}"


# ------------------------------------------------------------------------------------------------
# Storage and the layer-wise driver: a wrong bit order, a lost straddle, g_idx ignored, a missing
# bias, the classic mistake of calibrating on full-precision outputs
# ------------------------------------------------------------------------------------------------
import tests.test_oracle_pins_storage as PS  # noqa: E402


def _pack_factory(kind):
    def pack(codes, bits, asymmetric=False):
        v = np.asarray(codes, dtype=np.int64) + O.stored_code_offset(bits, asymmetric)
        if v.size and (v.min() < 0 or v.max() >= 2 ** bits):
            raise ValueError("range")
        out, d = v.shape
        words = np.zeros((out, (d * bits + 31) // 32), dtype=np.int64)
        for j in range(d):
            bit = j * bits
            w, sh = bit // 32, bit % 32
            if kind == "msb_first":
                sh = 32 - bits - sh if sh + bits <= 32 else sh
            words[:, w] |= (v[:, j] << sh) & 0xFFFFFFFF
            if sh + bits > 32 and kind != "no_straddle":
                words[:, w + 1] |= v[:, j] >> (32 - sh)
        return words.astype(np.uint32)
    return pack


def _dequant_factory(kind):
    def deq(codes, scales, g_idx, zeros=None):
        d = np.asarray(codes).shape[1]
        G = np.asarray(scales).shape[1]
        g = np.minimum(np.arange(d) * G // d, G - 1) if kind == "positional_groups" else np.asarray(g_idx)
        c = np.asarray(codes, dtype=np.float64)
        if zeros is not None and kind != "drop_zero":
            c = c - np.asarray(zeros, dtype=np.float64)[:, g]
        return np.asarray(scales, dtype=np.float64)[:, g] * c
    return deq


def _forward_factory(kind):
    def fwd(h, Wl, b, relu):
        y = np.asarray(h, dtype=np.float64) @ np.asarray(Wl, dtype=np.float64).T
        if b is not None and kind != "no_bias":
            y = y + np.asarray(b, dtype=np.float64)[None, :]
        if relu or kind == "relu_on_last":
            y = np.maximum(y, 0.0)
        return y.astype(np.float32).astype(np.float64)
    return fwd


def _layerwise_factory(kind):
    def drive(weights, biases, X64, quantize, skip_last=False):
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
                Wl = W64 if kind == "full_precision_inputs" else r["Q"].astype(np.float32)
            h = O.linear_forward(h.astype(np.float32), Wl, biases[i], relu=not last)
        return results, inputs, h
    return drive


PINS_STORAGE = [
    (PS.test_pack_hand_word_4bit, ()),
    (PS.test_pack_hand_words_3bit_straddle, ()),
    (PS.test_pack_equals_bigint_stream_and_round_trips, (3, False)),
    (PS.test_dequantize_hand_values, ()),
    (PS.test_dequantize_reproduces_quantizer_q, (True,)),
    (PS.test_linear_forward_hand_values, ()),
    (PS.test_layerwise_identity_quantizer_is_the_plain_forward, ()),
    (PS.test_layerwise_calibrates_on_quantized_outputs, ()),
    (PS.test_layerwise_skip_last_keeps_output_layer, ()),
]

MUTATIONS_STORAGE = [
    ("pack_rows", _pack_factory, k) for k in ["msb_first", "no_straddle"]
] + [
    ("dequantize", _dequant_factory, k) for k in ["positional_groups", "drop_zero"]
] + [
    ("linear_forward", _forward_factory, k) for k in ["no_bias", "relu_on_last"]
] + [
    ("apply_layerwise", _layerwise_factory, "full_precision_inputs"),
]


@pytest.mark.parametrize("name,factory,kind", MUTATIONS_STORAGE,
                         ids=[f"{m[0]}-{m[2]}" for m in MUTATIONS_STORAGE])
def test_storage_pins_catch_planted_mistake(monkeypatch, name, factory, kind):
    monkeypatch.setattr(O, name, factory(kind))
    caught = []
    for fn, args in PINS_STORAGE:
        try:
            fn(*args)
        except (AssertionError, ValueError, IndexError):
            caught.append(fn.__name__)
    assert caught, f"no pin caught mutation {name}:{kind}"


# ------------------------------------------------------------------------------------------------
# Input decoding and the noise-floor modes
# ------------------------------------------------------------------------------------------------
def _decode_factory(kind):
    def to_f64(a, dtype):
        if dtype == "bf16":
            u = np.asarray(a, dtype=np.uint16).astype(np.uint32)
            if kind == "low_half":
                return u.view(np.float32).astype(np.float64)
            if kind == "truncated_sign":
                return (u << np.uint32(17) >> np.uint32(1)).view(np.float32).astype(np.float64)
        return np.asarray(a, dtype=np.float32 if dtype == "f32" else np.float64).astype(np.float64)
    return to_f64


def _segments_factory(kind):
    def acc(S, colsq, X64, seg_rows=2048):
        n = X64.shape[0]
        for r0 in range(0, n, seg_rows):
            blk = X64[r0:r0 + seg_rows]
            if kind == "fp64_sums":
                S += blk.T @ blk
            elif kind == "fp32_total":
                S[:] = (S.astype(np.float32) + (blk.astype(np.float32).T @ blk.astype(np.float32))).astype(np.float64)
            colsq += np.einsum("ki,ki->i", blk, blk)
        return n
    return acc


def _chain_factory(kind):
    def block(XI, XJ, chain_rows=4096, group_rows=16):
        out = np.zeros((XI.shape[1], XJ.shape[1]))
        run = np.zeros(out.shape, dtype=np.float32)
        for c0 in range(0, XI.shape[0], chain_rows):
            if kind != "no_chain_reset":
                run = np.zeros(out.shape, dtype=np.float32)
            for g0 in range(c0, min(XI.shape[0], c0 + chain_rows), group_rows):
                step = run.astype(np.float64) + XI[g0:g0 + group_rows].T @ XJ[g0:g0 + group_rows]
                run = step if kind == "fp64_running_sum" else step.astype(np.float32)
            out = run.astype(np.float64) if kind == "no_chain_reset" else out + run
        return out
    return block


PINS_INPUTS = [
    (P.test_fp32_chain_model_equals_scalar_loop_and_is_exact_on_integers, ()),
    (P.test_fp32_chain_model_error_is_within_the_sequential_bound, ()),
    (P.test_bf16_decoding_matches_torch_for_every_pattern, ()),
    (P.test_fp32_segment_hessian_is_exact_on_integer_data, ()),
    (P.test_fp32_segment_hessian_error_is_fp32_sized, ()),
    (P.test_noise_floor_is_zero_when_the_fp32_sums_are_exact, ()),
]

MUTATIONS_INPUTS = [
    ("to_f64", _decode_factory, k) for k in ["low_half", "truncated_sign"]
] + [
    ("accumulate_fp32_segments", _segments_factory, k) for k in ["fp64_sums", "fp32_total"]
] + [
    ("fp32_chain_block", _chain_factory, k) for k in ["no_chain_reset", "fp64_running_sum"]
]


@pytest.mark.parametrize("name,factory,kind", MUTATIONS_INPUTS, ids=[f"{m[0]}-{m[2]}" for m in MUTATIONS_INPUTS])
def test_input_pins_catch_planted_mistake(monkeypatch, name, factory, kind):
    monkeypatch.setattr(O, name, factory(kind))
    caught = []
    for fn, args in PINS_INPUTS:
        try:
            with np.errstate(invalid="ignore"):
                fn(*args)
        except (AssertionError, ValueError, IndexError):
            caught.append(fn.__name__)
    assert caught, f"no pin caught mutation {name}:{kind}"
