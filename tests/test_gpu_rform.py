"""GPU parity of the R-form route (gptq_prepare_chol with GPTQ_FACTOR_R_FORM and gptq_quantize_layer_r)
against the CPU oracle: the factor form against oracle.gptq_oracle.r_form, the loop against the oracle's
loop with U, and the whole path against the oracle end to end.

The route needs in % 64 == 0: sizes 64 .. 1344 (1344 = 10.5 panels: a 64-column last panel, the two
factorization blocks per panel, several 256-column outer blocks of the factorization), 4096 rows x 3072
columns for the 128 x 128 products of the loop's block update. The loop's results are compared as for the
U route: codes equal except where the oracle's forced replay shows the GPU's code within rounding of a grid
midpoint, scales and per-row loss to rounding.
"""
import numpy as np
import pytest
import torch

import post_weight_quantization_05_amd as G
from oracle import gptq_oracle as O
import synthetic as syn
from tests.parity import (assert_gates, compare, compare_asym, dequantized, dev64, layer_inputs, to_device)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _cfg(name, out, d, n, **kw):
    return syn.custom_config(name, out, d, n, **kw)


TEACHER = syn.config_by_name("teacher")  # 256 x 256, dead inputs
MID = _cfg("bf16_mid", 96, 640, 5000, dtype="bf16", w_std=0.02, outlier_channels=6, w_seed=11, x_seed=12)
R1344 = _cfg("bf16_r1344", 72, 1344, 3000, dtype="bf16", w_std=0.02, outlier_channels=4, dead_channels=5,
             w_seed=31, x_seed=32)
RBIG = _cfg("bf16_rbig", 4100, 3072, 4096, dtype="bf16", w_std=0.02, outlier_channels=6, w_seed=33, x_seed=34)


def _oracle_prep(cfg, act, damp=0.01):
    W, X, W64, X64 = layer_inputs(cfg)
    S, colsq, n = O.hessian_from_x(X64)
    H_p, perm, dead, lam = O.prepare(S, colsq, n, damp, act)
    U = O.upper_factor_of_inverse(H_p)
    M = O.r_form(H_p)
    return W, W64, S, colsq, n, H_p, perm, dead, U, M


def _check_form(Mg, M):
    """Upper part (R) and the diagonal blocks' lower parts (U's blocks, reversed) to the accuracy of U."""
    up = np.triu(M)
    assert np.linalg.norm(np.triu(Mg) - up) <= 1e-10 * np.linalg.norm(up)
    lo = np.tril(M, -1)
    assert np.linalg.norm(np.tril(Mg, -1) - lo) <= 1e-10 * max(np.linalg.norm(lo), 1e-300)


@pytest.mark.parametrize("cfg,act", [(TEACHER, False), (MID, False), (MID, True), (R1344, True)],
                         ids=["teacher", "mid", "mid-act", "r1344-act"])
def test_prepare_r_form_matches_oracle(cfg, act):
    print(f"[r-prepare] {cfg.name} act={act}", flush=True)
    W, W64, S, colsq, n, H_p, perm, dead, U, M = _oracle_prep(cfg, act)
    Mg, p, dd = G.prepare_chol(dev64(S), dev64(colsq), n, 0.01, act, G.GPTQ_FACTOR_R_FORM)
    assert np.array_equal(p.cpu().numpy(), perm)
    assert np.array_equal(dd.cpu().numpy().astype(bool), dead)
    _check_form(Mg.cpu().numpy(), M)


# 2560 and 3136: the outer blocks switch partway to updating the next outer block's columns in their own
# steps (at most 2048 rows below it); 3136 ends on a 64-column outer block
@pytest.mark.parametrize("d", [64, 128, 192, 576, 1024, 1088, 2560, 3136])
def test_prepare_r_form_sizes(d):
    rng = np.random.default_rng(900 + d)
    X = rng.standard_normal((3 * d + 2, d)) @ (np.eye(d) + 0.2 * rng.standard_normal((d, d)))
    S, colsq, n = O.hessian_from_x(X)
    S = 0.5 * (S + S.T)
    colsq = np.diag(S).copy()
    H_p, perm, dead, lam = O.prepare(S, colsq, n, 0.01, True)
    Mg, p, dd = G.prepare_chol(dev64(S), dev64(colsq), n, 0.01, True, G.GPTQ_FACTOR_R_FORM)
    assert np.array_equal(p.cpu().numpy(), perm)
    _check_form(Mg.cpu().numpy(), O.r_form(H_p))


RQ_CASES = [
    # (cfg, bits, group, act, asymmetric)
    (TEACHER, 3, 0, False, False),
    (MID, 4, 0, False, False),
    (MID, 4, 128, True, False),
    (MID, 3, 64, False, True),
    (R1344, 4, 0, True, False),
    (R1344, 3, 128, True, False),
    (R1344, 4, 32, False, True),
    (MID, 4, 0, True, True),      # one asymmetric grid per row: T folded into the steps, D from the codes
    (R1344, 3, 0, False, True),
    (MID, 8, 0, False, False),
    (R1344, 2, 16, True, False),
]


@pytest.mark.parametrize("cfg,bits,group,act,asym", RQ_CASES,
                         ids=[f"{c.name}-b{b}-g{g}-a{int(a)}-{'asym' if s else 'sym'}" for c, b, g, a, s in RQ_CASES])
def test_quantize_r_matches_oracle(cfg, bits, group, act, asym):
    """Stage isolation: the oracle's R form / perm / dead in; the oracle's loop (with U) is the reference."""
    print(f"[r-quantize] {cfg.name} bits={bits} group={group} act={act} asym={asym}", flush=True)
    W, W64, S, colsq, n, H_p, perm, dead, U, M = _oracle_prep(cfg, act)
    W0 = O.start_weights(W64, perm, dead)
    if asym:
        codes_q, scales, zeros, errs, loss = O.compensation_loop_asym(W0, U, bits, group)
        codes, g_idx, Q = O.finalize_asym(codes_q, scales, zeros, perm, group)
    else:
        codes_q, scales, errs, loss = O.compensation_loop(W0, U, bits, group)
        codes, g_idx, Q = O.finalize(codes_q, scales, perm, group)
    r = G.quantize_layer(to_device(W, cfg.dtype), dev64(M), dev64(perm.astype(np.int32)),
                         dev64(dead.astype(np.uint8)), bits, group, asymmetric=asym, r_form=True)
    torch.cuda.synchronize()
    gc = r.codes.cpu().numpy().astype(np.int64)
    assert np.array_equal(r.g_idx.cpu().numpy(), g_idx)
    mism = int(np.sum(gc != codes))
    if mism:  # allowed only where the forced replay says the code was a valid choice
        if asym:
            dist = O.forced_replay_asym(W0, U, bits, group, gc[:, perm])
        else:
            dist, _ = O.forced_replay(W0, U, bits, group, gc[:, perm])
        assert dist.max() <= 0.5 + 1e-9, (mism, dist.max())
    assert mism <= 0.001 * gc.size
    if asym:
        np.testing.assert_array_equal(r.zeros.cpu().numpy(), zeros.astype(np.int32))
    np.testing.assert_allclose(r.scales.cpu().numpy(), scales.astype(np.float32), rtol=2e-7)
    np.testing.assert_allclose(r.row_loss.cpu().numpy(), loss, rtol=1e-9, atol=1e-12 * max(loss.max(), 1e-18))


@pytest.mark.parametrize("bits,group,act", [(4, 0, False), (3, 128, True)])
def test_quantize_r_large_products_sampled_rows(bits, group, act):
    """4100 x 3072: the first block update (4100 x 2048, K = 1024) takes the 128 x 128 kernel; the oracle's
    loop on sampled rows (rows are independent given U)."""
    cfg = RBIG
    print(f"[r-quantize-big] bits={bits} group={group} act={act}", flush=True)
    W, W64, S, colsq, n, H_p, perm, dead, U, M = _oracle_prep(cfg, act)
    r = G.quantize_layer(to_device(W, cfg.dtype), dev64(M), dev64(perm.astype(np.int32)),
                         dev64(dead.astype(np.uint8)), bits, group, r_form=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(10).choice(cfg.out, 40, replace=False),
                                     [0, 1, 127, 128, 4095, 4096, cfg.out - 1]]))
    W0 = O.start_weights(W64[rows], perm, dead)
    codes_q, scales, errs, loss = O.compensation_loop(W0, U, bits, group)
    codes, g_idx, Q = O.finalize(codes_q, scales, perm, group)
    gc = r.codes.cpu().numpy()[rows].astype(np.int64)
    assert np.array_equal(r.g_idx.cpu().numpy(), g_idx)
    mism = int(np.sum(gc != codes))
    if mism:
        dist, _ = O.forced_replay(W0, U, bits, group, gc[:, perm])
        assert dist.max() <= 0.5 + 1e-9, (mism, dist.max())
    assert mism <= 0.001 * gc.size
    np.testing.assert_allclose(r.scales.cpu().numpy()[rows], scales.astype(np.float32), rtol=2e-7)
    np.testing.assert_allclose(r.row_loss.cpu().numpy()[rows], loss, rtol=1e-9, atol=1e-12 * max(loss.max(), 1e-18))


E2E_R_CASES = [
    (TEACHER, 3, 0, False, False),
    (TEACHER, 2, 0, True, False),
    (MID, 4, 128, False, False),
    (R1344, 3, 128, True, False),
    (MID, 4, 128, False, True),
    (MID, 4, 0, True, True),
]


@pytest.mark.parametrize("cfg,bits,group,act,asym", E2E_R_CASES,
                         ids=[f"{c.name}-b{b}-g{g}-a{int(a)}-{'asym' if s else 'sym'}" for c, b, g, a, s in E2E_R_CASES])
def test_end_to_end_gates_r_form(cfg, bits, group, act, asym):
    print(f"[r-e2e] {cfg.name} bits={bits} group={group} act={act} asym={asym}", flush=True)
    W, X, W64, X64 = layer_inputs(cfg)
    if asym:
        ref = O.gptq_oracle_asym(W64, X64, bits=bits, group=group, damp=0.01, act_order=act)
    else:
        ref = O.gptq_oracle(W64, X64, bits=bits, group=group, damp=0.01, act_order=act)
    r = G.gptq_quantize(to_device(W, cfg.dtype), to_device(X, cfg.dtype), bits, group, 0.01, act,
                        G.GPTQ_FACTOR_R_FORM, asymmetric=asym)
    torch.cuda.synchronize()
    m = (compare_asym if asym else compare)(r, ref, W64, bits, group)
    print(m, flush=True)
    assert_gates(m)
    Qq = dequantized(r)[:, ref["perm"]]
    D = Qq - ref["W0"]
    quad = np.einsum("ri,ij,rj->r", D, ref["H_p"], D)
    np.testing.assert_allclose(r.row_loss.cpu().numpy(), quad, rtol=1e-4)
