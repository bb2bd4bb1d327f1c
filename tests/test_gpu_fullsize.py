"""GPU parity at the workloads' full sizes (q_proj 4096x4096 n=262144; up_gate 11008x4096 on the same
tokens; down 4096x11008 n=131072), in the launch configuration bench.py times (one accumulate call over
all rows, one prepare, one quantize).

Full-size outputs are checked where the CPU oracle can compute them one by one:
  * S: sampled entries against fp64 dot products of the same bf16 columns; colsq for every column;
  * U: stage isolation on an oracle-computed S of a row subset (the oracle's U is the reference);
  * codes: rows are independent given U, so the oracle runs its loop on sampled rows;
  * end to end (all three): the oracle's fp64 Hessian over all rows, its U, and its loop on sampled rows,
    against the GPU's own full path; gates C-1..C-4 on those rows, C-4 beside the oracle's noise floor
    where a file under tests/golden/ holds one.
The second quantize route (the R form of the factor, gptq_quantize_layer_r) is checked the same way on
q_proj and down, stage by stage and end to end.
"""
import json
import os
import time

import numpy as np
import pytest
import torch

import post_weight_quantization_05_amd as G
from oracle import gptq_oracle as O
import synthetic as syn
from tests.parity import TAU, dev64, plan_rows_per_slice, to_device

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

_CACHE = {}


def _x(name):
    cfg = syn.config_by_name(name)
    key = (cfg.x_seed, cfg.n, cfg.d_in)
    if key not in _CACHE:
        _CACHE.clear()
        t = time.time()
        _CACHE[key] = syn.gen_x(cfg)
        print(f"[fullsize] generated X {cfg.n}x{cfg.d_in} in {time.time() - t:.1f}s", flush=True)
    return _CACHE[key]


def _sample_pairs(d, rng, n=160):
    edges = [0, 1, 127, 128, 255, 256, 257, d // 2, d - 257, d - 256, d - 2, d - 1]
    ii = list(rng.integers(0, d, n)) + edges
    jj = list(rng.integers(0, d, n)) + edges[::-1]
    pairs = [(max(a, b), min(a, b)) for a, b in zip(ii, jj)] + [(e, e) for e in edges]
    return sorted(set((int(a), int(b)) for a, b in pairs))


@pytest.mark.parametrize("name", ["q_proj", "down"])
def test_fullsize_hessian_sampled(name):
    cfg = syn.config_by_name(name)
    print(f"[fullsize] hessian {name}", flush=True)
    X = _x(name)
    st = G.HessianState(cfg.d_in)
    G.hessian_accumulate(to_device(X, cfg.dtype), st)
    torch.cuda.synchronize()
    assert st.n_total == cfg.n
    rng = np.random.default_rng(7)
    pairs = _sample_pairs(cfg.d_in, rng)
    cols = sorted(set(a for a, _ in pairs) | set(b for _, b in pairs))
    Xc = {c: O.to_f64(X[:, c], cfg.dtype) for c in cols}
    idx_i = torch.tensor([a for a, _ in pairs], device="cuda")
    idx_j = torch.tensor([b for _, b in pairs], device="cuda")
    S_s = st.S[idx_i, idx_j].cpu().numpy()
    colsq = st.colsq.cpu().numpy()
    worst = 0.0
    for (a, b), s_gpu in zip(pairs, S_s):
        ref = float(Xc[a] @ Xc[b])
        scale = np.sqrt(float(Xc[a] @ Xc[a]) * float(Xc[b] @ Xc[b])) or 1.0
        worst = max(worst, abs(s_gpu - ref) / scale)
    print(f"[fullsize] {name}: worst sampled |dS|/sqrt(Sii Sjj) = {worst:.2e}", flush=True)
    assert worst <= 2e-5
    # colsq for every column, exact up to fp64 summation order
    ref_c = np.zeros(cfg.d_in)
    for r0 in range(0, cfg.n, 16384):
        blk = O.to_f64(X[r0:r0 + 16384], cfg.dtype)
        ref_c += np.einsum("ki,ki->i", blk, blk)
    assert np.max(np.abs(colsq - ref_c) / np.maximum(ref_c, 1e-300)) <= 1e-12
    assert np.array_equal(colsq == 0, ref_c == 0)


def _oracle_u_from_rows(cfg, rows, act_order):
    X = _x(cfg.name)
    S, colsq, n = O.hessian_from_x(O.to_f64(X[:rows], cfg.dtype))
    H_p, perm, dead, lam = O.prepare(S, colsq, n, cfg.damp, act_order)
    U = O.upper_factor_of_inverse(H_p)
    return S, colsq, n, H_p, perm, dead, U


@pytest.mark.parametrize("name,rows,flags", [("q_proj", 8192, G.GPTQ_FACTOR_INVERSE_RECHOL),
                                             ("q_proj", 8192, G.GPTQ_FACTOR_REVERSED),
                                             ("down", 16384, G.GPTQ_FACTOR_REVERSED)])
def test_fullsize_prepare_and_quantize_given_oracle_s(name, rows, flags):
    cfg = syn.config_by_name(name)
    print(f"[fullsize] prepare+quantize {name} rows={rows} flags={flags}", flush=True)
    t = time.time()
    S, colsq, n, H_p, perm, dead, U_ref = _oracle_u_from_rows(cfg, rows, cfg.act_order)
    print(f"[fullsize] oracle S/U in {time.time() - t:.1f}s", flush=True)
    U, p, dd = G.prepare_chol(dev64(S), dev64(colsq), n, cfg.damp, cfg.act_order, flags)
    assert np.array_equal(p.cpu().numpy(), perm)
    assert np.array_equal(dd.cpu().numpy().astype(bool), dead)
    Ug = U.cpu().numpy()
    rel = np.linalg.norm(Ug - U_ref) / np.linalg.norm(U_ref)
    print(f"[fullsize] {name}: |U - U_oracle| / |U_oracle| = {rel:.2e}", flush=True)
    assert rel <= (1e-10 if cfg.d_in <= 4096 else 1e-9)
    # quantize the full W with the oracle's U; check sampled rows against the oracle loop
    W = syn.gen_w(cfg)
    r = G.quantize_layer(to_device(W, cfg.dtype), dev64(U_ref), dev64(perm.astype(np.int32)),
                         dev64(dead.astype(np.uint8)), cfg.bits, cfg.group)
    torch.cuda.synchronize()
    _check_sampled_rows(cfg, W, r, perm, dead, U_ref)


def _check_sampled_rows(cfg, W, r, perm, dead, U_ref):
    """Codes (C-1, C-3 where they differ), g_idx, scales and the row loss of sampled rows against the
    oracle loop run with U_ref."""
    rows_s = np.random.default_rng(3).choice(cfg.out, 12, replace=False)
    rows_s = np.unique(np.concatenate([rows_s, [0, cfg.out - 1]]))
    W64 = O.to_f64(W[rows_s], cfg.dtype)
    W0 = O.start_weights(W64, perm, dead)
    codes_q, scales, errs, loss = O.compensation_loop(W0, U_ref, cfg.bits, cfg.group)
    codes, g_idx, Q = O.finalize(codes_q, scales, perm, cfg.group)
    gc = r.codes.cpu().numpy()[rows_s].astype(np.int64)
    mism = int(np.sum(gc != codes))
    if mism:
        dist, _ = O.forced_replay(W0, U_ref, cfg.bits, cfg.group, gc[:, perm])
        assert dist.max() <= 0.5 + 1e-9, (mism, dist.max())
    assert mism <= 0.001 * gc.size
    assert np.array_equal(r.g_idx.cpu().numpy(), g_idx)
    np.testing.assert_allclose(r.scales.cpu().numpy()[rows_s], scales.astype(np.float32), rtol=2e-7)
    np.testing.assert_allclose(r.row_loss.cpu().numpy()[rows_s], loss, rtol=1e-8)


@pytest.mark.parametrize("name,rows", [("q_proj", 8192), ("down", 16384)])
def test_fullsize_r_form_prepare_and_quantize_given_oracle_s(name, rows):
    """The R route at full size, stage by stage: prepare's R form (R = U^-1 in the upper triangle, U's
    128 x 128 diagonal blocks reversed below it) against the oracle's, then gptq_quantize_layer_r given
    the oracle's R form, on sampled rows against the oracle loop run with the oracle's U."""
    cfg = syn.config_by_name(name)
    print(f"[fullsize] R route prepare+quantize {name} rows={rows}", flush=True)
    S, colsq, n, H_p, perm, dead, U_ref = _oracle_u_from_rows(cfg, rows, cfg.act_order)
    M_ref = O.r_form(H_p)
    M, p, dd = G.prepare_chol(dev64(S), dev64(colsq), n, cfg.damp, cfg.act_order, G.GPTQ_FACTOR_R_FORM)
    assert np.array_equal(p.cpu().numpy(), perm)
    assert np.array_equal(dd.cpu().numpy().astype(bool), dead)
    Mg = M.cpu().numpy()
    tol = 1e-10 if cfg.d_in <= 4096 else 1e-9
    up, lo = np.triu(M_ref), np.tril(M_ref, -1)
    rel_up = np.linalg.norm(np.triu(Mg) - up) / np.linalg.norm(up)
    rel_lo = np.linalg.norm(np.tril(Mg, -1) - lo) / np.linalg.norm(lo)
    print(f"[fullsize] {name}: R part rel {rel_up:.2e}, U blocks rel {rel_lo:.2e}", flush=True)
    assert rel_up <= tol and rel_lo <= tol
    del M
    W = syn.gen_w(cfg)
    r = G.quantize_layer(to_device(W, cfg.dtype), dev64(M_ref), dev64(perm.astype(np.int32)),
                         dev64(dead.astype(np.uint8)), cfg.bits, cfg.group, r_form=True)
    torch.cuda.synchronize()
    _check_sampled_rows(cfg, W, r, perm, dead, U_ref)


def _oracle_s64(cfg):
    """The oracle's fp64 S and colsq over all rows of the workload's X (cached for the module)."""
    key = ("S64", cfg.x_seed, cfg.d_in)
    if key not in _CACHE:
        X = _x(cfg.name)
        S = np.zeros((cfg.d_in, cfg.d_in))
        colsq = np.zeros(cfg.d_in)
        t = time.time()
        for r0 in range(0, cfg.n, 16384):
            O.accumulate(S, colsq, O.to_f64(X[r0:r0 + 16384], cfg.dtype))
            print(f"[fullsize] oracle S: {min(cfg.n, r0 + 16384)}/{cfg.n} rows, {time.time() - t:.0f} s", flush=True)
        for k in [k for k in _CACHE if isinstance(k, tuple) and k[0] == "S64"]:
            del _CACHE[k]
        _CACHE[key] = (S, colsq)
    return _CACHE[key]


def _floor(name):
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", f"noise_floor_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        return json.load(f)


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name,flags", [("q_proj", G.GPTQ_FACTOR_REVERSED), ("q_proj", G.GPTQ_FACTOR_R_FORM),
                                        ("up_gate", G.GPTQ_FACTOR_REVERSED), ("down", G.GPTQ_FACTOR_REVERSED),
                                        ("down", G.GPTQ_FACTOR_R_FORM)],
                         ids=["q_proj", "q_proj-rform", "up_gate", "down", "down-rform"])
def test_fullsize_end_to_end_sampled_rows(name, flags):
    """The GPU's whole path at full size against the oracle's whole path (fp64 Hessian over all rows)
    on sampled rows: C-1 code agreement, C-3 forced replay, C-4 dequantized Q, C-2 output error, and for
    act_order + groups (down) perm and g_idx identical. Where a noise-floor file exists (the oracle's own
    drift under an fp32-accumulated Hessian, tests/golden/make_noise_floor.py), its rows are the ones
    checked and its floor is printed beside C-4."""
    cfg = syn.config_by_name(name)
    print(f"[fullsize] end-to-end {name} flags={flags}", flush=True)
    X = _x(name)
    W = syn.gen_w(cfg)
    r = G.gptq_quantize(to_device(W, cfg.dtype), to_device(X, cfg.dtype), cfg.bits, cfg.group, cfg.damp,
                        cfg.act_order, flags)
    torch.cuda.synchronize()
    gperm = r.perm.cpu().numpy()
    gg = r.g_idx.cpu().numpy()
    fl = _floor(name)
    if fl is not None:
        rows_s = np.array(fl["rows"])
    else:
        rows_s = np.unique(np.concatenate([np.random.default_rng(5).choice(cfg.out, 24, replace=False),
                                           [0, cfg.out - 1]]))
    gc = r.codes.cpu().numpy()[rows_s].astype(np.int64)
    gs = r.scales.cpu().numpy()[rows_s].astype(np.float64)
    del r
    torch.cuda.empty_cache()
    t = time.time()
    S, colsq = _oracle_s64(cfg)
    H_p, perm, dead, lam = O.prepare(S, colsq, cfg.n, cfg.damp, cfg.act_order)
    U = O.upper_factor_of_inverse(H_p)
    print(f"[fullsize] oracle fp64 Hessian + U in {time.time() - t:.1f}s", flush=True)
    W64 = O.to_f64(W[rows_s], cfg.dtype)
    W0 = O.start_weights(W64, perm, dead)
    parts = []
    for k0 in range(0, len(rows_s), 32):  # rows are independent given U: sweep them in chunks
        parts.append(O.compensation_loop(W0[k0:k0 + 32], U, cfg.bits, cfg.group))
        print(f"[fullsize] oracle sweep: {min(len(rows_s), k0 + 32)}/{len(rows_s)} rows, {time.time() - t:.0f} s",
              flush=True)
    codes_q, scales = np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])
    codes, g_idx, Q = O.finalize(codes_q, scales, perm, cfg.group)
    assert np.array_equal(gperm, perm)
    assert np.array_equal(gg, g_idx)
    agree = float(np.mean(gc == codes))
    Qg = gc * gs[:, gg]
    q_rel = float(np.linalg.norm(Qg - Q) / np.linalg.norm(Q))
    e_g, e_o = O.output_error(W64, Qg, S), O.output_error(W64, Q, S)
    dist = np.concatenate([O.forced_replay(W0[k0:k0 + 32], U, cfg.bits, cfg.group, gc[k0:k0 + 32, perm])[0]
                           for k0 in range(0, len(rows_s), 32)])
    print(f"[fullsize] {name}: rows {len(rows_s)} agree {agree:.7f} ({int(np.sum(gc != codes))} codes differ) "
          f"q_rel {q_rel:.2e} out_rel {abs(e_g - e_o) / e_o:.2e} replay excess {dist.max() - 0.5:.2e}", flush=True)
    assert agree >= 0.999
    assert dist.max() <= 0.5 + TAU
    assert abs(e_g - e_o) <= 0.01 * e_o
    if q_rel <= 1e-3:
        return
    # C-4 above 1e-3: by the noise-floor reading it must lie within the oracle's own
    # drift when its Hessian is summed as the kernel sums it: fp32 chains of the kernel's slice length,
    # 8 rows per rounding step (oracle.fp32_chain_block), combined in fp64
    rps = plan_rows_per_slice(cfg.n, cfg.d_in)
    key = f"fp32_chain_S_{rps}x8"
    assert fl is not None and key in fl["modes"], f"no noise floor for fp32 chains of {rps} rows"
    floor = fl["modes"][key]
    model = codes.copy()  # the model-accumulation oracle's codes: the fp64 run's, where they differ patched
    for r_i, c_i, v in floor["codes_that_differ"]:
        model[r_i, c_i] = v
    agree_model = float(np.mean(gc == model))
    print(f"[fullsize] {name}: noise floor {key}: {floor['mismatches']} codes differ, q_rel {floor['q_rel']:.2e}; "
          f"GPU vs that model's codes: agree {agree_model:.7f} ({int(np.sum(gc != model))} differ); "
          f"segment floors {json.dumps({k: v['q_rel'] for k, v in fl['modes'].items() if k.startswith('fp32_seg')})}",
          flush=True)
    # one realization of the same random near-tie flips on each side: allow twice the floor
    assert q_rel <= 2.0 * floor["q_rel"]
    assert agree_model >= agree  # the GPU is at least as close to the fp32 model as to the fp64 oracle
