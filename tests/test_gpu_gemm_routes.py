"""GPU parity of the library's test build in which every fp64 product takes the chunked-ring GEMM and the
factorization forms L^-1 by the level-wise doubling.

The main library sends small products (at most 1024 tiles, small K) to single-shot kernels, so at the
sizes the other tests use, the chunked ring's lower-triangle branch (the factorization's update of the
next outer block) only runs for in > 16640; and it forms L^-1 inside the factorization's steps up to
in = 6144, by the doubling levels above. libgptq_mi355x_ringonly.so is the same source built with both
cutoffs at 0; here it runs the prepare cases (ragged sizes, both factorization routes, act_order) and a
quantize case through its C ABI, against the CPU oracle.
"""
import numpy as np
import pytest
import torch

import post_weight_quantization_05_amd as G
from post_weight_quantization_05_amd import _lib, build
from oracle import gptq_oracle as O
import synthetic as syn
from tests.parity import dev64, layer_inputs, to_device

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


@pytest.fixture(scope="module")
def ring():
    return _lib.load(build.VARIANT_LIB)


def _prepare(lib, S, colsq, n, damp, act, flags):
    d = S.shape[0]
    U = torch.empty((d, d), dtype=torch.float64, device="cuda")
    perm = torch.empty(d, dtype=torch.int32, device="cuda")
    dead = torch.empty(d, dtype=torch.uint8, device="cuda")
    ws = torch.empty(lib.gptq_prepare_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    st = lib.gptq_prepare_chol(S.data_ptr(), colsq.data_ptr(), n, d, damp, int(act), flags, U.data_ptr(),
                               perm.data_ptr(), dead.data_ptr(), ws.data_ptr(), ws.numel(), None)
    assert st == 0, _lib.status_string(st)
    torch.cuda.synchronize()
    return U.cpu().numpy(), perm.cpu().numpy(), dead.cpu().numpy().astype(bool)


@pytest.mark.parametrize("d", [1, 65, 257, 513, 577, 1000])
@pytest.mark.parametrize("flags", [G.GPTQ_FACTOR_REVERSED, G.GPTQ_FACTOR_INVERSE_RECHOL], ids=["reversed", "rechol"])
def test_prepare_through_the_chunked_ring(ring, d, flags):
    print(f"[ring] prepare d={d} flags={flags}", flush=True)
    rng = np.random.default_rng(700 + d)
    X = rng.standard_normal((3 * d + 2, d)) @ (np.eye(d) + 0.2 * rng.standard_normal((d, d)))
    S, colsq, n = O.hessian_from_x(X)
    H_p, perm, dead, lam = O.prepare(S, colsq, n, 0.01, True)
    U_ref = O.upper_factor_of_inverse(H_p)
    U, p, dd = _prepare(ring, dev64(S), dev64(colsq), n, 0.01, True, flags)
    assert np.array_equal(p, perm) and np.array_equal(dd, dead)
    assert np.all(np.tril(U, -1) == 0.0)
    assert np.linalg.norm(U - U_ref) / np.linalg.norm(U_ref) <= 1e-10


def test_quantize_through_the_chunked_ring(ring):
    """Quantize (K = 128 in-block updates on the chunked ring) given the oracle's U; codes must equal the
    oracle's up to forced-replay-valid near-ties, scales and loss to fp64 rounding."""
    cfg = syn.custom_config("ring_q", 48, 1100, 3000, dtype="bf16", w_std=0.02, outlier_channels=5,
                            w_seed=41, x_seed=42)
    W, X, W64, X64 = layer_inputs(cfg)
    S, colsq, n = O.hessian_from_x(X64)
    H_p, perm, dead, lam = O.prepare(S, colsq, n, 0.01, True)
    U = O.upper_factor_of_inverse(H_p)
    codes_q, scales, errs, loss = O.compensation_loop(O.start_weights(W64, perm, dead), U, 4, 128)
    codes, g_idx, Q = O.finalize(codes_q, scales, perm, 128)
    out, d = W.shape
    Wd = to_device(W, cfg.dtype)
    Ud, pd, dd = dev64(U), dev64(perm.astype(np.int32)), dev64(dead.astype(np.uint8))
    c = torch.empty((out, d), dtype=torch.int8, device="cuda")
    s = torch.empty((out, -(-d // 128)), dtype=torch.float32, device="cuda")
    gi = torch.empty(d, dtype=torch.int32, device="cuda")
    rl = torch.empty(out, dtype=torch.float64, device="cuda")
    ws = torch.empty(ring.gptq_quantize_workspace_bytes(out, d), dtype=torch.uint8, device="cuda")
    st = ring.gptq_quantize_layer(Wd.data_ptr(), G.GPTQ_BF16, out, d, d, Ud.data_ptr(), pd.data_ptr(),
                                  dd.data_ptr(), 4, 128, c.data_ptr(), s.data_ptr(), gi.data_ptr(), rl.data_ptr(),
                                  ws.data_ptr(), ws.numel(), None)
    assert st == 0, _lib.status_string(st)
    torch.cuda.synchronize()
    gc = c.cpu().numpy().astype(np.int64)
    assert np.array_equal(gi.cpu().numpy(), g_idx)
    mism = int(np.sum(gc != codes))
    if mism:
        dist, _ = O.forced_replay(O.start_weights(W64, perm, dead), U, 4, 128, gc[:, perm])
        assert dist.max() <= 0.5 + 1e-9, (mism, dist.max())
    assert mism <= 0.001 * gc.size
    np.testing.assert_allclose(s.cpu().numpy(), scales.astype(np.float32), rtol=2e-7)
    np.testing.assert_allclose(rl.cpu().numpy(), loss, rtol=1e-9)
