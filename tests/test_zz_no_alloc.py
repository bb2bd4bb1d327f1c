"""gptq_hessian_accumulate_noalloc (scratch in the library's static device array) against
gptq_hessian_accumulate (caller workspace), through the C ABI, on two calls in a row: a large first chunk
and a smaller second one that adds to it, then a fresh smaller stream. The two entry points may cut the
rows into different slices (the static scratch holds fewer), so S agrees to fp32-within-slice rounding
(relative Frobenius 1e-6, the Hessian gate), colsq to fp64 rounding, n_total exactly; both are checked
against the oracle's fp64 S too."""
import ctypes

import numpy as np
import pytest
import torch

from post_weight_quantization_05_amd import _lib
from oracle import gptq_oracle as O
import synthetic as syn
from tests.parity import to_device

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _accumulate(lib, Xd, code, S, colsq, n_total, noalloc):
    n, d = Xd.shape
    nt = ctypes.c_int64(n_total)
    if noalloc:
        st = lib.gptq_hessian_accumulate_noalloc(Xd.data_ptr(), code, n, d, Xd.stride(0), S.data_ptr(),
                                                 colsq.data_ptr(), ctypes.byref(nt), None)
    else:
        need = lib.gptq_hessian_workspace_bytes(n, d, code)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        st = lib.gptq_hessian_accumulate(Xd.data_ptr(), code, n, d, Xd.stride(0), S.data_ptr(), colsq.data_ptr(),
                                         ctypes.byref(nt), ws.data_ptr(), ws.numel(), None)
        torch.cuda.synchronize()
        del ws
    assert st == 0, _lib.status_string(st)
    return nt.value


def _rel(a, b, low):
    return float(np.linalg.norm((a - b)[low]) / np.linalg.norm(b[low]))


@pytest.mark.parametrize("name,d,n1,n2", [("bf16", 4096, 20000, 3000), ("bf16", 700, 9000, 1500),
                                          ("f32", 300, 5000, 777)])
def test_noalloc_matches_workspace_entry_point(name, d, n1, n2):
    print(f"[noalloc] {name} d={d} chunks {n1} + {n2}", flush=True)
    lib = _lib.load()
    cfg = syn.custom_config(f"na_{name}_{d}", 8, d, n1 + n2, dtype=name, w_std=0.02, outlier_channels=3,
                            w_seed=51, x_seed=52)
    X = syn.gen_x(cfg)
    Xd = to_device(X, cfg.dtype)
    code = _lib.GPTQ_BF16 if name == "bf16" else _lib.GPTQ_F32
    res = {}
    for noalloc in (False, True):
        S = torch.full((d, d), 7.0, dtype=torch.float64, device="cuda")
        colsq = torch.full((d,), -1.0, dtype=torch.float64, device="cuda")
        n = _accumulate(lib, Xd[:n1], code, S, colsq, 0, noalloc)
        n = _accumulate(lib, Xd[n1:], code, S, colsq, n, noalloc)
        torch.cuda.synchronize()
        assert n == n1 + n2
        res[noalloc] = (S.cpu().numpy(), colsq.cpu().numpy())
    low = np.tril(np.ones((d, d), dtype=bool))
    (Sa, ca), (Sb, cb) = res[False], res[True]
    assert np.all(Sb[~low] == 7.0)  # the strictly upper triangle is not touched
    assert _rel(Sb, Sa, low) <= 1e-6
    np.testing.assert_allclose(cb, ca, rtol=1e-13, atol=0)
    S_ref, c_ref, _ = O.hessian_from_x(O.to_f64(X, cfg.dtype))
    assert _rel(Sb, S_ref, low) <= 1e-6 and _rel(Sa, S_ref, low) <= 1e-6
    np.testing.assert_allclose(cb, c_ref, rtol=1e-12, atol=0)
    # a fresh stream of a smaller chunk through the same (shared) scratch
    S = torch.empty((d, d), dtype=torch.float64, device="cuda")
    colsq = torch.empty((d,), dtype=torch.float64, device="cuda")
    assert _accumulate(lib, Xd[:n2], code, S, colsq, 0, True) == n2
    torch.cuda.synchronize()
    S2_ref, c2_ref, _ = O.hessian_from_x(O.to_f64(X[:n2], cfg.dtype))
    assert _rel(S.cpu().numpy(), S2_ref, low) <= 1e-6
    np.testing.assert_allclose(colsq.cpu().numpy(), c2_ref, rtol=1e-12, atol=0)


def test_noalloc_rejects_what_the_scratch_cannot_hold():
    lib = _lib.load()
    nt = ctypes.c_int64(0)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the call fails before any launch
    st = lib.gptq_hessian_accumulate_noalloc(fake, _lib.GPTQ_BF16, 4096, 8192, 8192, fake, fake, ctypes.byref(nt), None)
    assert st == _lib.GPTQ_ERR_UNSUPPORTED and nt.value == 0
    st = lib.gptq_hessian_accumulate_noalloc(fake, _lib.GPTQ_BF16, 0, 64, 64, fake, fake, ctypes.byref(nt), None)
    assert st == _lib.GPTQ_ERR_INVALID_ARG
