"""Python binding of the GPTQ layer path: same names as the C ABI, torch tensors supply device memory and
the stream. Every step of the computation runs in libgptq_mi355x's HIP kernels.

Defaults follow the GPTQ guide's gptq() signature (herodthegreater.github.io/pigeon/guide/gptq/,
"Source code"): bits=4, no groups, damp=0.01, act_order off.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import GPTQ_BF16, GPTQ_F32, GPTQ_FACTOR_INVERSE_RECHOL, GPTQ_FACTOR_REVERSED, check

__all__ = [
    "HessianState", "hessian_accumulate", "prepare_chol", "quantize_layer", "gptq_quantize", "QuantResult",
    "GPTQ_FACTOR_INVERSE_RECHOL", "GPTQ_FACTOR_REVERSED",
]


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GPTQ_BF16
    if t.dtype == torch.float32:
        return GPTQ_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _req_cuda(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _contig(t: torch.Tensor, name: str, dtype, shape) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")


def _ld(t: torch.Tensor, name: str) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D row-major tensor with unit column stride")
    return t.stride(0)


class HessianState:
    """Caller-owned running sums for streaming accumulation: S (lower triangle), colsq and n_total."""

    def __init__(self, d_in: int, device="cuda"):
        self.d_in = d_in
        self.S = torch.zeros((d_in, d_in), dtype=torch.float64, device=device)
        self.colsq = torch.zeros(d_in, dtype=torch.float64, device=device)
        self.n_total = 0
        self._ws = None

    def workspace(self, n_rows: int, dtype_code: int) -> torch.Tensor:
        need = _lib.load().gptq_hessian_workspace_bytes(n_rows, self.d_in, dtype_code)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 1), dtype=torch.uint8, device=self.S.device)
        return self._ws


def hessian_accumulate(X: torch.Tensor, state: HessianState, stream=None) -> HessianState:
    """S += X^T X, colsq += sum x^2, n_total += rows (X: n x in, bf16 or fp32; 3-D inputs are flattened
    to tokens as the handbook's compute_hessian does)."""
    _req_cuda(X, "X")
    if X.dim() == 3:
        X = X.reshape(-1, X.shape[-1])
    ld = _ld(X, "X")
    code = _dtype_code(X)
    n_rows, d_in = X.shape
    if d_in != state.d_in:
        raise ValueError("X width does not match the state")
    ws = state.workspace(n_rows, code)
    n_total = ctypes.c_int64(state.n_total)
    st = _lib.load().gptq_hessian_accumulate(
        X.data_ptr(), code, n_rows, d_in, ld, state.S.data_ptr(), state.colsq.data_ptr(), ctypes.byref(n_total),
        ws.data_ptr(), ws.numel(), _stream(stream))
    check(st, "gptq_hessian_accumulate")
    state.n_total = n_total.value
    return state


def prepare_chol(S: torch.Tensor, colsq: torch.Tensor, n_total: int, damp: float = 0.01, act_order: bool = False,
                 flags: int = GPTQ_FACTOR_INVERSE_RECHOL, stream=None, out=None):
    """Returns (U, perm, dead): U upper with U^T U = (P^T H P)^-1, perm int32, dead uint8."""
    _req_cuda(S, "S")
    d = S.shape[0]
    if S.shape != (d, d) or S.dtype != torch.float64 or not S.is_contiguous():
        raise ValueError("S must be a contiguous in x in float64 tensor")
    _contig(colsq, "colsq", torch.float64, (d,))
    if out is None:
        U = torch.empty((d, d), dtype=torch.float64, device=S.device)
        perm = torch.empty(d, dtype=torch.int32, device=S.device)
        dead = torch.empty(d, dtype=torch.uint8, device=S.device)
    else:
        U, perm, dead = out
    lib = _lib.load()
    ws = torch.empty(max(lib.gptq_prepare_workspace_bytes(d), 1), dtype=torch.uint8, device=S.device)
    st = lib.gptq_prepare_chol(S.data_ptr(), colsq.data_ptr(), int(n_total), d, float(damp), int(bool(act_order)),
                               int(flags), U.data_ptr(), perm.data_ptr(), dead.data_ptr(), ws.data_ptr(), ws.numel(),
                               _stream(stream))
    check(st, "gptq_prepare_chol")
    return U, perm, dead


@dataclass
class QuantResult:
    codes: torch.Tensor      # out x in, original column order: int8 (symmetric) or uint8 0..2^b-1 (asymmetric)
    scales: torch.Tensor     # fp32, out x G
    g_idx: torch.Tensor      # int32[in]
    row_loss: torch.Tensor   # fp64[out]
    perm: torch.Tensor | None = None
    dead: torch.Tensor | None = None
    U: torch.Tensor | None = None
    zeros: torch.Tensor | None = None  # int32, out x G (asymmetric grid only)

    def dequantize(self) -> torch.Tensor:
        g = self.g_idx.long()
        c = self.codes.to(torch.float64)
        if self.zeros is not None:
            c = c - self.zeros.to(torch.float64)[:, g]
        return c * self.scales.to(torch.float64)[:, g]


def quantize_layer(W: torch.Tensor, U: torch.Tensor, perm: torch.Tensor, dead: torch.Tensor, bits: int = 4,
                   group: int | None = None, stream=None, ws: torch.Tensor | None = None,
                   asymmetric: bool = False) -> QuantResult:
    """The column-by-column error-compensation loop; W (out x in) bf16 or fp32 is only read.
    asymmetric=True uses the min/max grid with a zero point (gptq_quantize_layer_ex)."""
    _req_cuda(W, "W")
    ld = _ld(W, "W")
    out, d = W.shape
    _contig(U, "U", torch.float64, (d, d))
    _contig(perm, "perm", torch.int32, (d,))
    _contig(dead, "dead", torch.uint8, (d,))
    group = int(group or 0)
    n_groups = -(-d // group) if group else 1
    dev = W.device
    codes = torch.empty((out, d), dtype=torch.int8, device=dev)
    scales = torch.empty((out, n_groups), dtype=torch.float32, device=dev)
    g_idx = torch.empty(d, dtype=torch.int32, device=dev)
    row_loss = torch.empty(out, dtype=torch.float64, device=dev)
    lib = _lib.load()
    need = lib.gptq_quantize_workspace_bytes(out, d)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    zeros = torch.empty((out, n_groups), dtype=torch.int32, device=dev) if asymmetric else None
    grid = _lib.GPTQ_GRID_ASYMMETRIC if asymmetric else _lib.GPTQ_GRID_SYMMETRIC
    st = lib.gptq_quantize_layer_ex(W.data_ptr(), _dtype_code(W), out, d, ld, U.data_ptr(), perm.data_ptr(),
                                    dead.data_ptr(), int(bits), group, grid, codes.data_ptr(), scales.data_ptr(),
                                    zeros.data_ptr() if zeros is not None else None, g_idx.data_ptr(),
                                    row_loss.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream))
    check(st, "gptq_quantize_layer_ex")
    if asymmetric:
        codes = codes.view(torch.uint8)
    return QuantResult(codes, scales, g_idx, row_loss, perm, dead, U, zeros)


def gptq_quantize(W: torch.Tensor, X: torch.Tensor, bits: int = 4, group: int | None = None, damp: float = 0.01,
                  act_order: bool = False, flags: int = GPTQ_FACTOR_INVERSE_RECHOL, stream=None,
                  asymmetric: bool = False) -> QuantResult:
    """The whole per-layer path: accumulate the Hessian over X, prepare U, quantize W."""
    state = HessianState(W.shape[1], device=W.device)
    hessian_accumulate(X, state, stream)
    U, perm, dead = prepare_chol(state.S, state.colsq, state.n_total, damp, act_order, flags, stream)
    return quantize_layer(W, U, perm, dead, bits, group, stream, asymmetric=asymmetric)
