"""Python binding of the GPTQ layer path: same names as the C ABI, torch tensors supply device memory and
the stream. Every step of the computation runs in libgptq_mi355x's HIP kernels.

Defaults follow the GPTQ guide's gptq() signature (herodthegreater.github.io/pigeon/guide/gptq/,
"Source code"): bits=4, no groups, damp=0.01, act_order off.
"""
from __future__ import annotations

import contextlib
import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import GPTQ_BF16, GPTQ_F32, GPTQ_FACTOR_INVERSE_RECHOL, GPTQ_FACTOR_R_FORM, GPTQ_FACTOR_REVERSED, check

__all__ = [
    "HessianState", "hessian_accumulate", "prepare_chol", "quantize_layer", "gptq_quantize", "QuantResult",
    "pack_codes", "dequant_matmul", "apply_layerwise", "QuantizedLayer", "factor_route",
    "GPTQ_FACTOR_INVERSE_RECHOL", "GPTQ_FACTOR_REVERSED", "GPTQ_FACTOR_R_FORM",
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


def _on(stream):
    """Context in which torch allocates for `stream`: the caching allocator then hands a freed block
    (a workspace dropped at return while the library's kernels may still run) only to later work on
    that same stream, which the stream orders after those kernels. None = the current stream."""
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream))
    return torch.cuda.stream(stream)


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
    """Caller-owned running sums for streaming accumulation: S (lower triangle), colsq and n_total.

    S and colsq start uninitialised: the first accumulate call (n_total == 0) writes them. Create the
    state on (or under torch.cuda.stream of) the stream that will accumulate into it."""

    def __init__(self, d_in: int, device="cuda", stream=None):
        self.d_in = d_in
        with _on(stream):
            self.S = torch.empty((d_in, d_in), dtype=torch.float64, device=device)
            self.colsq = torch.empty(d_in, dtype=torch.float64, device=device)
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
    with _on(stream):
        ws = state.workspace(n_rows, code)
    n_total = ctypes.c_int64(state.n_total)
    st = _lib.load().gptq_hessian_accumulate(
        X.data_ptr(), code, n_rows, d_in, ld, state.S.data_ptr(), state.colsq.data_ptr(), ctypes.byref(n_total),
        ws.data_ptr(), ws.numel(), _stream(stream))
    check(st, "gptq_hessian_accumulate")
    state.n_total = n_total.value
    return state


def prepare_chol(S: torch.Tensor, colsq: torch.Tensor, n_total: int, damp: float = 0.01, act_order: bool = False,
                 flags: int = GPTQ_FACTOR_REVERSED, stream=None, out=None):
    """Returns (U, perm, dead): U upper with U^T U = (P^T H P)^-1, perm int32, dead uint8."""
    _req_cuda(S, "S")
    d = S.shape[0]
    if S.shape != (d, d) or S.dtype != torch.float64 or not S.is_contiguous():
        raise ValueError("S must be a contiguous in x in float64 tensor")
    _contig(colsq, "colsq", torch.float64, (d,))
    lib = _lib.load()
    with _on(stream):
        if out is None:
            U = torch.empty((d, d), dtype=torch.float64, device=S.device)
            perm = torch.empty(d, dtype=torch.int32, device=S.device)
            dead = torch.empty(d, dtype=torch.uint8, device=S.device)
        else:
            U, perm, dead = out
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


def quantize_layer(W: torch.Tensor, U: torch.Tensor, perm: torch.Tensor, dead: torch.Tensor, bits: int = 4,
                   group: int | None = None, stream=None, ws: torch.Tensor | None = None,
                   asymmetric: bool = False, r_form: bool = False) -> QuantResult:
    """The column-by-column error-compensation loop; W (out x in) bf16 or fp32 is only read.
    asymmetric=True uses the min/max grid with a zero point (gptq_quantize_layer_ex). r_form=True: U is the
    R form of the factor (prepare_chol with GPTQ_FACTOR_R_FORM) and the loop runs from it
    (gptq_quantize_layer_r)."""
    _req_cuda(W, "W")
    ld = _ld(W, "W")
    out, d = W.shape
    _contig(U, "U", torch.float64, (d, d))
    _contig(perm, "perm", torch.int32, (d,))
    _contig(dead, "dead", torch.uint8, (d,))
    group = int(group or 0)
    n_groups = -(-d // group) if group else 1
    dev = W.device
    lib = _lib.load()
    need = (lib.gptq_quantize_r_workspace_bytes if r_form else lib.gptq_quantize_workspace_bytes)(out, d)
    with _on(stream):
        codes = torch.empty((out, d), dtype=torch.int8, device=dev)
        scales = torch.empty((out, n_groups), dtype=torch.float32, device=dev)
        g_idx = torch.empty(d, dtype=torch.int32, device=dev)
        row_loss = torch.empty(out, dtype=torch.float64, device=dev)
        if ws is None or ws.numel() < need:
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        zeros = torch.empty((out, n_groups), dtype=torch.int32, device=dev) if asymmetric else None
    grid = _lib.GPTQ_GRID_ASYMMETRIC if asymmetric else _lib.GPTQ_GRID_SYMMETRIC
    name = "gptq_quantize_layer_r" if r_form else "gptq_quantize_layer_ex"
    st = getattr(lib, name)(W.data_ptr(), _dtype_code(W), out, d, ld, U.data_ptr(), perm.data_ptr(),
                            dead.data_ptr(), int(bits), group, grid, codes.data_ptr(), scales.data_ptr(),
                            zeros.data_ptr() if zeros is not None else None, g_idx.data_ptr(),
                            row_loss.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream))
    check(st, name)
    if asymmetric:
        codes = codes.view(torch.uint8)
    return QuantResult(codes, scales, g_idx, row_loss, perm, dead, U, zeros)


def pack_codes(codes: torch.Tensor, bits: int, asymmetric: bool = False, stream=None) -> torch.Tensor:
    """Codes (out x in, as quantize_layer returns them) -> uint32 bit streams, out x ceil(in*bits/32)."""
    _req_cuda(codes, "codes")
    if codes.dim() != 2 or not codes.is_contiguous() or codes.element_size() != 1:
        raise ValueError("codes must be a contiguous 2-D int8/uint8 tensor")
    out, d = codes.shape
    lib = _lib.load()
    wpr = lib.gptq_packed_words_per_row(d, int(bits))
    if wpr <= 0:
        raise ValueError("bad in/bits")
    with _on(stream):
        packed = torch.empty((out, wpr), dtype=torch.int32, device=codes.device)
    grid = _lib.GPTQ_GRID_ASYMMETRIC if asymmetric else _lib.GPTQ_GRID_SYMMETRIC
    check(lib.gptq_pack_codes(codes.data_ptr(), out, d, int(bits), grid, packed.data_ptr(), _stream(stream)),
          "gptq_pack_codes")
    return packed


def dequant_matmul(X: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, g_idx: torch.Tensor, bits: int,
                   group: int | None = None, zeros: torch.Tensor | None = None, bias: torch.Tensor | None = None,
                   relu: bool = False, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y = X Q^T (+ bias, then ReLU when asked), fp32 n x out, with Q dequantized from packed codes, scales
    (and zeros) through g_idx."""
    _req_cuda(X, "X")
    ldx = _ld(X, "X")
    n, d = X.shape
    n_out = packed.shape[0]
    group = int(group or 0)
    n_groups = -(-d // group) if group else 1
    _contig(scales, "scales", torch.float32, (n_out, n_groups))
    _contig(g_idx, "g_idx", torch.int32, (d,))
    if zeros is not None:
        _contig(zeros, "zeros", torch.int32, (n_out, n_groups))
    if bias is not None:
        _contig(bias, "bias", torch.float32, (n_out,))
    lib = _lib.load()
    wpr = lib.gptq_packed_words_per_row(d, int(bits))
    _contig(packed, "packed", torch.int32, (n_out, wpr))
    if out is None:
        with _on(stream):
            out = torch.empty((n, n_out), dtype=torch.float32, device=X.device)
    else:
        _contig(out, "out", torch.float32, (n, n_out))
    grid = _lib.GPTQ_GRID_ASYMMETRIC if zeros is not None else _lib.GPTQ_GRID_SYMMETRIC
    st = lib.gptq_dequant_matmul(X.data_ptr(), _dtype_code(X), n, d, ldx, packed.data_ptr(), scales.data_ptr(),
                                 zeros.data_ptr() if zeros is not None else None, g_idx.data_ptr(), n_out, int(bits),
                                 grid, group, bias.data_ptr() if bias is not None else None, int(bool(relu)),
                                 out.data_ptr(), n_out, _stream(stream))
    check(st, "gptq_dequant_matmul")
    return out


def factor_route(in_features: int, group: int | None) -> int:
    """The factor route gptq_quantize takes when flags is None: the R form where the library takes it (in a
    multiple of 64; group 0 or dividing 128) and it is the faster of the two on MI355X, i.e. with one grid per
    row (its panels fold T into their steps at almost no cost) or with in >= 8192 (where leaving out L^-1
    saves more in prepare than the in-panel T_P U_PP costs the loop); otherwise the route through U.
    Measured per layer: q_proj (in 4096, group 0) 9.81 against 9.90 ms, down (in 11008, group 128) 48.2
    against 58.2 ms, up_gate (in 4096, group 128) 13.30 against 13.34 ms (a tie: the route through U)."""
    group = int(group or 0)
    if in_features % 64 != 0 or (group != 0 and 128 % group != 0):
        return GPTQ_FACTOR_REVERSED
    return GPTQ_FACTOR_R_FORM if (group == 0 or in_features >= 8192) else GPTQ_FACTOR_REVERSED


def gptq_quantize(W: torch.Tensor, X: torch.Tensor, bits: int = 4, group: int | None = None, damp: float = 0.01,
                  act_order: bool = False, flags: int | None = None, stream=None,
                  asymmetric: bool = False) -> QuantResult:
    """The whole per-layer path: accumulate the Hessian over X, prepare the factor, quantize W. flags picks
    the factor route: GPTQ_FACTOR_REVERSED (U), GPTQ_FACTOR_INVERSE_RECHOL (U by the guide's order) or
    GPTQ_FACTOR_R_FORM (the loop from R = U^-1 and U's diagonal blocks); None takes factor_route(in, group).
    Every kernel and every allocation is on `stream` (None = the current stream)."""
    if flags is None:
        flags = factor_route(W.shape[1], group)
    state = HessianState(W.shape[1], device=W.device, stream=stream)
    hessian_accumulate(X, state, stream)
    U, perm, dead = prepare_chol(state.S, state.colsq, state.n_total, damp, act_order, flags, stream)
    return quantize_layer(W, U, perm, dead, bits, group, stream, asymmetric=asymmetric,
                          r_form=(flags == GPTQ_FACTOR_R_FORM))


@dataclass
class QuantizedLayer:
    """One layer of a layer-wise quantized MLP: the quantizer's outputs and the packed codes the forward
    reads. result and packed are None for a layer kept at full precision (skip_last)."""
    result: QuantResult | None
    packed: torch.Tensor | None
    bias: torch.Tensor | None
    bits: int
    group: int


def apply_layerwise(weights, biases, X: torch.Tensor, bits: int = 4, group: int | None = None, damp: float = 0.01,
                    act_order: bool = False, asymmetric: bool = False, skip_last: bool = False,
                    flags: int | None = None, keep_inputs: bool = False, stream=None):
    """Quantize an MLP layer by layer, calibrating each layer on the outputs of the layers before it after
    they were quantized (GPTQ guide, "How it works", apply_layerwise).

    weights[i]: out_i x in_i CUDA tensor (fp32 or bf16); biases[i]: fp32 [out_i] or None; X: n x in_0.
    Each layer: Hessian of its input, the factor (route by flags, None = factor_route per layer), the
    compensation loop, packed codes; then its forward
    relu(h Q^T + b) (no ReLU on the last layer) by the dequantizing matmul, in fp32, is the next layer's
    input. Returns (layers, inputs, h): inputs[i] the tensor layer i was calibrated on (only with
    keep_inputs), h the network output, or None when the last layer is kept at full precision (its
    forward feeds nothing here)."""
    L = len(weights)
    if len(biases) != L or L == 0:
        raise ValueError("weights and biases must be non-empty lists of the same length")
    group = int(group or 0)
    h = X
    layers, inputs = [], []
    for i, W in enumerate(weights):
        last = i == L - 1
        if W.dim() != 2 or W.shape[1] != h.shape[1]:
            raise ValueError(f"layer {i}: weight shape {tuple(W.shape)} does not take inputs of width {h.shape[1]}")
        if keep_inputs:
            inputs.append(h)
        if skip_last and last:
            layers.append(QuantizedLayer(None, None, biases[i], bits, group))
            return layers, inputs, None
        res = gptq_quantize(W, h, bits, group, damp, act_order, flags, stream, asymmetric=asymmetric)
        packed = pack_codes(res.codes, bits, asymmetric, stream)
        layers.append(QuantizedLayer(res, packed, biases[i], bits, group))
        h = dequant_matmul(h, packed, res.scales, res.g_idx, bits, group, res.zeros, biases[i], relu=not last,
                           stream=stream)
    return layers, inputs, h
