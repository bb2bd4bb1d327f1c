"""Seeded synthetic layer workloads.

The GPTQ pages calibrate on real activations: the lesson page uses X of shape (N, in) with one weight
matrix W of shape (out, in); the guide's transformer paragraph ("How it works", last paragraph) uses
128 random 2048-token text segments (n about 262k) entering one linear layer; the handbook page's demo
uses W 128x256 ~ 0.1*N(0,1) and X 512x256 ~ N(0,1). Neither real text activations nor trained weights
are available here, so every workload below is drawn from numpy's PCG64 generator with the shapes and
value structure of those workloads (Gaussian tokens with a few large outlier channels, ReLU outputs
with never-firing "dead" channels and per-channel magnitudes).

Recipe (fixed, so the CPU oracle and the GPU path read identical bits):
  * W: ``default_rng([w_seed]).standard_normal((out, in), float32) * w_std`` in fp32, then encoded.
  * X structure: ``default_rng([x_seed, 0])`` draws, in this order and only when the config has them,
    the dead channels ``permutation(in)[:dead]``, the magnitudes ``lognormal(0, 1, in)`` and the
    outlier channels ``permutation(in)[:outliers]``.
  * X rows come in segments of 2048 rows; segment s is ``default_rng([x_seed, 1 + s])
    .standard_normal((rows_s, in), float32)``, then (fp32) outliers *= gain, ReLU, *= magnitudes,
    dead channels := 0. Segments make generation parallel and let callers draw any row range.
  * bf16 encoding is IEEE round-to-nearest-even of the fp32 value, kept as uint16 bit patterns.

Nothing here computes any part of the quantization method.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

SEGMENT_ROWS = 2048


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class LayerConfig:
    name: str
    out: int
    d_in: int
    n: int
    dtype: str  # storage type of W and X: "f32" or "bf16"
    w_std: float
    x_kind: str = "normal"  # "normal" or "relu"
    outlier_channels: int = 0
    outlier_gain: float = 20.0
    dead_channels: int = 0
    lognormal_magnitudes: bool = False
    bits: int = 4
    group: int = 0
    act_order: bool = False
    damp: float = 0.01
    w_seed: int = 0
    x_seed: int = 0

    @property
    def n_segments(self) -> int:
        return -(-self.n // SEGMENT_ROWS)


# The five workloads: two small ones the oracle finishes in seconds and three transformer-layer shapes.
CONFIGS = (
    # Handbook demo shape: W 128x256 ~0.1 N(0,1), X 512x256 N(0,1); 4-bit per-row scales.
    LayerConfig("tiny", 128, 256, 512, "f32", 0.1, "normal", bits=4, w_seed=1101, x_seed=1001),
    # Guide teacher-layer shape: 256 inputs, 512 calibration inputs, ReLU activations with ~5% dead.
    LayerConfig("teacher", 256, 256, 512, "f32", 1.0 / 16.0, "relu", dead_channels=13, bits=3,
                w_seed=2102, x_seed=2002),
    # Transformer q_proj: 4096x4096, 128 segments x 2048 tokens, 1% outlier channels x20.
    LayerConfig("q_proj", 4096, 4096, 262144, "bf16", 0.02, "normal", outlier_channels=41, bits=4,
                w_seed=3103, x_seed=3003),
    # MLP up/gate: 11008x4096 on the q_proj activations, group-128 scales.
    LayerConfig("up_gate", 11008, 4096, 262144, "bf16", 0.02, "normal", outlier_channels=41, bits=4,
                group=128, w_seed=4104, x_seed=3003),
    # MLP down: 4096x11008, ReLU activations with lognormal channel magnitudes and ~2% dead channels.
    LayerConfig("down", 4096, 11008, 131072, "bf16", 0.02, "relu", dead_channels=220,
                lognormal_magnitudes=True, bits=3, group=128, act_order=True, w_seed=5105, x_seed=5005),
)


def config_by_name(name: str) -> LayerConfig:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def custom_config(name: str, out: int, d_in: int, n: int, **kw) -> LayerConfig:
    """A workload of arbitrary shape with the same recipe (for parity cases and edge cases)."""
    base = LayerConfig(name, out, d_in, n, kw.pop("dtype", "f32"), kw.pop("w_std", 0.05))
    return replace(base, **kw)


def _encode(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    if dtype == "f32":
        return a32
    raise ValueError(dtype)


def gen_w(cfg: LayerConfig) -> np.ndarray:
    """W (out x in): float32 array for "f32", uint16 bf16 bit patterns for "bf16"."""
    rng = np.random.default_rng([cfg.w_seed])
    w = rng.standard_normal((cfg.out, cfg.d_in), dtype=np.float32) * np.float32(cfg.w_std)
    return _encode(w, cfg.dtype)


def _structure(cfg: LayerConfig):
    rng = np.random.default_rng([cfg.x_seed, 0])
    dead = rng.permutation(cfg.d_in)[: cfg.dead_channels] if cfg.dead_channels else None
    mags = rng.lognormal(0.0, 1.0, cfg.d_in).astype(np.float32) if cfg.lognormal_magnitudes else None
    outl = rng.permutation(cfg.d_in)[: cfg.outlier_channels] if cfg.outlier_channels else None
    return dead, mags, outl


def dead_channels(cfg: LayerConfig) -> np.ndarray:
    """Indices of the channels the recipe forces to zero (empty when none)."""
    dead, _, _ = _structure(cfg)
    return np.sort(dead) if dead is not None else np.zeros(0, dtype=np.int64)


def _segment(cfg: LayerConfig, s: int, rows: int, structure) -> np.ndarray:
    dead, mags, outl = structure
    rng = np.random.default_rng([cfg.x_seed, 1 + s])
    z = rng.standard_normal((rows, cfg.d_in), dtype=np.float32)
    if outl is not None:
        z[:, outl] *= np.float32(cfg.outlier_gain)
    if cfg.x_kind == "relu":
        np.maximum(z, np.float32(0.0), out=z)
    elif cfg.x_kind != "normal":
        raise ValueError(cfg.x_kind)
    if mags is not None:
        z *= mags[None, :]
    if dead is not None:
        z[:, dead] = 0.0
    return z


def gen_x(cfg: LayerConfig, row_start: int = 0, row_stop: int | None = None,
          threads: int | None = None) -> np.ndarray:
    """Rows [row_start, row_stop) of X (n x in), encoded as for gen_w. Segments are drawn in parallel."""
    row_stop = cfg.n if row_stop is None else min(row_stop, cfg.n)
    if not 0 <= row_start <= row_stop:
        raise ValueError("bad row range")
    structure = _structure(cfg)
    out_dtype = np.uint16 if cfg.dtype == "bf16" else np.float32
    out = np.empty((row_stop - row_start, cfg.d_in), dtype=out_dtype)
    s0, s1 = row_start // SEGMENT_ROWS, -(-row_stop // SEGMENT_ROWS)

    def work(s: int) -> None:
        seg_lo = s * SEGMENT_ROWS
        rows = min(SEGMENT_ROWS, cfg.n - seg_lo)
        z = _segment(cfg, s, rows, structure)
        lo, hi = max(seg_lo, row_start), min(seg_lo + rows, row_stop)
        out[lo - row_start: hi - row_start] = _encode(z[lo - seg_lo: hi - seg_lo], cfg.dtype)

    segs = range(s0, s1)
    nthreads = threads or min(16, os.cpu_count() or 1)
    if len(segs) <= 1 or nthreads == 1:
        for s in segs:
            work(s)
    else:
        with ThreadPoolExecutor(max_workers=nthreads) as ex:
            list(ex.map(work, segs))
    return out


def gen_layer(cfg: LayerConfig):
    """(W, X) for a config, both encoded per cfg.dtype."""
    return gen_w(cfg), gen_x(cfg)


# ------------------------------------------------------------------------------------------------
# A small MLP for the layer-wise driver (the guide's "3x256 teacher": 12 raw inputs, three hidden
# layers of 256 with ReLU, an output layer; 512 calibration inputs). The trained teacher is not
# available, so its weights are drawn:
#   * layer i (out_i x in_i): default_rng([seed, 1 + i]) draws W ~ N(0, 2 / in_i) (fp32), then the
#     bias ~ N(0, 0.1^2) (fp32); in hidden layers the first `dead` entries of permutation(out_i) get
#     bias -50, so those ReLU units never fire (the guide's dead inputs of the next layer).
#   * X: default_rng([seed, 0]).standard_normal((n, sizes[0]), float32).
# ------------------------------------------------------------------------------------------------
@dataclass(frozen=True)
class MLPConfig:
    name: str
    sizes: tuple
    n: int
    dead: int = 0
    seed: int = 0


MLP_CONFIGS = (
    MLPConfig("teacher_mlp", (12, 256, 256, 256, 2), 512, dead=6, seed=6006),
    MLPConfig("wide_mlp", (200, 640, 640, 10), 2048, dead=16, seed=7007),
)


def mlp_config_by_name(name: str) -> MLPConfig:
    for c in MLP_CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def gen_mlp(cfg: MLPConfig):
    """(weights, biases, X): fp32 arrays, weights[i] out_i x in_i, biases[i] out_i, X n x sizes[0]."""
    weights, biases = [], []
    L = len(cfg.sizes) - 1
    for i in range(L):
        d_in, d_out = cfg.sizes[i], cfg.sizes[i + 1]
        rng = np.random.default_rng([cfg.seed, 1 + i])
        w = rng.standard_normal((d_out, d_in), dtype=np.float32) * np.float32(np.sqrt(2.0 / d_in))
        b = rng.standard_normal(d_out, dtype=np.float32) * np.float32(0.1)
        if cfg.dead and i < L - 1:
            b[rng.permutation(d_out)[: cfg.dead]] = np.float32(-50.0)
        weights.append(w)
        biases.append(b)
    X = np.random.default_rng([cfg.seed, 0]).standard_normal((cfg.n, cfg.sizes[0]), dtype=np.float32)
    return weights, biases, X
