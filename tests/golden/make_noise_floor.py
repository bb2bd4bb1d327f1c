"""Write the oracle's own noise floor for a full-size workload to tests/golden/noise_floor_<name>.json.

The floor answers: how far does the CPU oracle move from itself when only the precision of its Hessian
path changes? Modes, each against the fp64 run on the same rows:
  * fp32_segment_S_<m>: X^T X summed in fp32 within each segment of m rows (one single-precision BLAS
    product per segment), the segments combined in fp64; the calibration set of the transformer
    workloads is 128 (or 64) segments of 2048 tokens (GPTQ guide, "How it works").
  * fp32_chain_S_<c>x<g>: the plainest fp32 accumulation: a sequential fp32 running sum over chains of
    c rows, g rows per step, one rounding per step, chains combined in fp64 (oracle.fp32_chain_block).
    With c the slice length of the library's Hessian kernel and g = 8 this is the arithmetic of that
    kernel's matrix-core accumulation (a bf16 32x32x16 step adds its 16 products as two rounded halves
    of 8: on small cases the model's S equals the kernel's on 85-99 % of entries, against 4-9 % for
    other step sizes).
  * fp32_U: the fp64 U rounded to fp32 before the sweep.
Reported per mode: the fraction f of codes that change, the relative Frobenius change of the
dequantized Q, and the relative change of the layer output error. Rows of W are independent given U
(guide, "How it works"), so a seeded sample of rows stands for the layer; the full-size GPU test checks
the GPU on the same rows and reads this file for them.

This script calls only oracle/ and synthetic/ (numpy on the CPU). Usage, from the repository root:
    python tests/golden/make_noise_floor.py down [--rows 256] [--seg-rows 2048 16384] [--chain-rows 4000]
        [--group-rows 8]
The `down` workload takes about half an hour on 8 cores and about 16 GB of memory.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import multiprocessing as mp

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import gptq_oracle as O  # noqa: E402
import synthetic as syn  # noqa: E402

CHUNK = 16384  # rows widened to fp64 at a time (memory only; the sums are the oracle's own)


def sample_rows(out: int, count: int, seed: int = 505) -> np.ndarray:
    """The rows the floor and the full-size GPU test use: a seeded sample plus the first and last row."""
    rows = np.random.default_rng(seed).choice(out, min(count, out), replace=False)
    return np.unique(np.concatenate([rows, [0, out - 1]]))


def hessians(cfg, seg_rows_list):
    """fp64 S and, per segment length, the fp32-segment S, in one pass over the synthetic X."""
    d = cfg.d_in
    S64, colsq = np.zeros((d, d)), np.zeros(d)
    S32 = {m: np.zeros((d, d)) for m in seg_rows_list}
    c32 = np.zeros(d)
    for r0 in range(0, cfg.n, CHUNK):
        blk = O.to_f64(syn.gen_x(cfg, r0, min(cfg.n, r0 + CHUNK)), cfg.dtype)
        O.accumulate(S64, colsq, blk)
        for m in seg_rows_list:
            if CHUNK % m:
                raise ValueError("segment length must divide the chunk")
            O.accumulate_fp32_segments(S32[m], c32 if m == seg_rows_list[0] else np.zeros(d), blk, m)
        print(f"  rows {r0 + blk.shape[0]}/{cfg.n}", flush=True)
    return S64, colsq, S32


_X = None  # the workload's X (bf16 bits or fp32), shared with the pool's forked workers


def _chain_blocks(args):
    """Worker: the fp32-chain sums of a list of 256 x 256 blocks of X^T X (single-threaded BLAS)."""
    blocks, chain_rows, group_rows, dtype = args
    from threadpoolctl import threadpool_limits
    out = []
    with threadpool_limits(1):
        for i0, j0 in blocks:
            XI = O.to_f64(_X[:, i0:i0 + 256], dtype)
            XJ = XI if i0 == j0 else O.to_f64(_X[:, j0:j0 + 256], dtype)
            out.append((i0, j0, O.fp32_chain_block(XI, XJ, chain_rows, group_rows)))
    return out


def chain_hessian(cfg, chain_rows, group_rows, workers):
    """S under the fp32-chain model, computed block by block in a process pool (lower triangle)."""
    global _X
    _X = syn.gen_x(cfg)
    d = cfg.d_in
    blocks = [(i0, j0) for i0 in range(0, d, 256) for j0 in range(0, i0 + 1, 256)]
    jobs = [(blocks[k::workers * 4], chain_rows, group_rows, cfg.dtype) for k in range(workers * 4)]
    S = np.zeros((d, d))
    t0 = time.time()
    with mp.get_context("fork").Pool(workers) as pool:
        for done, res in enumerate(pool.imap_unordered(_chain_blocks, jobs)):
            for i0, j0, b in res:
                S[i0:i0 + b.shape[0], j0:j0 + b.shape[1]] = b
            print(f"  chain blocks: {done + 1}/{len(jobs)} job lists, {time.time() - t0:.0f} s", flush=True)
    _X = None
    S[np.triu_indices(d, 1)] = 0.0  # diagonal blocks computed whole; keep the lower triangle
    return S


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("name")
    ap.add_argument("--rows", type=int, default=256)
    ap.add_argument("--seg-rows", type=int, nargs="*", default=[2048, 16384])
    ap.add_argument("--chain-rows", type=int, nargs="*", default=[])
    ap.add_argument("--group-rows", type=int, default=8)
    ap.add_argument("--workers", type=int, default=os.cpu_count() or 8)
    args = ap.parse_args()
    cfg = syn.config_by_name(args.name)
    t0 = time.time()
    rows = sample_rows(cfg.out, args.rows)
    W = O.to_f64(syn.gen_w(cfg)[rows], cfg.dtype)
    S64, colsq, S32 = hessians(cfg, args.seg_rows)
    for c in args.chain_rows:
        S32[("chain", c)] = chain_hessian(cfg, c, args.group_rows, args.workers)
    print(f"Hessians in {time.time() - t0:.0f} s", flush=True)
    path = os.path.join(HERE, f"noise_floor_{cfg.name}.json")
    modes = {}
    if os.path.exists(path):  # keep the modes of earlier runs on the same rows
        with open(path) as f:
            old = json.load(f)
        if old.get("rows") == [int(r) for r in rows]:
            modes.update(old.get("modes", {}))
    ref = O.quantize_rows(W, S64, colsq, cfg.n, cfg.bits, cfg.group, cfg.damp, cfg.act_order)
    for key, Sm in S32.items():
        alt = O.quantize_rows(W, Sm, colsq, cfg.n, cfg.bits, cfg.group, cfg.damp, cfg.act_order)
        name = f"fp32_chain_S_{key[1]}x{args.group_rows}" if isinstance(key, tuple) else f"fp32_segment_S_{key}"
        modes[name] = O.drift(ref, alt, W, S64)
        if isinstance(key, tuple):
            # the model's codes where they differ from the fp64 run's: [sample row index, column, code]
            r_i, c_i = np.nonzero(alt["codes"] != ref["codes"])
            modes[name]["codes_that_differ"] = [[int(a), int(b), int(alt["codes"][a, b])] for a, b in zip(r_i, c_i)]
        print(f"{name}: {modes[name]}  ({time.time() - t0:.0f} s)", flush=True)
    alt = O.quantize_rows(W, S64, colsq, cfg.n, cfg.bits, cfg.group, cfg.damp, cfg.act_order, u_round=np.float32)
    modes["fp32_U"] = O.drift(ref, alt, W, S64)
    print(f"fp32_U: {modes['fp32_U']}", flush=True)
    rec = {
        "workload": cfg.name,
        "shape": {"out": cfg.out, "in": cfg.d_in, "n": cfg.n, "bits": cfg.bits, "group": cfg.group,
                  "act_order": cfg.act_order, "damp": cfg.damp},
        "rows": [int(r) for r in rows],
        "modes": modes,
        "oracle_e_rel_on_rows": O.relative_output_error(W, ref["Q"], S64),
        "command": (f"python tests/golden/make_noise_floor.py {args.name} --rows {args.rows} --seg-rows "
                    + " ".join(str(m) for m in args.seg_rows) + " --chain-rows "
                    + " ".join(str(c) for c in args.chain_rows) + f" --group-rows {args.group_rows}"),
        "host": {"machine": platform.machine(), "numpy": np.__version__, "cpus": os.cpu_count()},
        "seconds": round(time.time() - t0, 1),
    }
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(f"wrote {path}")


if __name__ == "__main__":
    main()
