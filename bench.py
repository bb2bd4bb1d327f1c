#!/usr/bin/env python3
"""Benchmark of one GPTQ layer quantization on one MI355X.

A step is one pass of the whole path on the q_proj workload (W 4096 x 4096 bf16, X 262144 x 4096 bf16 =
128 segments x 2048 tokens, 4-bit per-row scales, damp 0.01): accumulate X^T X over all rows (the first
accumulate call writes S, so no zeroing pass is needed), prepare the factor, run the compensation loop. By
default the factor is in its R form (R = U^-1, the Cholesky factor of the reversed H, with U's 128 x 128
diagonal blocks) and the loop runs from it (gptq_quantize_layer_r); --factor reversed times the route through
U itself; with the R route the line also carries the same layer timed through U (`route_through_u`, after
the R route's steps; --single-route skips it). Inputs are resident in HBM before timing starts.
Prints ONE JSON line (see the fields below). `--gpus N` with N > 1 exits: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms per layer-quantize (4096², n=262k) + % MFMA/HBM roofline, at 1 GPU"
PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA
PEAK_FP64_TFLOPS = 78.6    # MI355X fp64 (vector = matrix rate)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="q_proj", help="workload name (q_proj, up_gate, down, tiny, teacher)")
    ap.add_argument("--factor", choices=["rechol", "reversed", "rform"], default="rform",
                    help="rform (default): prepare writes R = U^-1 with U's 128 x 128 diagonal blocks and the loop "
                         "runs from it (inputs a multiple of 64, group 0 or dividing 128; other workloads take "
                         "reversed); reversed: U by one Cholesky and one triangular inverse; rechol: U as the "
                         "Cholesky factor of the explicit inverse")
    ap.add_argument("--single-route", action="store_true",
                    help="skip the second timing of the layer through U that the R route's line carries "
                         "(route_through_u), e.g. for kernel traces of one route")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=65536)
    ap.add_argument("--cpu-loop-rows", type=int, default=64)
    ap.add_argument("--no-streamed-hessian", action="store_true",
                    help="skip the second Hessian figure (the same rows as 2048-row calls), e.g. for kernel traces")
    ap.add_argument("--mode", choices=["layer", "hessian", "copy"], default="layer",
                    help="layer: the timed benchmark; hessian: only the accumulate calls (for counter "
                         "passes); copy: a plain 1 GiB device copy (calibrates FETCH_SIZE/WRITE_SIZE)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_xtx_bf16_dma_q_proj_traffic.md")
HESSIAN_SRC = os.path.join(ROOT, "post_weight_quantization_05_amd", "csrc", "hessian.hip")


def hessian_traffic():
    """HBM bytes per launch of the Hessian kernel from the committed counter summary (FETCH_SIZE and
    WRITE_SIZE scaled by a plain-copy calibration), or None when that summary was taken on a different
    version of the kernel source than the one built here."""
    import hashlib
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith(("#", "|", " ")):
                    k, v = line.split(":", 1)
                    fields[k.strip().strip("`*- ")] = v.strip().strip("`* ")
        with open(HESSIAN_SRC, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
        if fields.get("source_sha256") != sha:
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def host_info():
    """CPU model (lscpu) and numpy's BLAS, for the CPU-baseline record."""
    import io
    import subprocess
    from contextlib import redirect_stdout

    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    blas = None
    try:
        cfg = np.show_config(mode="dicts")
        b = (cfg or {}).get("Build Dependencies", {}).get("blas", {})
        blas = " ".join(str(b.get(k, "")) for k in ("name", "version", "openblas configuration")).strip() or None
    except TypeError:  # older numpy: text only
        buf = io.StringIO()
        with redirect_stdout(buf):
            np.show_config()
        blas = buf.getvalue().split("blas", 1)[-1][:80].strip() or None
    return model, blas


def cpu_baseline(cfg, W, X, sample_rows, loop_rows):
    """The oracle as it stands, timed on this host on a bounded sample of the workload; the stage times
    are extrapolated to one whole layer (the sample is stated in the record)."""
    from oracle import gptq_oracle as O

    t_all = time.perf_counter()
    rows = min(sample_rows, cfg.n)
    X64 = O.to_f64(X[:rows], cfg.dtype)
    t0 = time.perf_counter()
    S, colsq, n = O.hessian_from_x(X64)
    t_hess = (time.perf_counter() - t0) * (cfg.n / rows)
    del X64
    t0 = time.perf_counter()
    H_p, perm, dead, lam = O.prepare(S, colsq, n, cfg.damp, cfg.act_order)
    U = O.upper_factor_of_inverse(H_p)
    t_factor = time.perf_counter() - t0
    lr = min(loop_rows, cfg.out)
    W64 = O.to_f64(W[:lr], cfg.dtype)
    t0 = time.perf_counter()
    W0 = O.start_weights(W64, perm, dead)
    O.compensation_loop(W0, U, cfg.bits, cfg.group)
    t_loop = (time.perf_counter() - t0) * (cfg.out / lr)
    total_ms = (t_hess + t_factor + t_loop) * 1e3
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    model, blas = host_info()
    return {
        "value": round(total_ms, 1),
        "unit": "ms",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"extrapolated from a sampled run of the numpy fp64 oracle: X^T X over {rows} of {cfg.n} rows "
                   f"(time x{cfg.n / rows:g}), inv+cholesky at full in={cfg.d_in} (not scaled), the sweep on {lr} "
                   f"of {cfg.out} rows (time x{cfg.out / lr:g}; a per-row Python loop, one core); "
                   f"sampled run took {time.perf_counter() - t_all:.1f} s"),
        "cpu_model": model,
        "numpy_blas": blas,
        "stages_ms": {"hessian": round(t_hess * 1e3, 1), "factor": round(t_factor * 1e3, 1),
                      "loop": round(t_loop * 1e3, 1)},
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this GPTQ layer path runs on one GPU; --gpus {args.gpus} is not supported "
              f"(rows of W and calibration tokens would shard across GPUs; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    import post_weight_quantization_05_amd as G
    import synthetic as syn

    G.load()  # fails loudly when the HIP library is missing
    if args.mode == "copy":
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes_per_copy": n, "copies": max(1, args.steps)}), flush=True)
        return
    cfg = syn.config_by_name(args.config)
    if args.factor == "rform" and (cfg.d_in % 64 or (cfg.group and 128 % cfg.group)):
        print(f"bench: the R form does not take in = {cfg.d_in}, group = {cfg.group}; running the reversed route",
              file=sys.stderr, flush=True)
        args.factor = "reversed"
    flags = {"reversed": G.GPTQ_FACTOR_REVERSED, "rechol": G.GPTQ_FACTOR_INVERSE_RECHOL,
             "rform": G.GPTQ_FACTOR_R_FORM}[args.factor]
    t0 = time.perf_counter()
    W = syn.gen_w(cfg)
    X = syn.gen_x(cfg)
    gen_s = time.perf_counter() - t0

    def dev(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    Wd, Xd = dev(W), dev(X)
    torch.cuda.synchronize()
    d, out = cfg.d_in, cfg.out
    st = G.HessianState(d)
    st.workspace(cfg.n, G.GPTQ_BF16 if cfg.dtype == "bf16" else G.GPTQ_F32)
    U = torch.empty((d, d), dtype=torch.float64, device="cuda")
    perm = torch.empty(d, dtype=torch.int32, device="cuda")
    dead = torch.empty(d, dtype=torch.uint8, device="cuda")
    lib = G.load()
    qws_bytes = (lib.gptq_quantize_r_workspace_bytes if flags == G.GPTQ_FACTOR_R_FORM
                 else lib.gptq_quantize_workspace_bytes)(out, d)
    qws = torch.empty(qws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(record, fl, ev):
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if record else None
        if record:
            marks[0].record(stream)
        st.n_total = 0  # the first accumulate call writes S and colsq (no zeroing pass)
        if record:
            marks[1].record(stream)
        G.hessian_accumulate(Xd, st)
        if record:
            marks[2].record(stream)
        G.prepare_chol(st.S, st.colsq, st.n_total, cfg.damp, cfg.act_order, fl, out=(U, perm, dead))
        if record:
            marks[3].record(stream)
        res = G.quantize_layer(Wd, U, perm, dead, cfg.bits, cfg.group, ws=qws, r_form=(fl == G.GPTQ_FACTOR_R_FORM))
        if record:
            marks[4].record(stream)
            for i, k in enumerate(("zero", "hessian", "prepare", "quantize")):
                ev[k].append((marks[i], marks[i + 1]))
        return res

    def run_route(fl):
        """W untimed steps, then K steps between two events on the stream; ms per step, mean stage times
        (HIP events) and the host wall time of the timed steps."""
        ev = {k: [] for k in ("zero", "hessian", "prepare", "quantize")}
        for _ in range(args.warmup):
            step(False, fl, ev)
        torch.cuda.synchronize()
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        t_start.record(stream)
        wall0 = time.perf_counter()
        for _ in range(args.steps):
            step(True, fl, ev)
        t_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        stage_ms = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in ev.items()}
        return t_start.elapsed_time(t_end) / args.steps, stage_ms, wall

    def streamed_hessian_ms(reps=3):
        """The same accumulation as 2048-row calls (the workload's segments), on the same stream: the
        first call writes S, the others add to it. Median of `reps` passes over all of X, HIP events."""
        seg = 2048
        ws = st.workspace(seg, G.GPTQ_BF16 if cfg.dtype == "bf16" else G.GPTQ_F32)
        times = []
        for _ in range(reps):
            a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            st.n_total = 0
            a.record(stream)
            for r0 in range(0, cfg.n, seg):
                G.hessian_accumulate(Xd[r0:r0 + seg], st)
            b_.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b_))
        del ws
        return float(np.median(times)), -(-cfg.n // seg)

    if args.mode == "hessian":
        for _ in range(max(1, args.steps)):
            st.n_total = 0
            G.hessian_accumulate(Xd, st)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "hessian", "config": cfg.name, "launches": max(1, args.steps)}), flush=True)
        return

    ms_per_step, stage_ms, wall = run_route(flags)

    # algorithmic work (lower triangle of X^T X, the two-step factor, the loop's multiply-adds)
    n = cfg.n
    hess_flops = n * d * (d + 1)
    # the factor's algorithmic work: Cholesky and triangular inverse (2/3 d^3) on the reversed route, twice that
    # with the inverse and its re-factorization; the R form needs the Cholesky factor only (1/3 d^3)
    factor_flops = {G.GPTQ_FACTOR_REVERSED: 2.0 / 3.0, G.GPTQ_FACTOR_INVERSE_RECHOL: 4.0 / 3.0,
                    G.GPTQ_FACTOR_R_FORM: 1.0 / 3.0}[flags] * d ** 3
    loop_flops = out * d * (d - 1)
    x_bytes = n * d * (2 if cfg.dtype == "bf16" else 4)
    hess_ms = stage_ms["hessian"]
    achieved = hess_flops / (hess_ms * 1e-3) / 1e12
    bound_ms = (hess_flops / (PEAK_BF16_TFLOPS * 1e12) + factor_flops / (PEAK_FP64_TFLOPS * 1e12)
                + loop_flops / (PEAK_FP64_TFLOPS * 1e12)) * 1e3

    def stage_roof(flops, ms, peak):
        # one stage against the peak of the arithmetic it is bound by (all three are compute-bound: their
        # algorithmic bytes take far less time at 8 TB/s than their flops at the peak)
        ach = flops / (ms * 1e-3) / 1e12
        return {"algorithmic_flop": float(f"{flops:.4e}"), "bound_ms": round(flops / (peak * 1e12) * 1e3, 4),
                "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s", "frac": round(ach / peak, 4)}
    line = {
        "metric": METRIC,
        "value": round(ms_per_step, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 products, fp32 accumulation, fp64 after the Hessian",
        "data": "synthetic (seeded; shapes and value structure of the workload)",
        "config": {"workload": f"{cfg.name}: W {out}x{d} {cfg.dtype}, X {n}x{d} {cfg.dtype} "
                               f"({cfg.n_segments} x 2048 tokens), {cfg.bits}-bit, group {cfg.group}, "
                               f"act_order {cfg.act_order}, damp {cfg.damp}",
                   "factor_route": args.factor},
        "roofline": {
            "kernel": "k_xtx_bf16_dma (Hessian X^T X, lower triangle)",
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": hessian_traffic() if cfg.name == "q_proj" else None,  # counters taken on q_proj only
            "algorithmic_per_launch": f"{hess_flops:.4e} flop (n*in*(in+1)), {x_bytes:.4e} B of X",
            "launch_ms": round(hess_ms, 4),
        },
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "stages_roofline": {
            "hessian": stage_roof(hess_flops, stage_ms["hessian"], PEAK_BF16_TFLOPS),
            "prepare": stage_roof(factor_flops, stage_ms["prepare"], PEAK_FP64_TFLOPS),
            "quantize": stage_roof(loop_flops, stage_ms["quantize"], PEAK_FP64_TFLOPS),
        },
        "weights_per_s": round(out * d / (ms_per_step * 1e-3), 1),
        "combined_bound_ms": round(bound_ms, 4),
        "frac_of_combined_bound": round(bound_ms / ms_per_step, 4),
        "wall_s_timed": round(wall, 3),
        "gen_s": round(gen_s, 2),
    }
    if flags == G.GPTQ_FACTOR_R_FORM and not args.single_route:
        # the same layer through U itself (one Cholesky and one triangular inverse, the loop subtracting
        # Err U), timed the same way after the R route, for comparison
        u_ms, u_stages, _ = run_route(G.GPTQ_FACTOR_REVERSED)
        u_bound = bound_ms + (2.0 / 3.0 - 1.0 / 3.0) * d ** 3 / (PEAK_FP64_TFLOPS * 1e12) * 1e3
        line["route_through_u"] = {"factor_route": "reversed", "ms_per_step": round(u_ms, 4),
                                   "stages_ms": {k: round(v, 4) for k, v in u_stages.items()},
                                   "combined_bound_ms": round(u_bound, 4),
                                   "frac_of_combined_bound": round(u_bound / u_ms, 4)}
    if cfg.n >= 2048 and not args.no_streamed_hessian:
        s_ms, calls = streamed_hessian_ms()
        line["hessian_streamed"] = {"calls": calls, "rows_per_call": 2048, "ms": round(s_ms, 4),
                                    "achieved_tflops": round(hess_flops / (s_ms * 1e-3) / 1e12, 1),
                                    "frac_of_bf16_peak": round(hess_flops / (s_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, W, X, args.cpu_sample_rows, args.cpu_loop_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
