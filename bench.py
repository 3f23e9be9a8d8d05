#!/usr/bin/env python3
"""Benchmark of the block-quantized weight matmul on one MI355X.

Workload ("llama7b_layer"): one 7B-like FFN weight, W 4096 x 11008 fp32 drawn
from N(0, 0.02^2), a decode activation x (11008, N(0,1)) and a prefill batch
of 512 tokens X (512 x 11008, N(0,1)); synthetic, seeded.

One step runs every part of the hot path once, each launch on the stream
torch uses, bracketed by HIP events:
  quantize W -> Q4_0, Q8_0, Q4_K       (fp32 read once per format)
  GEMV  Q4_0, Q8_0, Q4_K               (decode, one token)
  quantize X -> Q8_0                   (activation quantizer)
  GEMM  Q4_0 x Q8_0 activations        (prefill, int8 MFMA)
Inputs are resident in HBM before timing starts. The GEMVs read a different
copy of the packed weights every step, the copies together exceeding the
256 MB Infinity Cache, so they stream from HBM; the quantizers rotate fp32
copies the same way.

Output: one JSON line. ``value`` is the Q4_0 GEMV's algorithmic bytes
(packed weights + x + y) divided by its mean event-timed duration, the
headline of the metric; the GEMM's int8 TOPS and every other kernel's rate
and roofline fraction are reported beside it.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Q4_0 GEMV achieved HBM GB/s (% of peak) at 4096×11008; Q8 GEMM int8 TOPS"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA (5.0 POPS)
M, K, N = 4096, 11008, 512
COLD_BYTES = 1.5 * 2 ** 30  # > 256 MB Infinity Cache, several times over


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU time for the oracle baseline sample")
    p.add_argument("--only", default="all",
                   help="comma list of kernels to run (for counter runs): "
                        "quantize,gemv,actq,gemm or all")
    return p.parse_args()


def rel_l2(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(a - ref) / np.linalg.norm(ref))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the block-quantized GEMV/GEMM is run on a single "
              "MI355X (a multi-GPU row split would scale it per GPU; it is not built).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from block_quantized_weight_qmat_amd import binding, inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    only = set(args.only.split(",")) if args.only != "all" else {"quantize", "gemv", "actq", "gemm"}

    # ------------------------------------------------------------ inputs
    W_np, x_np = inputs.llama7b_layer(0)
    _, X_np = inputs.prefill()
    Wf = torch.from_numpy(W_np).to(dev)
    x = torch.from_numpy(x_np).to(dev)
    fmts = {"q4_0": 0, "q8_0": 1, "q4_k": 2}
    packed = {f: binding.quantize(i, Wf) for f, i in fmts.items()}
    torch.cuda.synchronize()

    def copies(t, total):
        n = max(2, math.ceil(total / t.numel()))
        return [t.clone() for _ in range(n)]

    cold = {f: copies(packed[f], COLD_BYTES) for f in fmts}
    W_rot = [Wf.clone() for _ in range(4)] if "quantize" in only else [Wf]
    X_rot = [torch.from_numpy(X_np).to(dev) for _ in range(12 if "actq" in only else 1)]
    q_out = {f: torch.empty_like(packed[f]) for f in fmts}
    y = {f: torch.empty(M, dtype=torch.float32, device=dev) for f in fmts}
    Xq = binding.quantize(1, X_rot[0])
    Y = torch.empty((N, M), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    rb = {f: binding.row_bytes(i, K) for f, i in fmts.items()}
    gemv_bytes = {f: M * rb[f] + 4 * K + 4 * M for f in fmts}
    quant_bytes = {f: 4 * M * K + M * rb[f] for f in fmts}
    actq_bytes = 4 * N * K + N * binding.row_bytes(1, K)
    gemm_ops = 2 * M * N * K

    ops = []
    if "quantize" in only:
        for f, i in fmts.items():
            ops.append((f"quantize_{f}", lambda s, f=f, i=i: binding.quantize(
                i, W_rot[s % len(W_rot)], out=q_out[f])))
    if "gemv" in only:
        for f, i in fmts.items():
            ops.append((f"gemv_{f}", lambda s, f=f, i=i: binding.gemv(
                i, cold[f][s % len(cold[f])], x, M, K, out=y[f])))
    if "actq" in only:
        ops.append(("quantize_act_q8_0", lambda s: binding.quantize(1, X_rot[s % len(X_rot)], out=Xq)))
    if "gemm" in only:
        ops.append(("gemm_q4_0", lambda s: binding.gemm(0, packed["q4_0"], Xq, M, K, N, out=Y)))

    def run(steps, offset, timed):
        evs = {name: [] for name, _ in ops}
        for s in range(steps):
            for name, fn in ops:
                if timed:
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record()
                    fn(s + offset)
                    b.record()
                    evs[name].append((a, b))
                else:
                    fn(s + offset)
        return evs

    run(args.warmup, 0, timed=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs = run(args.steps, args.warmup, timed=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    mean_us = {name: 1e3 * float(np.mean([a.elapsed_time(b) for a, b in v])) for name, v in evs.items()}

    # back-to-back GEMV launches (no events between): average includes the
    # dispatch gaps, i.e. what a decode loop of such GEMVs would see
    b2b = {}
    if "gemv" in only:
        for f, i in fmts.items():
            n = 4 * len(cold[f])
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for s in range(n):
                binding.gemv(i, cold[f][s % len(cold[f])], x, M, K, out=y[f])
            b.record()
            torch.cuda.synchronize()
            b2b[f] = 1e3 * a.elapsed_time(b) / n

    # ------------------------------------------------------------ rates
    kernels = {}
    for name, us in mean_us.items():
        if name.startswith("gemv_"):
            f = name[5:]
            gbs = gemv_bytes[f] / us / 1e3
            kernels[name] = {"us": us, "bytes": gemv_bytes[f], "GB/s": gbs, "bound": "hbm",
                             "frac": gbs / HBM_PEAK_GBS}
            if f in b2b:
                kernels[name]["us_back_to_back"] = b2b[f]
                kernels[name]["GB/s_back_to_back"] = gemv_bytes[f] / b2b[f] / 1e3
        elif name.startswith("quantize_act"):
            gbs = actq_bytes / us / 1e3
            kernels[name] = {"us": us, "bytes": actq_bytes, "GB/s": gbs, "bound": "hbm",
                             "frac": gbs / HBM_PEAK_GBS}
        elif name.startswith("quantize_"):
            f = name[9:]
            gbs = quant_bytes[f] / us / 1e3
            kernels[name] = {"us": us, "bytes": quant_bytes[f], "GB/s": gbs, "bound": "hbm",
                             "frac": gbs / HBM_PEAK_GBS}
        elif name.startswith("gemm_"):
            tops = gemm_ops / us / 1e6
            kernels[name] = {"us": us, "int8_ops": gemm_ops, "TOPS": tops, "bound": "mfma",
                             "frac": tops / INT8_PEAK_TOPS}

    # ------------------------------------------------------------ parity
    parity = {}
    import oracle
    if "gemv" in only:
        ref = oracle.gemv(0, packed["q4_0"].cpu().numpy(), x_np, M, K)
        parity["gemv_q4_0_rel_l2"] = rel_l2(y["q4_0"].cpu().numpy(), ref)
    if "gemm" in only:
        rng = np.random.default_rng(1)
        rows = np.sort(rng.choice(M, 32, replace=False))
        toks = np.sort(rng.choice(N, 16, replace=False))
        Bh = packed["q4_0"].cpu().numpy()
        Xh = Xq.cpu().numpy()
        refY = oracle.gemm(0, Bh[rows], Xh[toks], len(rows), K, len(toks))
        parity["gemm_q4_0_sampled_rel_l2"] = rel_l2(Y.cpu().numpy()[np.ix_(toks, rows)], refY)

    # ------------------------------------------------------------ CPU oracle
    cpu = None
    if not args.no_cpu_baseline and "gemv" in only:
        Bh = packed["q4_0"].cpu().numpy()
        reps, t_cpu = 0, 0.0
        t1 = time.perf_counter()
        while t_cpu < args.cpu_seconds:
            oracle.gemv(0, Bh, x_np, M, K)
            reps += 1
            t_cpu = time.perf_counter() - t1
        cpu = {"value": gemv_bytes["q4_0"] * reps / t_cpu / 1e9, "unit": "GB/s",
               "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"{reps} full Q4_0 GEMVs 4096x11008 (dequantize to fp64, fp64 dot), "
                         f"{t_cpu:.1f} s, same algorithmic bytes as the GPU figure"}

    headline = kernels.get("gemv_q4_0")
    gemm = kernels.get("gemm_q4_0")
    out = {
        "metric": METRIC,
        "value": round(headline["GB/s"], 1) if headline else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * wall / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "llama7b_layer: Q4_0 W 4096x11008 decode GEMV; prefill GEMM "
                               "over 512 tokens (Q8_0 activations, int8 MFMA)",
                   "M": M, "K": K, "prefill_tokens": N, "seed": 0},
        "roofline": None if not headline else {
            "bound": "hbm", "achieved": round(headline["GB/s"], 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(headline["frac"], 4), "traffic": None,
            "kernel": "gemv_q4_0"},
        "gemm_int8_tops": None if not gemm else round(gemm["TOPS"], 1),
        "gemm_frac_of_int8_peak": None if not gemm else round(gemm["frac"], 4),
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "parity": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
