#!/usr/bin/env python3
"""Benchmark of the block-quantized weight matmul on one MI355X.

Workload ("llama7b_layer"): one 7B-like FFN weight, W 4096 x 11008 fp32 drawn
from N(0, 0.02^2), a decode activation x (11008, N(0,1)) and a prefill batch
of 512 tokens X (512 x 11008, N(0,1)); synthetic, seeded.

One step runs every part of the hot path once, on the stream torch uses:
  quantize W -> Q4_0, Q8_0, Q4_K       (fp32 read once per format)
  GEMV  Q4_0, Q8_0, Q4_K               (decode, one token)
  quantize X -> Q8_0                   (activation quantizer)
  GEMM  Q4_0 x Q8_0 activations        (prefill, int8 MFMA)
Inputs are resident in HBM before timing starts. The GEMVs read a different
copy of the packed weights at every launch, the copies together exceeding the
256 MB Infinity Cache, so they stream from HBM; the quantizers rotate fp32
copies the same way.

Timing, two passes:
  * steps: the contract's K steps, bracketed by synchronisations, wall clock
    (ms_per_step; includes the host's launch cost).
  * kernels: each kernel launched K times back to back (at least 50), with a
    HIP event before and after the batch on the launch stream. The stream is
    first filled with a GPU sleep long enough for the host to enqueue the
    whole batch behind it (checked, and lengthened if the sleep ended first),
    so the events see the GPU's own time per launch, which agrees with
    rocprofv3's kernel durations. Each kernel is timed in three such
    batches, interleaved with the others; its time is their median
    (``us``), their spread ``us_range``.

Beside the step, every other workload of the measurement plan is timed per
kernel (``kernels``): the 1024x1024 Q4_0 GEMV (latency); the 196-matrix
Qwen3-0.6B-like decode set, Q4_0 and Q8_0, as one pass: one qmat_gemv_batch
call (a few launches), and beside it the same 196 products as 196 qmat_gemv
launches, each rotating over copies of the whole set; the 11008x4096
orientation of the 7B layer; the Q4_K-style GEMV at 4096x4096 and
4096x11008 with per-row scale spread; that model's Q6_K-style output head
(151936x1024, one token's logits); the decode batch, the
Q6_K-style kernels, the other GEMM formats, the KV-cache write, and the
activation quantizer on a warm X (what a GEMM prologue would repeat once per
128-row m-tile). The prefill GEMM reads a different copy of W at every
launch as the GEMVs do, and each GEMM entry carries its VALU ceiling: the
fp32 FMAs of its scale step at the measured FMA rate.

Output: one JSON line. ``value`` is the Q4_0 GEMV's algorithmic bytes
(packed weights + x + y) divided by its mean time per launch, the headline of
the metric; the GEMM's int8 TOPS and every other kernel's rate and roofline
fraction are reported beside it.

``--summarize-pmc FETCH.csv WRITE.csv`` (no GPU) turns the counter files of
two ``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs of
``bench.py --only gemv_q4_0,copy`` into the traffic summary that later runs
report as ``roofline.traffic``.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Q4_0 GEMV achieved HBM GB/s (% of peak) at 4096×11008; Q8 GEMM int8 TOPS"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA (5.0 POPS)
FP32_FMA_TFLOPS = 78.6      # MI355X fp32 vector FMA without packed math (157.3 packed)
# fp32 FMAs of the GEMM's scale step per output and 32-element block: S*dx,
# then the accumulation (Q6_K-style: per 16-element half; the Q4_K-style
# min term runs on an fp32 MFMA)
GEMM_VALU_FMAS = {"q4_0": 2, "q8_0": 2, "q4_k": 2, "q6_k": 4}
M, K, N = 4096, 11008, 512
COLD_BYTES = 1.5 * 2 ** 30  # > 256 MB Infinity Cache, several times over
COPY_BYTES = 64 * 2 ** 20   # calibration copy for the byte counters
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_q4_0_llama7b_traffic.json")
GEMV_SRC = os.path.join(ROOT, "block_quantized_weight_qmat_amd", "csrc", "gemv.hip")
ALL_OPS = ["quantize_q4_0", "quantize_q8_0", "quantize_q4_k", "gemv_q4_0", "gemv_q8_0",
           "gemv_q4_k", "quantize_act_q8_0", "gemm_q4_0"]
# timed per kernel, not part of the step: the few-token decode batch
# (qmat_gemm with N <= 48), the Q6_K-style quantizer, GEMV and GEMM, and
# the KV-cache write of a 512-token prefill (dim 1024: 8 KV heads of 128)
# into a 16384-cell cache, Q4_0 with the per-channel bias and Q8_0 without
KV_DIM, KV_CELLS, KV_N = 1024, 16384, 512
DECODE_NS = (4, 16)
# the other decode workloads: (name, format id, workload)
GEMV_EXTRA = [("gemv_q4_0_1024x1024", 0, "gemv_1024"),
              ("gemv_q4_0_11008x4096", 0, "llama7b_1"), ("gemv_q8_0_11008x4096", 1, "llama7b_1"),
              ("gemv_q4_k_4096x4096_spread", 2, "q4k_0"),
              ("gemv_q4_k_4096x11008_spread", 2, "q4k_1"),
              # the Qwen3-0.6B-like output head (tied embedding, q6_K in the
              # pages' model file): one token's logits over the vocabulary
              ("gemv_q6_k_lm_head_151936x1024", 3, "lm_head")]
# the Qwen3-like set as one qmat_gemv_batch call, and as 196 qmat_gemv calls
TIMING_BATCHES = 3  # timed batches per kernel; the median is reported
QWEN3_OPS = ["qwen3_pass_q4_0", "qwen3_pass_q8_0", "qwen3_launches_q4_0", "qwen3_launches_q8_0"]
# prompts of a few dozen to a few hundred tokens: the same layer through
# qmat_gemm (128 x 64 tiles, or the decode batch up to 48 tokens) and through
# qmat_gemm_ws (tiles also split along K)
MID_NS = (17, 64, 192)
MID_OPS = [f"gemm_q4_0_n{n}" for n in MID_NS] + [f"gemm_ws_q4_0_n{n}" for n in MID_NS]
EXTRA_OPS = ([f"decode_q4_0_n{n}" for n in DECODE_NS] + [g[0] for g in GEMV_EXTRA] + QWEN3_OPS
             + MID_OPS
             + ["quantize_q6_k", "gemv_q6_k", "gemm_q8_0", "gemm_q4_k", "gemm_q6_k",
                "quantize_act_q8_0_warm",
                "kv_write_q4_0", "kv_write_q8_0"])


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU time for the oracle baseline sample")
    p.add_argument("--only", default="all",
                   help="comma list of ops (" + ",".join(ALL_OPS + EXTRA_OPS) + ",copy) or all")
    p.add_argument("--batch", type=int, default=0,
                   help="launches per kernel-timing batch (default max(steps, 50))")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    p.add_argument("--no-peaks", action="store_true",
                   help="skip the measured-peak kernels (libqmat_micro.so)")
    return p.parse_args()


def read_slices(buf_bytes: int, slice_bytes: int, max_launches: int = 64):
    """Launch plan for reading slice_bytes at a time out of a buffer of
    buf_bytes: (bytes per launch, a multiple of 16; stride between launch
    starts, a multiple of 4096; number of disjoint slots; launches). Launch
    i reads [i * stride, i * stride + bytes), inside the buffer."""
    n16 = slice_bytes // 16 * 16
    if n16 < 16 or n16 > buf_bytes:
        raise ValueError(f"cannot read {slice_bytes} bytes at a time from {buf_bytes}")
    stride = -(-n16 // 4096) * 4096
    slots = max(1, buf_bytes // stride)
    return n16, stride, slots, min(max_launches, slots)


def measured_peaks(torch, slice_bytes: int | None = None) -> dict:
    """This GPU's own peaks, for the rooflines beside the nominal ones: HBM
    read bandwidth over a 2 GiB buffer (beyond the 256 MB Infinity Cache),
    the dense int8 MFMA rate, the plain (non-packed) fp32 FMA rate, and the
    FMA rate of waves that share their SIMDs with int8 MFMA waves. Each is
    the best of five event-timed launches.

    With slice_bytes, also the read rate of launches that each read only
    that many bytes, back to back, from a different part of the 2 GiB
    buffer every time (so from HBM): the ceiling that a kernel streaming
    slice_bytes per launch, timed the same way (timed_batch: the launches
    queued behind a GPU sleep, so host launch gaps do not count), can reach.
    The best of four launch shapes, each the mean over a batch of
    launches."""
    import ctypes
    from block_quantized_weight_qmat_amd import binding
    path = os.path.join(os.path.dirname(binding.library_path()), "libqmat_micro.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m block_quantized_weight_qmat_amd.build`")
    lib = ctypes.CDLL(path)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.qmat_micro_read.argtypes = [P, i64, P, i32, P]
    for f in (lib.qmat_micro_mfma_i8, lib.qmat_micro_fma_f32, lib.qmat_micro_mix):
        f.argtypes = [i32, P, i32, P]
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    sp = P(stream.cuda_stream)

    def best_ms(launch):
        ts = []
        for _ in range(6):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            rc = launch()
            b.record(stream)
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"measured-peak kernel failed to launch ({rc})")
            ts.append(a.elapsed_time(b))
        return min(ts[1:])  # the first launch warms up

    read_bytes, read_grids = 2 << 30, (1024, 2048, 4096, 8192)
    buf = torch.empty(read_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty(max(read_grids) * 512, dtype=torch.int32, device=dev)
    ms = min(best_ms(lambda g=g: lib.qmat_micro_read(P(buf.data_ptr()), read_bytes,
                                                     P(out.data_ptr()), g, sp))
             for g in read_grids)
    hbm = read_bytes / ms / 1e6
    sliced = None
    if slice_bytes:
        n16, stride, slots, launches = read_slices(read_bytes, slice_bytes)

        def launch_slice(g, i):
            rc = lib.qmat_micro_read(P(buf.data_ptr() + (i % slots) * stride), n16,
                                     P(out.data_ptr()), g, sp)
            if rc != 0:
                raise RuntimeError(f"measured-peak kernel failed to launch ({rc})")

        for g in (256, 512, 1024, 2048):  # warm up every launch shape
            launch_slice(g, 0)
        torch.cuda.synchronize()
        us = {g: timed_batch(torch, lambda i, g=g: launch_slice(g, i), launches)
              for g in (256, 512, 1024, 2048)}
        g_best = min(us, key=us.get)
        sliced = {"bytes": n16, "GBs": round(n16 / us[g_best] / 1e3, 1),
                  "us": round(us[g_best], 3), "workgroups": g_best, "launches": launches}
    del buf
    grid, iters = 2048, 2000
    ms = best_ms(lambda: lib.qmat_micro_mfma_i8(iters, P(out.data_ptr()), grid, sp))
    mfma = grid * 4 * iters * 4 * 2 * 32 * 32 * 32 / ms / 1e9
    iters = 20000
    ms = best_ms(lambda: lib.qmat_micro_fma_f32(iters, P(out.data_ptr()), grid, sp))
    fma = grid * 256 * iters * 8 * 2 / ms / 1e9
    mix_grid = 1024
    ms = best_ms(lambda: lib.qmat_micro_mix(iters, P(out.data_ptr()), mix_grid, sp))
    fma_mix = mix_grid * 256 * iters * 8 * 2 / ms / 1e9
    return {"hbm_read_GBs": round(hbm, 1), "int8_mfma_TOPS": round(mfma, 1),
            "fp32_fma_TFLOPs": round(fma, 2), "fp32_fma_TFLOPs_beside_mfma": round(fma_mix, 2),
            "hbm_read_same_bytes": sliced,
            "kernels": "libqmat_micro.so: 2 GiB coalesced read (best of 1024-8192 "
                       "workgroups); the same read over the GEMV's bytes per launch, "
                       f"{launches if slice_bytes else 0} launches back to back from "
                       "distinct offsets queued behind a GPU sleep (best of 256-2048 "
                       "workgroups); 4 chains of "
                       "v_mfma_i32_32x32x32_i8 per wave; 8 chains of v_fma_f32 per lane; "
                       "half MFMA, half FMA waves per SIMD"}


def rel_l2(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(a - ref) / np.linalg.norm(ref))


def source_hash(path: str) -> str:
    """Hash of a C/HIP source's code: comments and blank space removed, so
    that editing a comment does not mark the kernel as changed."""
    with open(path, encoding="utf-8") as f:
        text = f.read()
    code = re.sub(r"//[^\n]*|/\*.*?\*/", " ", text, flags=re.S)
    code = " ".join(code.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


# ------------------------------------------------------------------ counters
def _counter_rows(path: str, counter: str) -> list:
    with open(path) as f:
        return [r for r in csv.DictReader(f) if r.get("Counter_Name") == counter]


def summarize_pmc(fetch_csv: str, write_csv: str):
    """The two runs execute the same command, so their dispatch ids match.
    The calibration copies are the copy dispatches that write COPY_BYTES
    (the same copy kernel also serves the other tensor copies)."""
    fetch = _counter_rows(fetch_csv, "FETCH_SIZE")
    write = _counter_rows(write_csv, "WRITE_SIZE")
    is_gemv = lambda r: ("gemv_kernel" in r["Kernel_Name"] or "gemv_rows_kernel" in r["Kernel_Name"]) \
        and "FmtQ4_0" in r["Kernel_Name"]
    is_copy = lambda r: "copy" in r["Kernel_Name"].lower()
    kib = COPY_BYTES / 1024.0
    copy_ids = {r["Dispatch_Id"] for r in write
                if is_copy(r) and abs(float(r["Counter_Value"]) - kib) < 0.05 * kib}
    if not copy_ids:
        raise SystemExit("no calibration copy found in the WRITE_SIZE run")
    mean = lambda rows: float(np.mean([float(r["Counter_Value"]) for r in rows]))
    cfetch = mean([r for r in fetch if r["Dispatch_Id"] in copy_ids])
    cwrite = mean([r for r in write if r["Dispatch_Id"] in copy_ids])
    gf = [r for r in fetch if is_gemv(r)]
    gw = [r for r in write if is_gemv(r)]
    if not gf or not gw:
        raise SystemExit("no Q4_0 GEMV dispatch in the counter files")
    gfetch, gwrite = mean(gf), mean(gw)
    # the counters are in KiB per dispatch; the plain copy reads and writes
    # exactly COPY_BYTES, which calibrates each counter
    f_scale = COPY_BYTES / (cfetch * 1024.0)
    w_scale = COPY_BYTES / (cwrite * 1024.0)
    out = {
        "kernel": gf[0]["Kernel_Name"],
        "gemv_src_sha256_16": source_hash(GEMV_SRC),
        "gemv_dispatches": len(gf),
        "fetch_kib_per_dispatch": gfetch,
        "write_kib_per_dispatch": gwrite,
        "copy_kernel": next(r["Kernel_Name"] for r in write if r["Dispatch_Id"] in copy_ids),
        "copy_dispatches": len(copy_ids),
        "copy_bytes": COPY_BYTES,
        "copy_fetch_kib": cfetch,
        "copy_write_kib": cwrite,
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "traffic_bytes_per_launch": gfetch * 1024.0 * f_scale + gwrite * 1024.0 * w_scale,
        "algorithmic_bytes_per_launch": M * 18 * (K // 32) + 4 * K + 4 * M,
    }
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def traffic_for_current_kernel():
    """HBM bytes per Q4_0 GEMV launch from the stored counter summary, or
    None when there is none or the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("gemv_src_sha256_16") != source_hash(GEMV_SRC):
        return None
    return float(t["traffic_bytes_per_launch"])


# ------------------------------------------------------------------ timing
def timed_batch(torch, fn, n: int, launches_per_call: int = 1) -> float:
    """Mean GPU time per call (us) of n back-to-back calls of fn(i), each
    enqueueing launches_per_call kernels."""
    stream = torch.cuda.current_stream()
    fill_us = 40.0 * n * launches_per_call
    for _ in range(5):
        torch.cuda.synchronize()
        torch.cuda._sleep(int(fill_us * 2000))  # ~2 GHz shader clock
        mark = torch.cuda.Event()
        mark.record(stream)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            fn(i)
        b.record(stream)
        starved = mark.query()  # the sleep ended before the batch was queued
        torch.cuda.synchronize()
        if not starved:
            return 1e3 * a.elapsed_time(b) / n
        fill_us *= 3
    return 1e3 * a.elapsed_time(b) / n


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(Bh, x_np, Xh, gemv_nbytes: int, seconds: float) -> dict:
    """The oracle as it stands, timed on this host's cores: the Q4_0 GEMV at
    4096 x 11008 with all OpenMP threads (median of 3 timed samples of about
    seconds/4 each) and with one thread (median of 3 single products), and
    the Q4_0 GEMM on a 256-row x 512-token sample of the prefill workload
    (median of 3)."""
    import oracle
    all_threads = oracle.num_threads()

    def rate_gemv(budget):
        reps, t = 0, 0.0
        t1 = time.perf_counter()
        while t < budget or reps == 0:
            oracle.gemv(0, Bh, x_np, M, K)
            reps += 1
            t = time.perf_counter() - t1
        return gemv_nbytes * reps / t / 1e9, reps, t

    oracle.gemv(0, Bh, x_np, M, K)  # warm up
    samples = [rate_gemv(seconds / 4) for _ in range(3)]
    med = sorted(samples)[1]
    rows = 256
    gops = []
    for _ in range(3):
        t1 = time.perf_counter()
        oracle.gemm(0, Bh[:rows], Xh, rows, K, N)
        gops.append(2.0 * rows * N * K / (time.perf_counter() - t1) / 1e9)
    one = []
    try:
        oracle.set_threads(1)
        for _ in range(3):
            t1 = time.perf_counter()
            oracle.gemv(0, Bh, x_np, M, K)
            one.append(gemv_nbytes / (time.perf_counter() - t1) / 1e9)
    finally:
        oracle.set_threads(all_threads)
    return {"value": round(med[0], 3), "unit": "GB/s", "cores": all_threads, "kind": "oracle",
            "sample": f"median of 3 samples, each {med[1]} full Q4_0 GEMVs 4096x11008 "
                      f"(dequantize to fp64, fp64 dot, OpenMP over rows, {all_threads} "
                      f"threads) in {med[2]:.1f} s; same algorithmic bytes as value",
            "one_thread_GBs": round(sorted(one)[1], 3),
            "gemm_q4_0_GOPs": round(sorted(gops)[1], 3),
            "gemm_sample": f"Q4_0 GEMM {rows} rows x {N} tokens x {K}, {all_threads} threads, "
                           "median of 3",
            "nproc": os.cpu_count(), "cpu_model": cpu_model()}


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the block-quantized GEMV/GEMM runs on a single "
              "MI355X here (a row split of W would scale it across GPUs; that is not built).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from block_quantized_weight_qmat_amd import binding, inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    only = ALL_OPS + EXTRA_OPS if args.only == "all" else args.only.split(",")

    # ------------------------------------------------------------ inputs
    W_np, x_np = inputs.llama7b_layer(0)
    _, X_np = inputs.prefill()
    Wf = torch.from_numpy(W_np).to(dev)
    x = torch.from_numpy(x_np).to(dev)
    fmts = {"q4_0": 0, "q8_0": 1, "q4_k": 2, "q6_k": 3}
    packed = {f: binding.quantize(i, Wf) for f, i in fmts.items()}
    torch.cuda.synchronize()

    def copies(t, total):
        n = max(2, math.ceil(total / (t.numel() * t.element_size())))
        return [t.clone() for _ in range(n)]

    need = lambda prefix: any(o.startswith(prefix) for o in only)
    cold = {f: copies(packed[f], COLD_BYTES) if need("gemv_" + f) or need("decode_" + f)
            or need("gemm_" + f) or need("gemm_ws_" + f) else [packed[f]] for f in fmts}
    W_rot = [Wf] + ([Wf.clone()] if need("quantize_q") else [])
    X_rot = [torch.from_numpy(X_np).to(dev) for _ in range(12 if need("quantize_act") else 1)]
    q_out = {f: torch.empty_like(packed[f]) for f in fmts}
    y = {f: torch.empty(M, dtype=torch.float32, device=dev) for f in fmts}
    Xq = binding.quantize(1, X_rot[0])
    Y = torch.empty((N, M), dtype=torch.float32, device=dev)
    Xq_dec = {n: binding.quantize(1, X_rot[0][:n].contiguous()) for n in DECODE_NS}
    Y_dec = {n: torch.empty((n, M), dtype=torch.float32, device=dev) for n in DECODE_NS}
    mid = [n for n in MID_NS if f"gemm_q4_0_n{n}" in only or f"gemm_ws_q4_0_n{n}" in only]
    Xq_mid = {n: binding.quantize(1, X_rot[0][:n].contiguous()) for n in mid}
    Y_mid = {n: torch.empty((n, M), dtype=torch.float32, device=dev) for n in mid}
    ws_mid = {n: torch.empty(binding.gemm_workspace_bytes(0, M, K, n), dtype=torch.uint8,
                             device=dev) for n in mid}
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    # the other decode workloads, packed on the GPU, each rotated over copies
    # that together exceed the Infinity Cache
    gx = {}
    for name, fi, wl in GEMV_EXTRA:
        if name not in only:
            continue
        if wl == "gemv_1024":
            Wn, xn = inputs.gemv_1024()
        elif wl.startswith("llama7b_"):
            Wn, xn = inputs.llama7b_layer(int(wl[-1]))
        elif wl == "lm_head":
            Wn, xn = inputs.qwen3_lm_head()
        else:
            Wn, xn = inputs.q4k_rows(int(wl[-1]))
        pk = binding.quantize(fi, torch.from_numpy(Wn).to(dev))
        gx[name] = (fi, copies(pk, COLD_BYTES), torch.from_numpy(xn).to(dev),
                    torch.empty(Wn.shape[0], dtype=torch.float32, device=dev), Wn.shape)
        del pk
    # the Qwen3-0.6B-like decode set: every matrix packed on the GPU; a pass
    # is one batch call (or 196 GEMV launches), and passes rotate over copies
    # of the whole set
    qwen = {}
    for name in QWEN3_OPS:
        if name not in only:
            continue
        fi = fmts[name.split("_", 2)[2]]
        mats = []
        for i in range(len(inputs.qwen3_shapes())):
            _, Wn, xn = inputs.qwen3_matrix(i)
            pk = binding.quantize(fi, torch.from_numpy(Wn).to(dev))
            mats.append((pk, torch.from_numpy(xn).to(dev), Wn.shape))
        set_bytes = sum(m[0].numel() for m in mats)
        sets = [mats] + [[(m[0].clone(), m[1], m[2]) for m in mats]
                         for _ in range(max(1, math.ceil(COLD_BYTES / set_bytes)) - 1)]
        yq = torch.empty(max(m[2][0] for m in mats), dtype=torch.float32, device=dev)
        # the batch writes every product at once: one output per matrix
        ys = [torch.empty(m[2][0], dtype=torch.float32, device=dev) for m in mats]
        jobs = [binding.gemv_jobs(fi, [(pk, xv, yv, shp[0], shp[1])
                                       for (pk, xv, shp), yv in zip(st, ys)]) for st in sets]
        qwen[name] = (fi, sets, yq, ys, jobs)
    torch.cuda.synchronize()

    rb = {f: binding.row_bytes(i, K) for f, i in fmts.items()}
    gemv_bytes = {f: M * rb[f] + 4 * K + 4 * M for f in fmts}
    quant_bytes = {f: 4 * M * K + M * rb[f] for f in fmts}
    actq_bytes = 4 * N * K + N * binding.row_bytes(1, K)
    gemm_ops = 2 * M * N * K
    dec_bytes = {n: M * rb["q4_0"] + n * binding.row_bytes(1, K) + 4 * n * M for n in DECODE_NS}

    table = {}
    for f, i in fmts.items():
        table[f"quantize_{f}"] = lambda s, f=f, i=i: binding.quantize(
            i, W_rot[s % len(W_rot)], out=q_out[f])
        table[f"gemv_{f}"] = lambda s, f=f, i=i: binding.gemv(
            i, cold[f][s % len(cold[f])], x, M, K, out=y[f])
    table["quantize_act_q8_0"] = lambda s: binding.quantize(1, X_rot[s % len(X_rot)], out=Xq)
    # the same X every launch (22.5 MB, resident in the 256 MB Infinity
    # Cache): the work a GEMM prologue would repeat once per 128-row m-tile
    table["quantize_act_q8_0_warm"] = lambda s: binding.quantize(1, X_rot[0], out=Xq)
    # W from HBM at every launch, as in a prefill that streams each layer once
    table["gemm_q4_0"] = lambda s: binding.gemm(0, cold["q4_0"][s % len(cold["q4_0"])], Xq,
                                                M, K, N, out=Y)
    for name, (fi, cps, xv, yv, shp) in gx.items():
        table[name] = lambda s, fi=fi, cps=cps, xv=xv, yv=yv, shp=shp: binding.gemv(
            fi, cps[s % len(cps)], xv, shp[0], shp[1], out=yv)

    def qwen_launches(s, fi, sets, yq):
        for pk, xv, (rows, kk) in sets[s % len(sets)]:
            binding.gemv(fi, pk, xv, rows, kk, out=yq[:rows])
    for name, (fi, sets, yq, _, jobs) in qwen.items():
        if name.startswith("qwen3_launches"):
            table[name] = lambda s, fi=fi, sets=sets, yq=yq: qwen_launches(s, fi, sets, yq)
        else:
            table[name] = lambda s, fi=fi, jobs=jobs: binding.gemv_batch(fi, jobs[s % len(jobs)])
    # the other formats write elsewhere: the Q4_0 parity check below reads Y
    Yx = torch.empty_like(Y) if any(need(f"gemm_{f}") for f in ("q8_0", "q4_k", "q6_k")) else Y
    for f, i in (("q8_0", 1), ("q4_k", 2), ("q6_k", 3)):
        table[f"gemm_{f}"] = lambda s, f=f, i=i: binding.gemm(
            i, cold[f][s % len(cold[f])], Xq, M, K, N, out=Yx)
    kv_rows = X_rot[0][:KV_N, :KV_DIM].contiguous()
    kv_bias = X_rot[0][0, KV_DIM:2 * KV_DIM].contiguous()
    kv_cache = {f: torch.empty((KV_CELLS, binding.row_bytes(i, KV_DIM)), dtype=torch.uint8,
                               device=dev) for f, i in (("q4_0", 0), ("q8_0", 1))}
    kv_bytes = {f: 4 * KV_N * KV_DIM + (4 * KV_DIM if f == "q4_0" else 0)
                + KV_N * binding.row_bytes(i, KV_DIM) for f, i in (("q4_0", 0), ("q8_0", 1))}
    table["kv_write_q4_0"] = lambda s: binding.kv_write(
        0, kv_rows, kv_cache["q4_0"], (s * KV_N) % (KV_CELLS - KV_N), bias=kv_bias)
    table["kv_write_q8_0"] = lambda s: binding.kv_write(
        1, kv_rows, kv_cache["q8_0"], (s * KV_N) % (KV_CELLS - KV_N))
    for n in DECODE_NS:
        table[f"decode_q4_0_n{n}"] = lambda s, n=n: binding.gemm(
            0, cold["q4_0"][s % len(cold["q4_0"])], Xq_dec[n], M, K, n, out=Y_dec[n])
    for n in mid:
        table[f"gemm_q4_0_n{n}"] = lambda s, n=n: binding.gemm(
            0, cold["q4_0"][s % len(cold["q4_0"])], Xq_mid[n], M, K, n, out=Y_mid[n])
        table[f"gemm_ws_q4_0_n{n}"] = lambda s, n=n: binding.gemm_ws(
            0, cold["q4_0"][s % len(cold["q4_0"])], Xq_mid[n], M, K, n, out=Y_mid[n],
            workspace=ws_mid[n])
    table["copy"] = lambda s: dst.copy_(src)
    ops = [(name, table[name]) for name in only if name not in EXTRA_OPS]
    extra = [(name, table[name]) for name in only if name in EXTRA_OPS]

    # ------------------------------------------------------------ steps
    for s in range(args.warmup):
        for _, fn in ops:
            fn(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for _, fn in ops:
            fn(args.warmup + s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # ------------------------------------------------------------ kernels
    nb = args.batch if args.batch > 0 else max(args.steps, 50)
    nq = len(inputs.qwen3_shapes())

    def batch_us(name, fn):
        if name in QWEN3_OPS:
            return timed_batch(torch, fn, max(4, nb // 10),
                               nq if name.startswith("qwen3_launches") else 8)
        return timed_batch(torch, fn, nb)

    # every kernel: the median of TIMING_BATCHES batches (one batch can
    # catch the clocks settling), the spread kept beside it
    runs_us = {name: [] for name, _ in ops + extra if name != "copy"}
    for rep in range(TIMING_BATCHES):
        for name, fn in ops + extra:
            if name != "copy":
                runs_us[name].append(batch_us(name, fn))
        print(f"[bench] timing batches {rep + 1}/{TIMING_BATCHES} done", file=sys.stderr, flush=True)
    mean_us = {name: statistics.median(r) for name, r in runs_us.items()}

    kernels = {}
    for name, us in mean_us.items():
        if name in gx:
            fi, cps, _, _, (rows, kk) = gx[name]
            nbytes = cps[0].numel() + 4 * kk + 4 * rows
            gbs = nbytes / us / 1e3
            kernels[name] = {"us": us, "bytes": nbytes, "GB/s": gbs, "bound": "hbm",
                             "frac": gbs / HBM_PEAK_GBS}
        elif name in qwen:
            mats = qwen[name][1][0]
            nbytes = sum(m[0].numel() + 4 * m[2][1] + 4 * m[2][0] for m in mats)
            gbs = nbytes / us / 1e3
            kernels[name] = {"us": us, "matrices": len(mats), "bytes": nbytes, "GB/s": gbs,
                             "bound": "hbm", "frac": gbs / HBM_PEAK_GBS,
                             "calls": len(mats) if name.startswith("qwen3_launches") else 1}
        elif name.startswith("gemv_"):
            f = name[5:]
            gbs = gemv_bytes[f] / us / 1e3
            kernels[name] = {"us": us, "bytes": gemv_bytes[f], "GB/s": gbs, "bound": "hbm",
                             "frac": gbs / HBM_PEAK_GBS}
        elif name.startswith("kv_write_"):
            f = name[9:]
            gbs = kv_bytes[f] / us / 1e3
            kernels[name] = {"us": us, "bytes": kv_bytes[f], "GB/s": gbs, "bound": "hbm",
                             "frac": gbs / HBM_PEAK_GBS}
        elif name.startswith("quantize_act"):
            gbs = actq_bytes / us / 1e3
            kernels[name] = {"us": us, "bytes": actq_bytes, "GB/s": gbs, "bound": "hbm",
                             "frac": gbs / HBM_PEAK_GBS}
            if name.endswith("_warm"):
                # a prologue-fused GEMM repeats it once per 128-row m-tile
                kernels[name]["m_tiles"] = M // 128
                kernels[name]["repeated_per_m_tile_us"] = us * (M // 128)
        elif name.startswith("quantize_"):
            f = name[9:]
            gbs = quant_bytes[f] / us / 1e3
            kernels[name] = {"us": us, "bytes": quant_bytes[f], "GB/s": gbs, "bound": "hbm",
                             "frac": gbs / HBM_PEAK_GBS}
        elif name.startswith("decode_"):
            n = int(name.rsplit("_n", 1)[1])
            gbs = dec_bytes[n] / us / 1e3
            kernels[name] = {"us": us, "bytes": dec_bytes[n], "GB/s": gbs, "bound": "hbm",
                             "frac": gbs / HBM_PEAK_GBS, "tokens_per_s": n / us * 1e6}
        elif name in MID_OPS:
            n = int(name.rsplit("_n", 1)[1])
            ops_n = 2 * M * K * n
            tops = ops_n / us / 1e6
            splits = ws_mid[n].numel() // (4 * n * M) + 1 if name.startswith("gemm_ws") else 1
            kernels[name] = {"us": us, "tokens": n, "int8_ops": ops_n, "TOPS": tops,
                             "bound": "mfma", "frac": tops / INT8_PEAK_TOPS,
                             "path": f"qmat_gemm_ws, {splits} K range(s)"
                             if name.startswith("gemm_ws") else "qmat_gemm (no workspace)"}
        elif name.startswith("gemm_"):
            tops = gemm_ops / us / 1e6
            kernels[name] = {"us": us, "int8_ops": gemm_ops, "TOPS": tops, "bound": "mfma",
                             "frac": tops / INT8_PEAK_TOPS}

    for name, k in kernels.items():
        k["us_range"] = [round(min(runs_us[name]), 3), round(max(runs_us[name]), 3)]

    # ------------------------------------------------------------ parity
    parity = {}
    if "gemv_q4_0" in mean_us or "gemm_q4_0" in mean_us:
        import oracle
        if "gemv_q4_0" in mean_us:
            ref = oracle.gemv(0, packed["q4_0"].cpu().numpy(), x_np, M, K)
            parity["gemv_q4_0_rel_l2"] = rel_l2(y["q4_0"].cpu().numpy(), ref)
        if "gemm_q4_0" in mean_us:
            rng = np.random.default_rng(1)
            rows = np.sort(rng.choice(M, 32, replace=False))
            toks = np.sort(rng.choice(N, 16, replace=False))
            # the last launch read copy (launches - 1) of W; all copies are equal
            Bh = packed["q4_0"].cpu().numpy()
            Xh = Xq.cpu().numpy()
            refY = oracle.gemm(0, Bh[rows], Xh[toks], len(rows), K, len(toks))
            parity["gemm_q4_0_sampled_rel_l2"] = rel_l2(Y.cpu().numpy()[np.ix_(toks, rows)], refY)

    # ------------------------------------------------------------ CPU oracle
    cpu = None
    if not args.no_cpu_baseline and "gemv_q4_0" in mean_us:
        cpu = cpu_baseline(packed["q4_0"].cpu().numpy(), x_np, Xq.cpu().numpy(),
                           gemv_bytes["q4_0"], args.cpu_seconds)

    peaks = None if args.no_peaks else measured_peaks(torch, gemv_bytes.get("q4_0"))
    # The GEMM's VALU ceiling: its scale step alone, at the fp32 FMA rate that
    # waves sharing their SIMD with int8 MFMA waves reach (measured), or the
    # nominal non-packed rate
    fma_rate = peaks["fp32_fma_TFLOPs_beside_mfma"] if peaks else FP32_FMA_TFLOPS
    for name, kv in kernels.items():
        if name.startswith("gemm_") and name not in MID_OPS:
            flops = 2 * GEMM_VALU_FMAS[name[5:]] * M * N * (K // 32)
            ceil_us = flops / fma_rate / 1e6
            kv.update({"valu_fma_flops": flops, "valu_ceiling_us": ceil_us,
                       "valu_rate_TFLOPs": fma_rate, "frac_of_valu_ceiling": ceil_us / kv["us"]})
    headline = kernels.get("gemv_q4_0")
    gemm = kernels.get("gemm_q4_0")
    traffic = traffic_for_current_kernel() if headline else None
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
        "dtype": "i4*i20->i32, f32 acc",
        "data": "synthetic",
        "config": {"workload": "llama7b_layer: Q4_0 GEMV W 4096x11008 (decode, one token); "
                               "prefill GEMM over 512 tokens (Q8_0 activations, int8 MFMA)",
                   "M": M, "K": K, "prefill_tokens": N, "seed": 0},
        "roofline": None if not headline else {
            "bound": "hbm", "achieved": round(headline["GB/s"], 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(headline["frac"], 4),
            "traffic": None if traffic is None else round(traffic),
            "kernel": "gemv_q4_0", "bytes_per_launch": gemv_bytes["q4_0"],
            "us_per_launch": round(headline["us"], 3),
            "frac_of_measured": None if not peaks else round(
                headline["GB/s"] / peaks["hbm_read_GBs"], 4),
            "frac_of_same_bytes_read": None if not (peaks and peaks["hbm_read_same_bytes"]) else round(
                headline["GB/s"] / peaks["hbm_read_same_bytes"]["GBs"], 4)},
        "gemm_int8_tops": None if not gemm else round(gemm["TOPS"], 1),
        "gemm_frac_of_int8_peak": None if not gemm else round(gemm["frac"], 4),
        "gemm_frac_of_measured_int8": None if not (gemm and peaks) else round(
            gemm["TOPS"] / peaks["int8_mfma_TOPS"], 4),
        "gemm_valu_ceiling": None if not gemm else {
            "us": round(gemm["valu_ceiling_us"], 3), "frac": round(gemm["frac_of_valu_ceiling"], 4),
            "fmas_per_output_block": GEMM_VALU_FMAS["q4_0"], "rate_TFLOPs": gemm["valu_rate_TFLOPs"],
            "what": "2 fp32 FMAs per (m, n, 32-block) scale step at the fp32 FMA rate measured "
                    "beside int8 MFMA waves (nominal 78.6 TFLOP/s without peaks)"},
        "measured_peaks": peaks,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "parity": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
