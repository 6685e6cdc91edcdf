#!/usr/bin/env python3
"""Benchmark of the quantized projection matmul on one MI355X.

Workload (one "step"): the seven Qwen3-0.6B projections of all 28 layers
(196 distinct weights, fp32 N(0, 0.02), packed once by pack_b_int8 before the
timed region: ~420 MiB of int8 codes, more than the 256 MiB Infinity Cache)
run as decode at M = 1, 16 and 32 rows of fp32 N(0, 1) activations.  Every
call is quantize_rows_int8 (per-row amax/127) followed by int8_gemm with the
fp32 epilogue (row scale x column scale).  Each M's 196 calls are captured in
one HIP graph; a step replays the three graphs.

`value` is the step's algorithmic bytes (per call K*N weight bytes + 4N column
scales + 4MK activations + 4MN outputs) over its wall time, in GB/s.
`roofline` is the int8 decode GEMM kernel alone: its algorithmic bytes per
launch (K*N + 4N + M*K + 4M + 4MN) over its average launch duration, timed
with HIP events around each launch on the launch stream.  `extra` carries the
per-M figures and the other configurations (int8 prefill at M = 2048).
`cpu_baseline` times the CPU oracle on one whole step.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, published
METRIC = "GB/s & %HBM peak at M=1/16; int8 TOPS & %MFMA peak at M=2048"


def log(msg: str) -> None:
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--layers", type=int, default=None, help="(debug) fewer layers")
    return ap.parse_args()


def call_bytes(M, K, N):
    """Algorithmic bytes of one projection call (quantize + product + epilogue)."""
    return K * N + 4 * N + 4 * M * K + 4 * M * N


def gemm_kernel_bytes(M, K, N):
    """Algorithmic bytes of one int8 decode GEMM launch."""
    return K * N + 4 * N + M * K + 4 * M + 4 * M * N


def time_launches(torch, launches):
    """GPU duration of each launch: a spin kernel holds the stream while the
    host enqueues (event, launch, event) triples, so the events bracket the
    kernels back to back with no host gap."""
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2.4e9 * 0.25))
    pairs = []
    for f in launches:
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        f()
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e-3 for a, b in pairs]


def main() -> int:
    args = parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)." % args.gpus, file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import int8_bit_weight_amd as q
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers = args.layers or wl.QWEN3_0_6B_LAYERS
    projs = wl.QWEN3_0_6B_PROJECTIONS
    rows = wl.DECODE_ROWS

    # ------------------------------------------------------------- setup ---
    log("packing %d weights" % (layers * len(projs)))
    t0 = time.perf_counter()
    packed = {}
    host_w = {}
    for l in range(layers):
        for p, (_, K, N) in enumerate(projs):
            W = wl.projection_weight(l, p)
            if not args.no_cpu_baseline:
                host_w[(l, p)] = W
            packed[(l, p)] = q.pack_b_int8(torch.from_numpy(W).to(dev))
    torch.cuda.synchronize()
    log("packed in %.1f s" % (time.perf_counter() - t0))

    calls = {}     # M -> list of (l, p, K, N, X, Xq, rs, Y)
    for M in rows:
        lst = []
        for l in range(layers):
            for p, (_, K, N) in enumerate(projs):
                X = torch.from_numpy(wl.projection_activations(M, K, seed_index=10000 + l * 16 + p)).to(dev)
                Xq = torch.empty((M, K), dtype=torch.int8, device=dev)
                rs = torch.empty((M,), dtype=torch.float32, device=dev)
                Y = torch.empty((M, N), dtype=torch.float32, device=dev)
                lst.append((l, p, K, N, X, Xq, rs, Y))
        calls[M] = lst
    ws_need = max(q.lib.qmm_int8_gemm_workspace_bytes(M, K, N) for M in rows for (_, K, N) in projs)
    ws = torch.zeros(max(ws_need, 256), dtype=torch.uint8, device=dev)

    def run_m(M):
        for (l, p, K, N, X, Xq, rs, Y) in calls[M]:
            q.quantize_rows_int8(X, out=(Xq, rs))
            q.int8_gemm(Xq, 0, packed[(l, p)], 0, out_f32=Y, row_scale=rs, ws=ws)

    # eager reference outputs, then one graph per M, checked bit for bit
    for M in rows:
        run_m(M)
    torch.cuda.synchronize()
    eager = {M: [c[7].clone() for c in calls[M]] for M in rows}
    graphs = {}
    for M in rows:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_m(M)
        graphs[M] = g
    for rep in range(2):
        for M in rows:
            for c in calls[M]:
                c[7].fill_(float("nan"))
            graphs[M].replay()
        torch.cuda.synchronize()
        for M in rows:
            for c, ref in zip(calls[M], eager[M]):
                if not torch.equal(c[7].view(torch.int32), ref.view(torch.int32)):
                    raise RuntimeError("graph replay differs from eager result (M=%d)" % M)

    step_bytes = {M: sum(call_bytes(M, K, N) for (_, _, K, N, *_r) in calls[M]) for M in rows}
    total_bytes = sum(step_bytes.values())

    # -------------------------------------------------------------- timed ---
    for _ in range(args.warmup):
        for M in rows:
            graphs[M].replay()
    torch.cuda.synchronize()
    ev = {M: [] for M in rows}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for M in rows:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            graphs[M].replay()
            b.record()
            ev[M].append((a, b))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = total_bytes / (ms_per_step * 1e-3) / 1e9
    per_m = {}
    for M in rows:
        sec = sum(a.elapsed_time(b) for a, b in ev[M]) * 1e-3 / args.steps
        per_m[M] = dict(ms=sec * 1e3, gbs=step_bytes[M] / sec / 1e9, calls=len(calls[M]))
    log("step %.3f ms, %.1f GB/s" % (ms_per_step, value))

    # ----------------------------------------- dominant kernel: int8 GEMM ---
    def mk(M, c):
        l, p, K, N, X, Xq, rs, Y = c
        return lambda: q.int8_gemm(Xq, 0, packed[(l, p)], 0, out_f32=Y, row_scale=rs, ws=ws)

    kern = {}
    tot_b, tot_t, n_launch = 0, 0.0, 0
    for M in rows:
        launches = [mk(M, c) for c in calls[M]]
        durs = []
        for _ in range(3):
            durs.append(time_launches(torch, launches))
        durs = np.min(np.array(durs), axis=0)   # best of 3 per launch
        kb = sum(gemm_kernel_bytes(M, c[2], c[3]) for c in calls[M])
        kern[M] = dict(avg_us=float(durs.mean() * 1e6), gbs=kb / float(durs.sum()) / 1e9)
        tot_b += kb
        tot_t += float(durs.sum())
        n_launch += len(launches)
    achieved = tot_b / tot_t / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "k_int8_decode", "avg_launch_us": round(tot_t / n_launch * 1e6, 3),
                "launches_per_step": n_launch}

    extra = {"per_m": {str(M): {"step_ms": round(per_m[M]["ms"], 4), "GB/s": round(per_m[M]["gbs"], 2),
                                "%HBM": round(100 * per_m[M]["gbs"] / HBM_PEAK_GBS, 2),
                                "gemm_kernel_avg_us": round(kern[M]["avg_us"], 3),
                                "gemm_kernel_GB/s": round(kern[M]["gbs"], 2)} for M in rows}}

    # --------------------------------------------- int8 prefill, M = 2048 ---
    if not args.no_extra:
        pre = {}
        for i, (K, N) in enumerate(wl.PREFILL_SHAPES):
            d = wl.prefill_inputs(K, N, seed_index=i)
            pk = q.pack_b_int8(torch.from_numpy(d["W"]).to(dev))
            A = torch.from_numpy(d["A"]).to(dev)
            rs = torch.from_numpy(d["rs"]).to(dev)
            Y = torch.empty((wl.PREFILL_M, N), dtype=torch.float32, device=dev)
            f = (lambda A=A, pk=pk, Y=Y, rs=rs: q.int8_gemm(A, 0, pk, 0, out_f32=Y, row_scale=rs))
            f()
            ts = time_launches(torch, [f] * 10)
            t = float(np.median(ts))
            tops = 2.0 * wl.PREFILL_M * K * N / t / 1e12
            pre["%dx%d" % (K, N)] = {"us": round(t * 1e6, 2), "TOPS": round(tops, 1),
                                     "%MFMA": round(100 * tops / INT8_PEAK_TOPS, 2)}
            del pk, A, Y
        extra["int8_prefill_m2048"] = pre

    # ------------------------------------------------------- CPU baseline ---
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline: oracle on one whole step")
        qb = {k: oracle.pack_b_int8(w) for k, w in host_w.items()}
        xs = {M: [c[4].cpu().numpy() for c in calls[M]] for M in rows}
        t0 = time.perf_counter()
        for M in rows:
            for c, X in zip(calls[M], xs[M]):
                Qb, sb, _ = qb[(c[0], c[1])]
                Qa, sa = oracle.quantize_rows_int8(X)
                oracle.epilogue_f64(oracle.int8_gemm_i64(Qa, 0, Qb, 0), sa, sb)
        tc = time.perf_counter() - t0
        cpu = {"value": round(total_bytes / tc / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
               "kind": "oracle",
               "sample": "one whole step (%d calls: %d layers x 7 projections x M in {1,16,32}), "
                         "%.2f s" % (sum(len(calls[M]) for M in rows), layers, tc)}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "qwen3-0.6b-projections-int8-decode", "layers": layers,
                   "projections": [p[0] for p in projs], "rows": list(rows),
                   "calls_per_step": sum(len(calls[M]) for M in rows),
                   "bytes_per_step": total_bytes, "parallelism": "single-gpu"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
