#!/usr/bin/env python3
"""Benchmark of the quantized projection matmul on one MI355X.

Workload (one "step"): the seven Qwen3-0.6B projections of all 28 layers
(196 distinct weights, fp32 N(0, 0.02), packed once by pack_b_int8 before the
timed region: ~420 MiB of int8 codes, more than the 256 MiB Infinity Cache)
run as decode at M = 1, 16 and 32 rows of fp32 N(0, 1) activations.  Every
call is int8_gemm_dynamic: per-row amax/127 quantisation of the activations
(inside the int8 product kernel when the rows cut into 1, 2, 4 or 8 groups give
M' * K <= 16384 with M' = rows per group rounded up to a power of two <= 16, a
separate kernel otherwise) and the int8 product with the fp32 epilogue (row
scale x column scale).  Each M's 196 calls are
captured in one HIP graph; a step replays the three graphs.

`value` is the step's algorithmic bytes (per call K*N weight bytes + 4N column
scales + 4MK activations + 4MN outputs) over its wall time, in GB/s.
`roofline` is the dominant kernel, the int8 decode GEMM (k_int8_decode_q with
the quantisation inside, k_int8_decode on pre-quantised rows): its
algorithmic bytes per launch (K*N + 4N + 4MK + 4MN with the activations
quantised inside; K*N + 4N + MK + 4M + 4MN on pre-quantised rows) over its
average launch time from graphs of its launches alone (HIP events on the
replay stream, dispatch gaps included).  `extra` carries the
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


# HBM traffic of the dominant kernel per launch, from two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE) of `bench.py --probe --no-cpu-baseline`, each
# scaled by what the counter reads for the probe's 1 GiB device copy (FETCH_SIZE
# x 2.0, WRITE_SIZE x 1.0).  Valid only for the kernel sources it was taken on.
MEASURED_TRAFFIC = {"sources_sha1": "6ab42b7448f671a4659fdb238afb51f26ce78a39", "bytes_per_launch": 3244656}


def decode_traffic():
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha1()
    for f in ("k_int8.hip", "int8_common.h", "qmm_internal.h", "api.cpp"):
        with open(os.path.join(here, "int8_bit_weight_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return MEASURED_TRAFFIC["bytes_per_launch"] if h.hexdigest() == MEASURED_TRAFFIC["sources_sha1"] else None


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
    ap.add_argument("--probe", action="store_true",
                    help="counter probe: one 1 GiB device copy (the calibration kernel), then each decode "
                         "call of one step once, eagerly; for rocprofv3 --pmc runs")
    return ap.parse_args()


def fused_quant(M, K):
    """int8_gemm_dynamic quantises inside the product kernel (one launch; the
    rows in 1, 2, 4 or 8 groups of M' <= 16 rows with M' * K <= 16384)."""
    if K > 4096:
        return False
    for g in (1, 2, 4, 8):
        r = -(-M // g)
        e = 1
        while e < r:
            e <<= 1
        if e <= 16 and e * K <= 16384:
            return True
    return False


def call_bytes(M, K, N):
    """Algorithmic bytes of one projection call (quantize + product + epilogue)."""
    return K * N + 4 * N + 4 * M * K + 4 * M * N


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

    calls = {}     # M -> list of (l, p, K, N, X, Y)
    for M in rows:
        lst = []
        for l in range(layers):
            for p, (_, K, N) in enumerate(projs):
                X = torch.from_numpy(wl.projection_activations(M, K, seed_index=10000 + l * 16 + p)).to(dev)
                Y = torch.empty((M, N), dtype=torch.float32, device=dev)
                lst.append((l, p, K, N, X, Y))
        calls[M] = lst

    def run_m(M):
        for (l, p, K, N, X, Y) in calls[M]:
            q.int8_gemm_dynamic(X, packed[(l, p)], out_f32=Y)

    if args.probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        for M in rows:
            run_m(M)
        torch.cuda.synchronize()
        print(json.dumps({"probe": "copy 1073741824 bytes, then %d decode calls" %
                          sum(len(calls[M]) for M in rows),
                          "decode_algorithmic_bytes": {str(M): sum(call_bytes(M, c[2], c[3]) for c in calls[M])
                                                       for M in rows}}))
        return 0

    # eager reference outputs, then one graph per M, checked bit for bit
    for M in rows:
        run_m(M)
    torch.cuda.synchronize()
    eager = {M: [c[5].clone() for c in calls[M]] for M in rows}
    graphs = {}
    for M in rows:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_m(M)
        graphs[M] = g
    for rep in range(2):
        for M in rows:
            for c in calls[M]:
                c[5].fill_(float("nan"))
            graphs[M].replay()
        torch.cuda.synchronize()
        for M in rows:
            for c, ref in zip(calls[M], eager[M]):
                if not torch.equal(c[5].view(torch.int32), ref.view(torch.int32)):
                    raise RuntimeError("graph replay differs from eager result (M=%d)" % M)

    step_bytes = {M: sum(call_bytes(M, c[2], c[3]) for c in calls[M]) for M in rows}
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
        per_m[M] = dict(sec=sec, gbs=step_bytes[M] / sec / 1e9, calls=len(calls[M]))
    log("step %.3f ms, %.1f GB/s" % (ms_per_step, value))

    # Dominant kernel: the int8 decode GEMM.  A call is one launch of it with
    # the activations quantised inside (fused_quant) or the row quantiser
    # plus it.  Its average launch time is
    # taken from graphs holding only its launches, replayed back to back and
    # timed with HIP events on the replay stream (so the short dispatch gaps
    # between launches are included).
    kern_b, kern_t, n_launch = 0, 0.0, 0
    kern = {}
    for M in rows:
        pre = []
        kb = 0
        for (l, p, K, N, X, Y) in calls[M]:
            if fused_quant(M, K):
                pre.append((packed[(l, p)], X, None, Y))
                kb += call_bytes(M, K, N)
            else:
                Xq, rs = q.quantize_rows_int8(X)
                pre.append((packed[(l, p)], Xq, rs, Y))
                kb += K * N + 4 * N + M * K + 4 * M + 4 * M * N
        torch.cuda.synchronize()

        def run_kernels(pre=pre):
            for (pk, A, rs, Y) in pre:
                if rs is None:
                    q.int8_gemm_dynamic(A, pk, out_f32=Y)
                else:
                    q.int8_gemm(A, 0, pk, 0, out_f32=Y, row_scale=rs)
        run_kernels()
        gk = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gk):
            run_kernels()
        gk.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            gk.replay()
        b.record()
        torch.cuda.synchronize()
        sec = a.elapsed_time(b) * 1e-3 / args.steps
        kern[M] = dict(us=sec / len(calls[M]) * 1e6, gbs=kb / sec / 1e9)
        kern_b += kb
        kern_t += sec
        n_launch += len(calls[M])
    achieved = kern_b / kern_t / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": decode_traffic(),
                "kernel": "int8 decode GEMM (k_int8_decode_q, k_int8_decode)",
                "algorithmic_bytes_per_launch": round(kern_b / n_launch),
                "avg_launch_us": round(kern_t / n_launch * 1e6, 3), "launches_per_step": n_launch}

    extra = {"per_m": {str(M): {"step_ms": round(per_m[M]["sec"] * 1e3, 4), "GB/s": round(per_m[M]["gbs"], 2),
                                "%HBM": round(100 * per_m[M]["gbs"] / HBM_PEAK_GBS, 2),
                                "call_us": round(per_m[M]["sec"] / per_m[M]["calls"] * 1e6, 3),
                                "decode_kernel_us": round(kern[M]["us"], 3),
                                "decode_kernel_GB/s": round(kern[M]["gbs"], 2)}
                       for M in rows}}

    # ---------------- the same projections with shared inputs fused ---
    # q, k and v read the same activations, and so do gate and up: packing
    # their weights side by side (per-column packing makes the codes, scales
    # and column sums those of the separate packs) gives 4 calls per layer
    # instead of 7, with the same output columns bit for bit.
    if not args.no_extra:
        groups = ((0, 1, 2), (3,), (4, 5), (6,))
        fpk = {}
        for l in range(layers):
            for gi, grp in enumerate(groups):
                W = np.concatenate([wl.projection_weight(l, p) for p in grp], axis=1)
                fpk[(l, gi)] = q.pack_b_int8(torch.from_numpy(W).to(dev))
        fused = {}
        for M in rows:
            lst, fb = [], 0
            for l in range(layers):
                for gi, grp in enumerate(groups):
                    K = projs[grp[0]][1]
                    N = sum(projs[p][2] for p in grp)
                    X = next(c[4] for c in calls[M] if c[0] == l and c[1] == grp[0])
                    Y = torch.empty((M, N), dtype=torch.float32, device=dev)
                    lst.append((fpk[(l, gi)], X, Y))
                    fb += call_bytes(M, K, N)

            def run_fused(lst=lst):
                for (pk, X, Y) in lst:
                    q.int8_gemm_dynamic(X, pk, out_f32=Y)
            run_fused()
            torch.cuda.synchronize()
            # bit-identical to separate calls on the same activations
            for l in range(layers):
                for gi, grp in enumerate(groups):
                    _, X, Yf = lst[l * len(groups) + gi]
                    c0 = 0
                    for p in grp:
                        n = projs[p][2]
                        Ys = torch.empty((M, n), dtype=torch.float32, device=dev)
                        q.int8_gemm_dynamic(X, packed[(l, p)], out_f32=Ys)
                        if not torch.equal(Yf[:, c0:c0 + n].contiguous().view(torch.int32), Ys.view(torch.int32)):
                            raise RuntimeError("fused projection differs from the separate call (M=%d)" % M)
                        c0 += n
            gf = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gf):
                run_fused()
            gf.replay()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(args.steps):
                gf.replay()
            b.record()
            torch.cuda.synchronize()
            sec = a.elapsed_time(b) * 1e-3 / args.steps
            fused[str(M)] = {"step_ms": round(sec * 1e3, 4), "GB/s": round(fb / sec / 1e9, 2),
                             "%HBM": round(100 * fb / sec / 1e9 / HBM_PEAK_GBS, 2),
                             "calls": len(lst), "call_us": round(sec / len(lst) * 1e6, 3)}
        extra["fused_qkv_gate_up"] = fused
        del fpk

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

        # context, not this library: the vendor BLAS int8 product (torch._int_mm,
        # int32 out, no epilogue) on the same shapes
        blas = {}
        for i, (K, N) in enumerate(wl.PREFILL_SHAPES):
            try:
                g_ = wl.rng(4, 50 + i)
                A = torch.from_numpy(wl.uniform_i8(g_, (wl.PREFILL_M, K))).to(dev)
                B = torch.from_numpy(wl.uniform_i8(g_, (N, K))).to(dev).t()     # column-major K x N
                f = (lambda A=A, B=B: torch._int_mm(A, B))
                f()
                t = float(np.median(time_launches(torch, [f] * 10)))
                tops = 2.0 * wl.PREFILL_M * K * N / t / 1e12
                blas["%dx%d" % (K, N)] = {"us": round(t * 1e6, 2), "TOPS": round(tops, 1),
                                          "%MFMA": round(100 * tops / INT8_PEAK_TOPS, 2)}
                del A, B
            except Exception as exc:  # the vendor routine may not take this layout
                blas["%dx%d" % (K, N)] = {"error": str(exc)[:120]}
        extra["vendor_int8_mm_m2048"] = blas

        # ------------------------------- q4_1 product, M = 1 and 16 ---
        q4, q4q8 = {}, {}
        for i, (K, N) in enumerate(wl.Q4_SHAPES):
            _, blocks = wl.q4_weight(K, N, seed_index=i)
            bd = torch.from_numpy(blocks.reshape(-1)).to(dev)
            ring = [q.q4_1_repack(bd, K, N) for _ in range(16)]   # 16 copies: ~590 MB, past the MALL
            torch.cuda.synchronize()
            wbytes = ring[0].data.numel() - 64
            for M in wl.Q4_ROWS:
                X = torch.from_numpy(wl.q4_activations(M, K, seed_index=i)).to(dev)
                Y = torch.empty((M, N), dtype=torch.float32, device=dev)
                wsq = q.workspace(q.lib.qmm_q4_1_matmul_workspace_bytes(M, K, N), dev)
                fs = [(lambda W=W, X=X, Y=Y, wsq=wsq: q.q4_1_matmul(X, W, out=Y, ws=wsq)) for W in ring]
                fs[0]()
                ts = np.array(time_launches(torch, fs * 3))
                t = float(np.median(ts))
                b = wbytes + 4 * M * K + 4 * M * N
                q4["%dx%d_m%d" % (K, N, M)] = {"us": round(t * 1e6, 2), "GB/s": round(b / t / 1e9, 1),
                                               "%HBM": round(100 * b / t / 1e9 / HBM_PEAK_GBS, 2)}
                # the same weights against per-row int8 activations
                Xq, sa = q.quantize_rows_int8(X)
                fs = [(lambda W=W, Xq=Xq, sa=sa, Y=Y: q.q4_1_matmul_q8(Xq, sa, W, out=Y)) for W in ring]
                fs[0]()
                t = float(np.median(np.array(time_launches(torch, fs * 3))))
                b = wbytes + M * K + 4 * M + 4 * M * N
                q4q8["%dx%d_m%d" % (K, N, M)] = {"us": round(t * 1e6, 2), "GB/s": round(b / t / 1e9, 1),
                                                 "%HBM": round(100 * b / t / 1e9 / HBM_PEAK_GBS, 2)}
            del ring, bd
        extra["q4_1_matmul"] = q4
        extra["q4_1_matmul_q8"] = q4q8

        # --------------------------------------------- MUL_MAT_ID ---
        d = wl.moe_inputs()
        E, K, N = wl.MOE_EXPERTS, wl.MOE_K, wl.MOE_N
        ed = torch.from_numpy(d["experts"]).to(dev)
        rings = [q.q4_1_repack_experts(ed, K, N) for _ in range(4)]   # 4 copies: ~500 MB
        X = torch.from_numpy(d["X"]).to(dev)
        ids = torch.from_numpy(d["ids"]).to(dev)
        Y = torch.empty((wl.MOE_TOKENS, wl.MOE_USED, N), dtype=torch.float32, device=dev)
        wsm = q.workspace(q.lib.qmm_q4_1_matmul_id_workspace_bytes(wl.MOE_TOKENS, wl.MOE_USED, E, K, N), dev)
        fs = [(lambda buf=buf, st=st: q.q4_1_matmul_id(X, buf, E, K, N, st, ids, wl.MOE_USED, out=Y, ws=wsm))
              for buf, st in rings]
        fs[0]()
        t = float(np.median(time_launches(torch, fs * 5)))
        wb = E * (K * N // 2 + (K // 32) * N * 4)     # codes + bf16 (d, m) per block
        b = wb + X.numel() * 4 + wl.MOE_TOKENS * wl.MOE_IDS_STRIDE * 4 + Y.numel() * 4
        extra["q4_1_matmul_id"] = {"us": round(t * 1e6, 2), "GB/s": round(b / t / 1e9, 1),
                                   "%HBM": round(100 * b / t / 1e9 / HBM_PEAK_GBS, 2),
                                   "experts": E, "tokens": wl.MOE_TOKENS, "top_k": wl.MOE_USED}
        del rings, ed

        # MUL_MAT_ID of the down experts: a row per (token, slot)
        d = wl.moe_down_inputs()
        K, N = wl.MOE_DOWN_K, wl.MOE_DOWN_N
        ed = torch.from_numpy(d["experts"]).to(dev)
        rings = [q.q4_1_repack_experts(ed, K, N) for _ in range(4)]   # 4 copies: ~500 MB
        X = torch.from_numpy(d["X"]).to(dev)
        ids = torch.from_numpy(d["ids"]).to(dev)
        Y = torch.empty((wl.MOE_TOKENS, wl.MOE_USED, N), dtype=torch.float32, device=dev)
        wsm = q.workspace(q.lib.qmm_q4_1_matmul_id_per_slot_workspace_bytes(wl.MOE_TOKENS, wl.MOE_USED, E, K, N),
                          dev)
        fs = [(lambda buf=buf, st=st: q.q4_1_matmul_id_per_slot(X, buf, E, K, N, st, ids, wl.MOE_USED, out=Y,
                                                               ws=wsm))
              for buf, st in rings]
        fs[0]()
        t = float(np.median(time_launches(torch, fs * 5)))
        wb = E * (K * N // 2 + (K // 32) * N * 4)     # codes + bf16 (d, m) per block
        b = wb + X.numel() * 4 + wl.MOE_TOKENS * wl.MOE_IDS_STRIDE * 4 + Y.numel() * 4
        extra["q4_1_matmul_id_per_slot"] = {"us": round(t * 1e6, 2), "GB/s": round(b / t / 1e9, 1),
                                            "%HBM": round(100 * b / t / 1e9 / HBM_PEAK_GBS, 2),
                                            "experts": E, "K": K, "N": N, "tokens": wl.MOE_TOKENS,
                                            "top_k": wl.MOE_USED}
        del rings, ed

        # ------------ lm_head-shaped projection: K = 1024, N = 151936 ---
        K, N = wl.LM_HEAD_K, wl.LM_HEAD_N
        Wh = wl.lm_head_weight()
        Wl = torch.from_numpy(Wh).to(dev)
        ring = [q.pack_b_int8(Wl) for _ in range(4)]          # 4 copies: ~623 MB, past the MALL
        del Wl
        lm = {}
        for M in wl.LM_HEAD_ROWS:
            X = torch.from_numpy(wl.lm_head_activations(M, seed_index=M)).to(dev)
            Y = torch.empty((M, N), dtype=torch.float32, device=dev)
            fs = [(lambda pk=pk, X=X, Y=Y: q.int8_gemm_dynamic(X, pk, out_f32=Y)) for pk in ring]
            fs[0]()
            t = float(np.median(time_launches(torch, fs * 3)))
            b = call_bytes(M, K, N)
            lm["int8_m%d" % M] = {"us": round(t * 1e6, 2), "GB/s": round(b / t / 1e9, 1),
                                  "%HBM": round(100 * b / t / 1e9 / HBM_PEAK_GBS, 2)}
        del ring
        bd = torch.from_numpy(wl.encode_q4_1(Wh).reshape(-1)).to(dev)
        del Wh
        ring = [q.q4_1_repack(bd, K, N) for _ in range(6)]    # 6 copies: ~583 MB
        del bd
        wbytes = ring[0].data.numel() - 64
        for M in wl.LM_HEAD_ROWS:
            X = torch.from_numpy(wl.lm_head_activations(M, seed_index=100 + M)).to(dev)
            Y = torch.empty((M, N), dtype=torch.float32, device=dev)
            wsq = q.workspace(q.lib.qmm_q4_1_matmul_workspace_bytes(M, K, N), dev)
            fs = [(lambda W=W, X=X, Y=Y, wsq=wsq: q.q4_1_matmul(X, W, out=Y, ws=wsq)) for W in ring]
            fs[0]()
            t = float(np.median(time_launches(torch, fs * 3)))
            b = wbytes + 4 * M * K + 4 * M * N
            lm["q4_1_m%d" % M] = {"us": round(t * 1e6, 2), "GB/s": round(b / t / 1e9, 1),
                                  "%HBM": round(100 * b / t / 1e9 / HBM_PEAK_GBS, 2)}
        del ring
        extra["lm_head_1024x151936"] = lm

        # ------------- streaming-read floor: the same sizes, read cold ---
        floor = {}
        for nbytes in (2301952, 36700160, 155582464):
            nb = (nbytes + 15) // 16 * 16
            copies = max(4, -(-640 * 2 ** 20 // nb))                 # > 2 x (MALL + L2) in all
            bufs = [torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1) for _ in range(copies)]
            for wg in (1024, 4096, -(-nb // 4096)):                   # the last: one load per thread
                sink = torch.empty(wg, dtype=torch.int32, device=dev)
                fs = [(lambda b_=b_, sink=sink, wg=wg: q.read_probe(b_, sink, wg)) for b_ in bufs]
                fs[0]()
                # per launch through the (event, launch, event) timer, and back to
                # back (one graph of all copies, as the decode calls are timed)
                t = float(np.median(time_launches(torch, fs * max(1, 48 // copies))))
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr):
                    for f in fs:
                        f()
                gr.replay()
                torch.cuda.synchronize()
                a_ = torch.cuda.Event(enable_timing=True)
                b2 = torch.cuda.Event(enable_timing=True)
                a_.record()
                for _ in range(3):
                    gr.replay()
                b2.record()
                torch.cuda.synchronize()
                tb = a_.elapsed_time(b2) * 1e-3 / (3 * len(fs))
                floor["%d_B_wg%d" % (nbytes, wg)] = {"us": round(t * 1e6, 2), "GB/s": round(nbytes / t / 1e9, 1),
                                                     "back_to_back_us": round(tb * 1e6, 2),
                                                     "back_to_back_GB/s": round(nbytes / tb / 1e9, 1)}
                del gr
            del bufs
        extra["read_floor"] = floor

        # -------------------------------- one-time packing (a1, a5) ---
        K, N = 4096, 14336
        W = torch.from_numpy(wl.normal_f32(wl.rng(4, 77), (K, N), 0.02)).to(dev)
        f = lambda: q.pack_b_int8(W)  # noqa: E731
        f()
        t = float(np.median(time_launches(torch, [f] * 5)))
        extra["pack_b_int8_4096x14336"] = {"us": round(t * 1e6, 1), "GB/s": round((4 * K * N + K * N) / t / 1e9, 1)}
        _, blocks = wl.q4_weight(K, N, seed_index=0)
        bd = torch.from_numpy(blocks.reshape(-1)).to(dev)
        f = lambda: q.q4_1_repack(bd, K, N)  # noqa: E731
        f()
        t = float(np.median(time_launches(torch, [f] * 5)))
        extra["q4_1_repack_4096x14336"] = {"us": round(t * 1e6, 1), "GB/s": round(2 * blocks.nbytes / t / 1e9, 1)}
        del W, bd

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
