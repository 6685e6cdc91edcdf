#!/usr/bin/env python3
"""Benchmark of the quantized projection matmul on one MI355X.

Workload (one "step"): the seven Qwen3-0.6B projections of all 28 layers
(196 distinct weights, fp32 N(0, 0.02), packed once by pack_b_int8 before the
timed region: ~420 MiB of int8 codes, more than the 256 MiB Infinity Cache)
run as decode at M = 1, 16 and 32 rows of fp32 N(0, 1) activations, in a
decoder layer's call structure: q, k and v read one activation matrix and run
as one int8_gemm_dynamic_grouped launch, o is a call of its own, gate and up
share one grouped launch, down is a call of its own (4 launches per layer).
Every call quantises its activations per row (amax/127) inside the int8
product kernel and writes fp32 (row scale x column scale).  Each M's 112
launches are captured in one HIP graph; a step replays the three graphs.

`value` is the step's algorithmic bytes (per launch: every item's K*N weight
bytes + 4N column scales + 4MN outputs, plus the 4MK activations read once)
over its wall time, in GB/s.  `roofline` is the dominant kernel, the fused
quantise-and-multiply decode (k_int8_decode_q, its grouped and single-weight
forms: every launch of the step): its algorithmic bytes over the summed time
of the timed replays (HIP events on the replay stream, so the dispatch gap
between back-to-back launches is included).  `extra` carries the per-M
figures, the same projections as seven separate calls per layer, the other
configurations (the zero-point product, int8 prefill at M = 2048 with its own
roofline record, q4_1, MUL_MAT_ID, lm_head), the streaming-read floor and the
oracle's CPU timings.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline] [--no-extra]
    python bench.py --profile            # the timed leg alone (for rocprofv3)
    python bench.py --probe              # 1 GiB probe read, then one eager step (for --pmc runs)
    python bench.py --summarize DB [--kernel PATTERN] [--last N]   # a rocprofv3 database, as text
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
DECODE_KERNEL = "k_int8_decode_q"
PROBE_BYTES = 1 << 30

# HBM traffic of the dominant kernel per launch, from two rocprofv3 --pmc runs
# of `bench.py --probe` (FETCH_SIZE, then WRITE_SIZE; mean over the step's 336
# decode launches): FETCH_SIZE x 2.0, the factor the probe's plain read of
# 1 GiB gives in the same run (524306 KiB), plus WRITE_SIZE x 1.0, the factor
# the 1 GiB fill of the probe buffer gives (1048576 KiB).  Valid only for the
# kernel sources it was taken on.
MEASURED_TRAFFIC = {"sources_sha1": "d295d6161d471587ad0b7c0f6809491c2db0c3d9",
                    "bytes_per_launch": round((2463.5 * 2.0 + 196.0) * 1024)}


def decode_sources_sha1():
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha1()
    for f in ("k_int8.hip", "int8_common.h", "qmm_internal.h", "api.cpp"):
        with open(os.path.join(here, "int8_bit_weight_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def decode_traffic():
    ok = MEASURED_TRAFFIC["sources_sha1"] == decode_sources_sha1()
    return MEASURED_TRAFFIC["bytes_per_launch"] if ok else None


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
                    help="counter probe: one plain read of 1 GiB (the calibration read), then one eager step")
    ap.add_argument("--profile", action="store_true",
                    help="the timed leg alone (setup, graph capture, warm-up and timed replays)")
    ap.add_argument("--profile-leg", choices=("decode", "prefill", "q4", "lmhead"), default="decode",
                    help="--profile: the decode step (default), the M = 2048 prefill shapes (each warmed up "
                         "and then launched --steps times in a row), the q4_1 calls (M = 1 and 16 on both "
                         "shapes, then MUL_MAT_ID in both forms) over rings of weight copies, or the "
                         "lm_head-shaped calls (int8 and q4_1, M = 1 and 16) over rings of weight copies")
    ap.add_argument("--summarize", metavar="DB", help="summarize a rocprofv3 database (no GPU needed)")
    ap.add_argument("--kernel", default="", help="--summarize: kernel name substring")
    ap.add_argument("--last", type=int, default=0, help="--summarize: only the last N matching dispatches")
    ap.add_argument("--skip", type=int, default=0, help="--summarize: leave out the first N matching dispatches")
    ap.add_argument("--count", type=int, default=0, help="--summarize: then keep only the next N")
    ap.add_argument("--cycle", default="",
                    help="--summarize: LABEL:N,LABEL:N,... the selected dispatches come in repeating runs of "
                         "these lengths (e.g. 1:112,16:112,32:112 for the decode step's rows); one table per label")
    return ap.parse_args()


# --------------------------------------------------------------- layout ---

# A decoder layer's projection launches: items that share one activation
# matrix (q, k, v; gate, up) run as one grouped launch.
LAYER_LAUNCHES = ((0, 1, 2), (3,), (4, 5), (6,))


def launch_bytes(M, K, Ns):
    """Algorithmic bytes of one launch over weights of widths Ns that share
    the activations: weights, column scales and outputs of every item, the
    fp32 activations once."""
    return sum(K * N + 4 * N + 4 * M * N for N in Ns) + 4 * M * K


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


def time_graph(torch, fn, reps):
    """Seconds per replay of a graph of fn's launches, replayed back to back
    (HIP events on the replay stream: dispatch gaps included)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / reps


def time_ring(torch, fs, reps=3):
    """Seconds per launch of a list of launches (a ring over cold weight
    copies) captured in one graph and replayed back to back, like the
    decode step (dispatch gaps included)."""
    def run():
        for f in fs:
            f()
    return time_graph(torch, run, reps) / len(fs)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------ summarize ---

def summarize(path, pattern, last, skip=0, count=0, cycle=""):
    """Per-kernel duration statistics (and per-dispatch counter means) from a
    rocprofv3 SQLite database, restricted to kernels whose name contains
    `pattern`, past the first `skip` of them, and to the last `last` of those
    when given.  `cycle` ("LABEL:N,..."): the selection repeats runs of those
    lengths; a table per label as well."""
    import sqlite3
    import numpy as np
    db = sqlite3.connect(path)
    rows = list(db.execute("select dispatch_id, name, start, duration from kernels order by start"))
    sel = [r for r in rows if pattern in r[1]][skip:]
    if count:
        sel = sel[:count]
    if last:
        sel = sel[-last:]
    print("database: %s" % os.path.basename(path))
    print("dispatches: %d in all, %d selected (kernel name contains %r%s%s%s)"
          % (len(rows), len(sel), pattern, ", first %d left out" % skip if skip else "",
             ", the next %d" % count if count else "", ", last %d" % last if last else ""))
    def table(rows_):
        by = {}
        for did, name, _, dur in rows_:
            by.setdefault(name, []).append(dur)
        print("| kernel | launches | mean us | median us | p10 us | p90 us | min us | max us | total ms |")
        print("|---|---|---|---|---|---|---|---|---|")
        for name, d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
            a = np.array(d, dtype=np.float64) * 1e-3
            short = name.split("(")[0] if not name.startswith("void ") else name[5:].split("(Int8")[0].split("(qmm")[0]
            print("| %s | %d | %.3f | %.3f | %.3f | %.3f | %.3f | %.3f | %.3f |"
                  % (short[-70:], a.size, a.mean(), np.median(a), np.percentile(a, 10), np.percentile(a, 90),
                     a.min(), a.max(), a.sum() * 1e-3))
        if rows_:
            a = np.array([r[3] for r in rows_], dtype=np.float64) * 1e-3
            print("| (all selected) | %d | %.3f | %.3f | %.3f | %.3f | %.3f | %.3f | %.3f |"
                  % (a.size, a.mean(), np.median(a), np.percentile(a, 10), np.percentile(a, 90), a.min(), a.max(),
                     a.sum() * 1e-3))
    table(sel)
    if cycle:
        runs = [(lab, int(n)) for lab, n in (c.split(":") for c in cycle.split(","))]
        period = sum(n for _, n in runs)
        groups = {lab: [] for lab, _ in runs}
        for i, r in enumerate(sel):
            pos = i % period
            for lab, n in runs:
                if pos < n:
                    groups[lab].append(r)
                    break
                pos -= n
        for lab, _ in runs:
            print("\n%s (%d dispatches):" % (lab, len(groups[lab])))
            table(groups[lab])
    ids = {r[0] for r in sel}
    try:
        crows = list(db.execute("select dispatch_id, counter_name, sum(value) from counters_collection "
                                "group by dispatch_id, counter_name"))
    except sqlite3.OperationalError:
        crows = []
    if crows:
        cnt = {}
        for did, cn, v in crows:
            if did in ids:
                cnt.setdefault(cn, []).append(v)
        if cnt:
            print("\ncounters, mean per selected dispatch (summed over XCDs / shader engines):")
            for cn, v in sorted(cnt.items()):
                print("  %s = %.1f (%d dispatches)" % (cn, float(np.mean(v)), len(v)))
    return 0


# ----------------------------------------------------------------- main ---

def main() -> int:
    args = parse_args()
    if args.summarize:
        return summarize(args.summarize, args.kernel, args.last, args.skip, args.count, args.cycle)
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
    if args.profile and args.profile_leg == "prefill":
        return profile_prefill(args, q, wl, torch, np, dev)
    if args.profile and args.profile_leg == "q4":
        return profile_q4(args, q, wl, torch, np, dev)
    if args.profile and args.profile_leg == "lmhead":
        return profile_lm_head(args, q, wl, torch, np, dev)
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

    # per M: the step's launches, (layer, items, K, X, outputs)
    calls = {}
    for M in rows:
        lst = []
        for l in range(layers):
            for gi, grp in enumerate(LAYER_LAUNCHES):
                K = projs[grp[0]][1]
                X = torch.from_numpy(wl.projection_activations(M, K, seed_index=10000 + l * 16 + gi)).to(dev)
                Ys = [torch.empty((M, projs[p][2]), dtype=torch.float32, device=dev) for p in grp]
                lst.append((l, grp, K, X, Ys))
        calls[M] = lst
    for M in rows:
        for (_, grp, K, _, _) in calls[M]:
            assert fused_quant(M, K), "every launch of the step is the fused decode kernel"

    def run_m(M):
        for (l, grp, K, X, Ys) in calls[M]:
            if len(grp) == 1:
                q.int8_gemm_dynamic(X, packed[(l, grp[0])], out_f32=Ys[0])
            else:
                q.int8_gemm_dynamic_grouped(X, [packed[(l, p)] for p in grp], outs=Ys)

    step_bytes = {M: sum(launch_bytes(M, c[2], [projs[p][2] for p in c[1]]) for c in calls[M]) for M in rows}
    total_bytes = sum(step_bytes.values())
    n_launch = sum(len(calls[M]) for M in rows)

    if args.probe:
        from int8_bit_weight_amd.probe import read_probe
        buf = torch.empty(PROBE_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        sink = torch.empty(4096, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        read_probe(buf, sink, 4096, 4)
        torch.cuda.synchronize()
        for M in rows:
            run_m(M)
        torch.cuda.synchronize()
        print(json.dumps({"probe": "plain read of %d bytes, then %d decode launches" % (PROBE_BYTES, n_launch),
                          "decode_algorithmic_bytes": total_bytes, "decode_launches": n_launch,
                          "decode_sources_sha1": decode_sources_sha1()}))
        return 0

    graphs = {}
    if not args.profile:
        # eager reference outputs, then one graph per M, checked bit for bit
        for M in rows:
            run_m(M)
        torch.cuda.synchronize()
        eager = {M: [[y.clone() for y in c[4]] for c in calls[M]] for M in rows}
    for M in rows:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_m(M)
        graphs[M] = g
    if not args.profile:
        for rep in range(2):
            for M in rows:
                for c in calls[M]:
                    for y in c[4]:
                        y.fill_(float("nan"))
                graphs[M].replay()
            torch.cuda.synchronize()
            for M in rows:
                for c, ref in zip(calls[M], eager[M]):
                    for y, r in zip(c[4], ref):
                        if not torch.equal(y.view(torch.int32), r.view(torch.int32)):
                            raise RuntimeError("graph replay differs from eager result (M=%d)" % M)
        del eager

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
        per_m[M] = dict(sec=sec, gbs=step_bytes[M] / sec / 1e9, launches=len(calls[M]))
    log("step %.3f ms, %.1f GB/s" % (ms_per_step, value))

    # Dominant kernel: every launch of the step is the fused decode kernel,
    # so its time is the timed replays' event time and its bytes the step's.
    kern_t = sum(per_m[M]["sec"] for M in rows)
    achieved = total_bytes / kern_t / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": decode_traffic(),
                "kernel": "fused quantise + int8 decode GEMM (%s, grouped and single-weight forms)" % DECODE_KERNEL,
                "algorithmic_bytes_per_launch": round(total_bytes / n_launch),
                "avg_launch_us": round(kern_t / n_launch * 1e6, 3), "launches_per_step": n_launch,
                "timing": "HIP events around back-to-back graph replays (dispatch gaps included)"}
    extra = {"per_m": {str(M): {"step_ms": round(per_m[M]["sec"] * 1e3, 4), "GB/s": round(per_m[M]["gbs"], 2),
                                "%HBM": round(100 * per_m[M]["gbs"] / HBM_PEAK_GBS, 2),
                                "launches": per_m[M]["launches"],
                                "launch_us": round(per_m[M]["sec"] / per_m[M]["launches"] * 1e6, 3)}
                       for M in rows}}

    if args.profile:
        print(json.dumps({"metric": METRIC, "value": round(value, 2), "unit": "GB/s", "profile": True,
                          "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
                          "timed_launches": args.steps * n_launch, "roofline": roofline, "extra": extra}),
              flush=True)
        return 0

    if not args.no_extra:
        extra.update(extras(args, q, wl, torch, np, dev, packed, projs, layers, rows))

    # ------------------------------------------------------- CPU baseline ---
    cpu = None
    if not args.no_cpu_baseline:
        cpu, timings = cpu_oracle(wl, np, host_w, calls, projs, rows, layers, total_bytes)
        extra["cpu_oracle"] = timings

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "qwen3-0.6b-projections-int8-decode", "layers": layers,
                   "projections": [p[0] for p in projs], "rows": list(rows),
                   "launches_per_layer": "q+k+v grouped, o, gate+up grouped, down",
                   "launches_per_step": n_launch, "bytes_per_step": total_bytes, "parallelism": "single-gpu"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)
    return 0


def profile_prefill(args, q, wl, torch, np, dev):
    """The M = 2048 prefill shapes alone, in order: per shape 2 eager
    launches, one untimed and one timed replay of a graph of --steps
    launches (for rocprofv3: shape i's timed dispatches are the
    (2 + 2 steps) i + 2 + steps .. + steps ones, --skip / --count)."""
    res = {}
    for i, (K, N) in enumerate(wl.PREFILL_SHAPES):
        dp = wl.prefill_inputs(K, N, seed_index=i)
        pk = q.pack_b_int8(torch.from_numpy(dp["W"]).to(dev))
        A = torch.from_numpy(dp["A"]).to(dev)
        rs = torch.from_numpy(dp["rs"]).to(dev)
        Y = torch.empty((wl.PREFILL_M, N), dtype=torch.float32, device=dev)

        def f(A=A, pk=pk, Y=Y, rs=rs):
            q.int8_gemm(A, 0, pk, 0, out_f32=Y, row_scale=rs)
        f()
        f()
        torch.cuda.synchronize()

        def run(f=f):
            for _ in range(args.steps):
                f()
        t = time_graph(torch, run, 1) / args.steps
        tops = 2.0 * wl.PREFILL_M * K * N / t / 1e12
        res["%dx%d" % (K, N)] = {"us": round(t * 1e6, 2), "TOPS": round(tops, 1),
                                 "%MFMA": round(100 * tops / INT8_PEAK_TOPS, 2)}
        del pk, A, Y
    print(json.dumps({"profile": "prefill", "steps": args.steps, "shapes": res,
                      "dispatches_per_shape": 2 + 2 * args.steps}), flush=True)
    return 0


def q4_moe_bytes(wl, E, K, N, X, Y):
    """Algorithmic bytes of one MUL_MAT_ID call: every expert's codes and
    bf16 (d, m) per block, the activations, the id rows and the outputs."""
    wb = E * (K * N // 2 + (K // 32) * N * 4)
    return wb + X.numel() * 4 + wl.MOE_TOKENS * wl.MOE_IDS_STRIDE * 4 + Y.numel() * 4


def profile_q4(args, q, wl, torch, np, dev):
    """The q4_1 calls alone, eager, in order (for rocprofv3 counters and
    traces): per shape of the q4_1 product and per M in (1, 16), one call on
    each of 16 weight copies (~590 MB, past the 256 MB Infinity Cache); then
    MUL_MAT_ID in the shared and the per-slot form, 2 x 4 calls over 4
    copies of the experts."""
    res = {}
    for i, (K, N) in enumerate(wl.Q4_SHAPES):
        _, blocks = wl.q4_weight(K, N, seed_index=i)
        bd = torch.from_numpy(blocks.reshape(-1)).to(dev)
        ring = [q.q4_1_repack(bd, K, N) for _ in range(16)]
        wbytes = ring[0].data.numel() - 64
        for M in wl.Q4_ROWS:
            X = torch.from_numpy(wl.q4_activations(M, K, seed_index=i)).to(dev)
            Y = torch.empty((M, N), dtype=torch.float32, device=dev)
            wsq = q.workspace(q.lib.qmm_q4_1_matmul_workspace_bytes(M, K, N), dev)
            torch.cuda.synchronize()
            for W in ring:
                q.q4_1_matmul(X, W, out=Y, ws=wsq)
            torch.cuda.synchronize()
            res["q4_1_%dx%d_m%d" % (K, N, M)] = {"calls": len(ring), "variant": q.last_variant(),
                                                 "algorithmic_bytes_per_call": wbytes + 4 * M * K + 4 * M * N}
        del ring, bd
    for name, inputs, per_slot in (("q4_1_matmul_id", wl.moe_inputs, False),
                                   ("q4_1_matmul_id_per_slot", wl.moe_down_inputs, True)):
        dm = inputs()
        E = wl.MOE_EXPERTS
        K, N = (wl.MOE_DOWN_K, wl.MOE_DOWN_N) if per_slot else (wl.MOE_K, wl.MOE_N)
        ed = torch.from_numpy(dm["experts"]).to(dev)
        rings = [q.q4_1_repack_experts(ed, K, N) for _ in range(4)]
        X = torch.from_numpy(dm["X"]).to(dev)
        ids = torch.from_numpy(dm["ids"]).to(dev)
        Y = torch.empty((wl.MOE_TOKENS, wl.MOE_USED, N), dtype=torch.float32, device=dev)
        fn = q.q4_1_matmul_id_per_slot if per_slot else q.q4_1_matmul_id
        torch.cuda.synchronize()
        for _ in range(2):
            for buf, st in rings:
                fn(X, buf, E, K, N, st, ids, wl.MOE_USED, out=Y)
        torch.cuda.synchronize()
        res[name] = {"calls": 2 * len(rings), "algorithmic_bytes_per_call": q4_moe_bytes(wl, E, K, N, X, Y)}
        del rings, ed
    print(json.dumps({"profile": "q4", "calls": res}), flush=True)
    return 0


def profile_lm_head(args, q, wl, torch, np, dev):
    """The lm_head-shaped calls alone, eager, in order (for rocprofv3): the
    int8 path (int8_gemm_dynamic, fp32 out) at M = 1 and 16, one call on each
    of 4 packed copies twice over (~623 MB), then the q4_1 path at M = 1 and
    16, one call on each of 6 copies (~583 MB)."""
    K, N = wl.LM_HEAD_K, wl.LM_HEAD_N
    Wh = wl.lm_head_weight()
    Wl = torch.from_numpy(Wh).to(dev)
    ring = [q.pack_b_int8(Wl) for _ in range(4)]
    del Wl
    res = {}
    for M in wl.LM_HEAD_ROWS:
        X = torch.from_numpy(wl.lm_head_activations(M, seed_index=M)).to(dev)
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        for pk in ring * 2:
            q.int8_gemm_dynamic(X, pk, out_f32=Y)
        torch.cuda.synchronize()
        res["int8_m%d" % M] = {"calls": 2 * len(ring), "variant": q.last_variant(),
                               "algorithmic_bytes_per_call": launch_bytes(M, K, [N])}
    del ring
    bd = torch.from_numpy(wl.encode_q4_1(Wh).reshape(-1)).to(dev)
    del Wh
    ring = [q.q4_1_repack(bd, K, N) for _ in range(6)]
    del bd
    wbytes = ring[0].data.numel() - 64
    for M in wl.LM_HEAD_ROWS:
        X = torch.from_numpy(wl.lm_head_activations(M, seed_index=100 + M)).to(dev)
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        wsq = q.workspace(q.lib.qmm_q4_1_matmul_workspace_bytes(M, K, N), dev)
        torch.cuda.synchronize()
        for W in ring:
            q.q4_1_matmul(X, W, out=Y, ws=wsq)
        torch.cuda.synchronize()
        res["q4_1_m%d" % M] = {"calls": len(ring), "variant": q.last_variant(),
                               "algorithmic_bytes_per_call": wbytes + 4 * M * K + 4 * M * N}
    del ring
    print(json.dumps({"profile": "lmhead", "calls": res}), flush=True)
    return 0


# ---------------------------------------------------------------- extras ---

def extras(args, q, wl, torch, np, dev, packed, projs, layers, rows):
    extra = {}

    # --------- the same projections as seven separate calls per layer ---
    sep = {}
    for M in rows:
        lst, sb = [], 0
        for l in range(layers):
            for p, (_, K, N) in enumerate(projs):
                X = torch.from_numpy(wl.projection_activations(M, K, seed_index=20000 + l * 16 + p)).to(dev)
                Y = torch.empty((M, N), dtype=torch.float32, device=dev)
                lst.append((packed[(l, p)], X, Y))
                sb += launch_bytes(M, K, [N])

        def run_sep(lst=lst):
            for (pk, X, Y) in lst:
                q.int8_gemm_dynamic(X, pk, out_f32=Y)
        run_sep()
        sec = time_graph(torch, run_sep, args.steps)
        sep[str(M)] = {"step_ms": round(sec * 1e3, 4), "GB/s": round(sb / sec / 1e9, 2),
                       "%HBM": round(100 * sb / sec / 1e9 / HBM_PEAK_GBS, 2), "calls": len(lst),
                       "call_us": round(sec / len(lst) * 1e6, 3)}
    extra["separate_calls"] = sep

    # ------ the zero-point product: uint8 A with zA, int8 B with zB, I32+F32 ---
    d = wl.int8_product_inputs(M=16, K=1024, N=1024)
    Bd = torch.from_numpy(d["B"]).to(dev)
    ring = [q.pack_b_int8_raw(Bd) for _ in range(640)]   # 1 MiB each: 640 MiB, past the MALL
    A = torch.from_numpy(d["A"]).to(dev)
    bias = torch.from_numpy(d["bias"]).to(dev)
    y32 = torch.empty((16, 1024), dtype=torch.int32, device=dev)
    yf = torch.empty((16, 1024), dtype=torch.float32, device=dev)

    def run_zp():
        for pk in ring:
            q.int8_gemm(A, d["zA"], pk, d["zB"], out_i32=y32, out_f32=yf, scale=float(d["scale"]), bias_f32=bias)
    run_zp()
    sec = time_graph(torch, run_zp, 3) / len(ring)
    zb = 1024 * 1024 + 16 * 1024 + 4 * 1024 + 4 * 1024 + 2 * 16 * 1024 * 4
    extra["zero_point_product_16x1024x1024"] = {
        "us": round(sec * 1e6, 3), "GB/s": round(zb / sec / 1e9, 1), "%HBM": round(100 * zb / sec / 1e9 / HBM_PEAK_GBS, 2),
        "algorithmic_bytes": zb, "outputs": "int32 + fp32 (bias)", "variant": q.last_variant(),
        "timing": "one graph of calls over 640 packed copies, back to back"}
    del ring, Bd

    # --------------------------------------------- int8 prefill, M = 2048 ---
    pre = {}
    ops_all, t_all = 0.0, 0.0
    for i, (K, N) in enumerate(wl.PREFILL_SHAPES):
        dp = wl.prefill_inputs(K, N, seed_index=i)
        pk = q.pack_b_int8(torch.from_numpy(dp["W"]).to(dev))
        A = torch.from_numpy(dp["A"]).to(dev)
        rs = torch.from_numpy(dp["rs"]).to(dev)
        Y = torch.empty((wl.PREFILL_M, N), dtype=torch.float32, device=dev)
        f = (lambda A=A, pk=pk, Y=Y, rs=rs: q.int8_gemm(A, 0, pk, 0, out_f32=Y, row_scale=rs))
        f()
        ts = np.array(time_launches(torch, [f] * 12))
        t = time_ring(torch, [f] * 6)
        ops = 2.0 * wl.PREFILL_M * K * N
        ops_all += ops
        t_all += t
        tops = ops / t / 1e12
        pre["%dx%d" % (K, N)] = {"us": round(t * 1e6, 2), "per_launch_median_us": round(float(np.median(ts)) * 1e6, 2),
                                 "per_launch_p10_us": round(float(np.percentile(ts, 10)) * 1e6, 2),
                                 "per_launch_p90_us": round(float(np.percentile(ts, 90)) * 1e6, 2), "TOPS": round(tops, 1),
                                 "%MFMA": round(100 * tops / INT8_PEAK_TOPS, 2), "variant": q.last_variant()}
        del pk, A, Y
    extra["int8_prefill_m2048"] = pre
    ach = ops_all / t_all / 1e12
    extra["roofline_prefill"] = {"bound": "mfma", "achieved": round(ach, 1), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                                 "frac": round(ach / INT8_PEAK_TOPS, 4),
                                 "kernel": "k_int8_prefill (the three M = 2048 shapes: their ops over their summed "
                                           "back-to-back launch times)"}

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
            t = time_ring(torch, fs)
            b = wbytes + 4 * M * K + 4 * M * N
            q4["%dx%d_m%d" % (K, N, M)] = {"us": round(t * 1e6, 2), "GB/s": round(b / t / 1e9, 1),
                                           "%HBM": round(100 * b / t / 1e9 / HBM_PEAK_GBS, 2),
                                           "variant": q.last_variant()}
            # the same weights against per-row int8 activations
            Xq, sa = q.quantize_rows_int8(X)
            fs = [(lambda W=W, Xq=Xq, sa=sa, Y=Y: q.q4_1_matmul_q8(Xq, sa, W, out=Y)) for W in ring]
            fs[0]()
            t = time_ring(torch, fs)
            b = wbytes + M * K + 4 * M + 4 * M * N
            q4q8["%dx%d_m%d" % (K, N, M)] = {"us": round(t * 1e6, 2), "GB/s": round(b / t / 1e9, 1),
                                             "%HBM": round(100 * b / t / 1e9 / HBM_PEAK_GBS, 2)}
        del ring, bd
    extra["q4_1_matmul"] = q4
    extra["q4_1_matmul_q8"] = q4q8

    # --------------------------------------------- MUL_MAT_ID ---
    for name, inputs, per_slot in (("q4_1_matmul_id", wl.moe_inputs, False),
                                   ("q4_1_matmul_id_per_slot", wl.moe_down_inputs, True)):
        dm = inputs()
        E = wl.MOE_EXPERTS
        K, N = (wl.MOE_DOWN_K, wl.MOE_DOWN_N) if per_slot else (wl.MOE_K, wl.MOE_N)
        ed = torch.from_numpy(dm["experts"]).to(dev)
        rings = [q.q4_1_repack_experts(ed, K, N) for _ in range(4)]   # 4 copies: ~500 MB
        X = torch.from_numpy(dm["X"]).to(dev)
        ids = torch.from_numpy(dm["ids"]).to(dev)
        Y = torch.empty((wl.MOE_TOKENS, wl.MOE_USED, N), dtype=torch.float32, device=dev)
        if per_slot:
            wsm = q.workspace(q.lib.qmm_q4_1_matmul_id_per_slot_workspace_bytes(wl.MOE_TOKENS, wl.MOE_USED, E, K, N),
                              dev)
            fs = [(lambda buf=buf, st=st: q.q4_1_matmul_id_per_slot(X, buf, E, K, N, st, ids, wl.MOE_USED, out=Y,
                                                                   ws=wsm)) for buf, st in rings]
        else:
            wsm = q.workspace(q.lib.qmm_q4_1_matmul_id_workspace_bytes(wl.MOE_TOKENS, wl.MOE_USED, E, K, N), dev)
            fs = [(lambda buf=buf, st=st: q.q4_1_matmul_id(X, buf, E, K, N, st, ids, wl.MOE_USED, out=Y, ws=wsm))
                  for buf, st in rings]
        fs[0]()
        t = time_ring(torch, fs * 2)
        b = q4_moe_bytes(wl, E, K, N, X, Y)
        extra[name] = {"us": round(t * 1e6, 2), "GB/s": round(b / t / 1e9, 1),
                       "%HBM": round(100 * b / t / 1e9 / HBM_PEAK_GBS, 2), "algorithmic_bytes": b,
                       "experts": E, "K": K, "N": N, "tokens": wl.MOE_TOKENS, "top_k": wl.MOE_USED}
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
        t = time_ring(torch, fs * 2)
        b = launch_bytes(M, K, [N])
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
        t = time_ring(torch, fs)
        b = wbytes + 4 * M * K + 4 * M * N
        lm["q4_1_m%d" % M] = {"us": round(t * 1e6, 2), "GB/s": round(b / t / 1e9, 1),
                              "%HBM": round(100 * b / t / 1e9 / HBM_PEAK_GBS, 2)}
    del ring
    extra["lm_head_1024x151936"] = lm

    # ------------- streaming-read floor: the call sizes, read cold ---
    from int8_bit_weight_amd.probe import read_probe
    floor = {}
    for nbytes in (4198400, 36700160, 155582464):
        nb = (nbytes + 15) // 16 * 16
        copies = max(4, -(-640 * 2 ** 20 // nb))                 # > 2 x (MALL + L2) in all
        bufs = [torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1) for _ in range(copies)]
        best = None
        for u in (1, 4, 8):
            for wg in (256, 1024, 4096):
                sink = torch.empty(wg, dtype=torch.int32, device=dev)

                def run_rd(bufs=bufs, sink=sink, wg=wg, u=u):
                    for b_ in bufs:
                        read_probe(b_, sink, wg, u)
                run_rd()
                tb = time_graph(torch, run_rd, 3) / len(bufs)
                key = "u%d_wg%d" % (u, wg)
                if best is None or tb < best[1]:
                    best = (key, tb)
        floor["%d_B" % nbytes] = {"best": best[0], "back_to_back_us": round(best[1] * 1e6, 2),
                                  "GB/s": round(nbytes / best[1] / 1e9, 1)}
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
    return extra


# ----------------------------------------------------------- CPU oracle ---

def cpu_oracle(wl, np, host_w, calls, projs, rows, layers, total_bytes):
    """The oracle as it stands, timed on the host cores: one whole step of
    the headline workload (the cpu_baseline), and every configuration (the
    large ones on a stated sample), with all threads and, for the small
    configurations, one thread."""
    import oracle
    threads = oracle.num_threads()
    log("cpu baseline: oracle on one whole step (%d threads)" % threads)
    qb = {k: oracle.pack_b_int8(w) for k, w in host_w.items()}
    xs = {M: [c[3].cpu().numpy() for c in calls[M]] for M in rows}

    def step(layer_set):
        for M in rows:
            for c, X in zip(calls[M], xs[M]):
                if c[0] not in layer_set:
                    continue
                Qa, sa = oracle.quantize_rows_int8(X)
                for p in c[1]:
                    Qb, sb, _ = qb[(c[0], p)]
                    oracle.epilogue_f64(oracle.int8_gemm_i64(Qa, 0, Qb, 0), sa, sb)

    t0 = time.perf_counter()
    step(set(range(layers)))
    tc = time.perf_counter() - t0
    cpu = {"value": round(total_bytes / tc / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": "one whole step (%d launches' projections: %d layers x 7 projections x M in {1,16,32}), "
                     "%.2f s" % (sum(len(calls[M]) for M in rows), layers, tc)}
    tim = {"cpu_model": cpu_model(), "threads": threads}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    def both(fn):
        ta = timed(fn)
        oracle.set_num_threads(1)
        try:
            t1 = timed(fn)
        finally:
            oracle.set_num_threads(threads)
        return ta, t1

    # config 1: the zero-point product with both outputs
    d = wl.int8_product_inputs(M=16, K=1024, N=1024)

    def c1():
        Y = oracle.int8_gemm_i64(d["A"], d["zA"], d["B"], d["zB"])
        oracle.epilogue_f64(Y, None, None, d["scale"], d["bias"])
    ta, t1 = both(c1)
    tim["zero_point_product_16x1024x1024"] = {"s_all_threads": round(ta, 4), "s_one_thread": round(t1, 4),
                                              "GB/s_all_threads": round(1204224 / ta / 1e9, 4)}
    # config 2: one layer on one thread (the whole step is the cpu_baseline)
    t1 = 0.0
    oracle.set_num_threads(1)
    try:
        t1 = timed(lambda: step({0}))
    finally:
        oracle.set_num_threads(threads)
    lb = sum(projs[p][1] * projs[p][2] for M in rows for c in calls[M] if c[0] == 0 for p in c[1])
    tim["projections_one_layer_one_thread"] = {"s": round(t1, 3), "weight_bytes": lb,
                                               "sample": "layer 0's 7 projections at M in {1,16,32}"}
    # config 3: q4_1 4096 x 14336, M = 1 in full on both; M = 16 on all threads
    K, N = wl.Q4_SHAPES[0]
    _, blocks = wl.q4_weight(K, N, seed_index=0)
    X1 = wl.q4_activations(1, K, seed_index=0)
    X16 = wl.q4_activations(16, K, seed_index=0)
    ta, t1 = both(lambda: oracle.q4_1_matmul(X1, blocks, K, N))
    t16 = timed(lambda: oracle.q4_1_matmul(X16, blocks, K, N))
    tim["q4_1_4096x14336"] = {"m1_s_all_threads": round(ta, 4), "m1_s_one_thread": round(t1, 4),
                              "m16_s_all_threads": round(t16, 4)}
    # config 4: the 4096 x 4096 prefill on 32 of its 2048 rows (scaled)
    K, N = wl.PREFILL_SHAPES[0]
    dp = wl.prefill_inputs(K, N, seed_index=0)
    Qb, sb, _ = oracle.pack_b_int8(dp["W"])
    A32 = np.ascontiguousarray(dp["A"][:32])
    ts = timed(lambda: oracle.epilogue_f64(oracle.int8_gemm_i64(A32, 0, Qb, 0), dp["rs"][:32], sb))
    tim["prefill_4096x4096"] = {"sample": "32 of 2048 rows", "s_sample": round(ts, 3),
                                "s_full_scaled": round(ts * wl.PREFILL_M / 32, 2),
                                "GOPS": round(2.0 * 32 * K * N / ts / 1e9, 2)}
    # config 5: MUL_MAT_ID on 16 of 512 tokens (scaled)
    dm = wl.moe_inputs()
    ts = timed(lambda: oracle.q4_1_matmul_id(dm["X"][:16], dm["experts"], wl.MOE_EXPERTS, wl.MOE_K, wl.MOE_N,
                                             dm["ids"][:16], wl.MOE_USED))
    tim["q4_1_matmul_id"] = {"sample": "16 of 512 tokens", "s_sample": round(ts, 3),
                             "s_full_scaled": round(ts * wl.MOE_TOKENS / 16, 2)}
    return cpu, tim


if __name__ == "__main__":
    sys.exit(main())
