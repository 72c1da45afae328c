#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X: fp32 GEMM at 2048^3 and the
2-bit GEMV at 12,288 x 1,536.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

A step is one pass of the whole path over one batch of synthetic input:
  * one gemm_f32 of two 2048 x 2048 fp32 matrices (uniform [-1, 1), seed 3),
    the largest size of the kernel sweep in "I built a GPT-2 in the browser,
    then made it 2.6x-12.1x faster" (section "The kernel sweep");
  * one token of 2-bit GEMVs: 40 consecutive gemv_q2 calls ("Kernel 0112",
    section "What is being measured": the kernel runs 40 times per token),
    call n using weight matrix n mod 128 of a 128-matrix set (648 MiB of codes
    and scales, far above the 256 MB Infinity Cache, as the page's "cold"
    rotation keeps reuse between runs unlikely).
Every input is generated, hashed and copied to HBM before timing.  Launches
are captured into HIP graphs (through torch.cuda.CUDAGraph) so that timed
regions replay kernels back to back, without host launch gaps.  HIP events on
the replay stream time K whole steps (ms_per_step), and, for each kernel's
average launch duration, runs of back-to-back launches of that kernel alone
(K GEMMs; K tokens of 40 q2 calls).

Output: one JSON line.  `value` is the GEMM's TFLOP/s (2 * 2048^3 flops per
launch over its average launch duration); the 2-bit GEMV's weight GB/s
(codes + scales per call over its average duration) is in `q2_gemv`.  Both
carry a roofline object.  `q2_gemv_batched` times the same tokens with each
token's 40 products in one gemv_q2_batched launch; `q4_gemv` times the 4-bit
product the same two ways, `q2_gemv_transposed` the 2-bit product at the
transposed 1,536 x 12,288 shape, and `gemv_f32` the fp32 product.  Before any number is
printed the outputs are checked against the CPU oracle on sampled cells; a
failing kernel reports no speed.  `cpu_baseline` times the oracle itself on a bounded sample.
After the main timing, `spread` gives each kernel's per-launch median, p10,
p90 and minimum over 16 single replays, and `context` the 2-bit GEMV on one
cache-resident matrix (its launch-and-compute floor) and the rate of a plain
device-to-device copy.  `gemm_configs` checks and times the other GEMM
configurations: the nine products of a GPT-2-small block at 1,024 tokens
(alone and as one graph), the 346 x 768 x 768 classifier layer and 256^3.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

GEMM_N = 2048
GEMM_FLOPS = 2 * GEMM_N ** 3                       # 17,179,869,184
Q2_M, Q2_K = 12288, 1536
Q2_CODE_BYTES = Q2_M * Q2_K // 4                   # 4,718,592
Q2_SCALE_BYTES = Q2_M * (Q2_K // 64) * 2           # 589,824
Q2_WEIGHT_BYTES = Q2_CODE_BYTES + Q2_SCALE_BYTES   # 5,308,416
Q2_ALG_BYTES = Q2_WEIGHT_BYTES + Q2_K * 4 + Q2_M * 4   # + x + y = 5,363,712
Q2_ROTATION = 128
CALLS_PER_TOKEN = 40
Q4_CODE_BYTES = Q2_M * Q2_K // 2                   # 9,437,184
Q4_WEIGHT_BYTES = Q4_CODE_BYTES + Q2_SCALE_BYTES   # 10,027,008
Q4_ALG_BYTES = Q4_WEIGHT_BYTES + Q2_K * 4 + Q2_M * 4   # + x + y = 10,082,304
Q4_ROTATION = 64                                   # 642 MB of codes+scales
QT_M, QT_K = 1536, 12288                           # the transposed 2-bit shape
F32_ROTATION = 48                                  # 3.375 GiB of fp32 weights
F32_ALG_BYTES = Q2_M * Q2_K * 4 + Q2_K * 4 + Q2_M * 4   # W + x + y = 75,552,768
QT_ALG_BYTES = Q2_WEIGHT_BYTES + QT_K * 4 + QT_M * 4   # 5,363,712

PEAK_FP32_MFMA_TFLOPS = 157.3      # MI355X dense fp32 matrix peak
PEAK_HBM_GBS = 8000.0              # MI355X HBM3E
# "I built a GPT-2 in the browser...", table of section "The kernel sweep":
# blocked4 at 2048^3 took 9.12 ms on an Apple M-series laptop (WebGPU).
PAGE_GEMM_2048_TFLOPS = GEMM_FLOPS / 9.12e-3 / 1e12

PROFILES = os.path.join(ROOT, "profiles")
CALIBRATION_BYTES = 256 << 20      # the copy used to scale byte counters


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gemv_gemm_f32_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(name, sha):
    """HBM bytes per launch measured with rocprofv3 counters, if they were
    taken on the kernel source as it is now; else None."""
    path = os.path.join(PROFILES, name)
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_src_sha") != sha:
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(A, B, Q, S, x, budget_s=12.0):
    """The oracle, single-threaded as written, on a bounded sample of the
    same workload: leading rows of the 2048^3 product, sized to about
    `budget_s` seconds, and whole 2-bit GEMVs on one rotation matrix."""
    import oracle
    oracle.build(force=False)
    # calibrate on 4 rows, then fill the budget (at most all 2048 rows)
    t0 = time.perf_counter()
    oracle.gemm_nn(A[:4], B)
    t4 = time.perf_counter() - t0
    rows = int(max(4, min(GEMM_N, 4 * (0.75 * budget_s) / max(t4, 1e-6))))
    t0 = time.perf_counter()
    oracle.gemm_nn(A[:rows], B)
    tg = time.perf_counter() - t0
    gemm_tflops = 2.0 * rows * GEMM_N * GEMM_N / tg / 1e12
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.gemv_q2(Q, S, x)
        reps += 1
        if time.perf_counter() - t0 > 0.25 * budget_s or reps >= 50:
            break
    tq = (time.perf_counter() - t0) / reps
    return {
        "value": gemm_tflops,
        "unit": "TFLOP/s",
        "cores": 1,
        "kind": "oracle",
        "sample": ("fp64 triple-loop oracle: rows 0..%d of the 2048^3 product "
                   "(%.1f s); 2-bit unpack-then-dot oracle on one 12288x1536 "
                   "matrix, %d calls" % (rows - 1, tg, reps)),
        "q2_gemv_weight_gbs": Q2_WEIGHT_BYTES / tq / 1e9,
        "cpu": platform.processor() or platform.machine(),
    }


def vendor_context(torch, stream, capture, timed, token_runner, n_tok, per_replay, dA, dB, Wf,
                   dx, A, B, args):
    """The vendor library on the same inputs, for context only (never part of
    the library's path): torch.matmul in fp32 with TF32 off (hipBLASLt or
    rocBLAS) at 2048^3, and torch.mv over the fp32 GEMV rotation set, timed
    like the library's kernels (back-to-back launches in graph replays)."""
    out = {"note": ("torch.matmul / torch.mv in fp32 with TF32 off on the same operands, "
                    "graph-replayed back to back like the library's kernels: context, "
                    "not part of the library")}
    try:
        torch.backends.cuda.matmul.allow_tf32 = False
        C = torch.empty_like(dA)
        with torch.cuda.stream(stream):
            torch.matmul(dA, dB, out=C)
            stream.synchronize()
        ref = (A[:4].astype(np.float64) @ B.astype(np.float64))
        err = float(np.max(np.abs(C[:4].cpu().numpy() - ref)))
        g = capture(lambda: [torch.matmul(dA, dB, out=C) for _ in range(per_replay)])
        reps = max(1, (args.steps + per_replay - 1) // per_replay)

        def run(i):
            if i is not None:
                g.replay()
                return 1
            for _ in range(reps):
                g.replay()
            return reps * per_replay
        ms, n, _ = timed(run, 2)
        us = 1e3 * ms / n
        out["matmul_2048_us"] = us
        out["matmul_2048_tflops"] = GEMM_FLOPS / us / 1e6
        out["matmul_2048_max_abs_err_first_rows"] = err
        y = torch.empty(Q2_M, dtype=torch.float32, device=dA.device)

        def tok(t):
            for c in range(CALLS_PER_TOKEN):
                torch.mv(Wf[(t * CALLS_PER_TOKEN + c) % F32_ROTATION], dx, out=y)
        with torch.cuda.stream(stream):
            tok(0)
            stream.synchronize()
        graphs = [capture(lambda t=t: tok(t)) for t in range(n_tok)]
        ms, n, _ = timed(token_runner(graphs), 2)
        us = 1e3 * ms / n
        out["mv_12288x1536_us"] = us
        out["mv_12288x1536_gbs"] = F32_ALG_BYTES / us / 1e3
    except Exception as e:   # context only: report, never fail the bench
        out["error"] = "%s: %s" % (type(e).__name__, e)
    return out


def gemm_configs(torch, bd, inputs, oracle, dev, stream, capture, timed, steps, per_replay=8):
    """The GEMM configurations besides 2048^3, each checked against the oracle
    on sampled cells before it is timed: the nine products of a GPT-2-small
    block at 1,024 tokens (three forward, six backward; "I built a GPT-2 in
    the browser...", section "The kernel sweep", where matmul is most of
    training time), the 346 x 768 x 768 classifier layer (the 346-token
    prompt of the polyomino classifier page) and 256^3.  Each product is
    timed over back-to-back launches in graph replays (the median of three
    interleaved rounds), the block's nine products also as one graph;
    torch.matmul (fp32, TF32 off) on the same operands is context only.  A
    product that fails parity reports no time."""
    torch.backends.cuda.matmul.allow_tf32 = False
    entry = {"nn": bd.gemm_f32, "tn": bd.gemm_f32_tn, "nt": bd.gemm_f32_nt}
    rng = np.random.default_rng(77)
    t = inputs.gpt2_tensors(2)
    ops = [(name, lay, M, N, K, t[an], t[bn]) for name, lay, M, N, K, (an, bn) in inputs.GPT2_OPS]
    A346, B346 = inputs.classifier(33)
    A256, B256 = inputs.small_square(0)
    ops += [("classifier_346x768x768", "nn", 346, 768, 768, A346, B346),
            ("square_256", "nn", 256, 256, 256, A256, B256)]
    reps = max(1, (steps + per_replay - 1) // per_replay)
    out, launches, all_ok = {}, [], True
    timing = []                # (name, our graph, vendor graph or error, flops)
    for name, lay, M, N, K, A, B in ops:
        dA, dB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
        dC = torch.empty((M, N), dtype=torch.float32, device=dev)
        f = entry[lay]
        f(dA, dB, C=dC)
        C = dC.cpu().numpy()
        rows = np.concatenate([rng.integers(0, M, 384), [0, 0, M - 1, M - 1]])
        cols = np.concatenate([rng.integers(0, N, 384), [0, N - 1, 0, N - 1]])
        ref, bound = oracle.gemm_cells(A, B, rows, cols, trans_a=lay == "tn", trans_b=lay == "nt")
        ok, worst, _ = oracle.check(C[rows, cols], ref, bound)
        all_ok = all_ok and ok
        out[name] = {"shape": "%s %dx%dx%d" % (lay.upper(), M, N, K),
                     "parity": "pass" if ok else "FAIL", "worst_err_over_bound": worst}
        flops = 2.0 * M * N * K
        if name in {o[0] for o in inputs.GPT2_OPS}:
            launches.append((f, dA, dB, dC, flops))
        if not ok:
            continue
        g = capture(lambda f=f, dA=dA, dB=dB, dC=dC: [f(dA, dB, C=dC) for _ in range(per_replay)])
        try:
            oa = dA.t() if lay == "tn" else dA
            ob = dB.t() if lay == "nt" else dB
            gv = capture(lambda oa=oa, ob=ob, dC=dC: [torch.matmul(oa, ob, out=dC)
                                                      for _ in range(per_replay)])
        except Exception as e:   # context only
            gv = "%s: %s" % (type(e).__name__, e)
        timing.append((name, g, gv, flops))

    def runner(graph):
        def run(i):
            if i is not None:
                graph.replay()
                return 1
            for _ in range(reps):
                graph.replay()
            return reps * per_replay
        return run

    def one_us(graph):
        stream.synchronize()
        ms, n, _ = timed(runner(graph), 4)
        return 1e3 * ms / n

    # Three rounds over every product (ours, then the vendor's), the median
    # per product: a product timed right after the parity checks, or after a
    # long burst of these launches, has read up to 1.8x slow on some boxes,
    # and interleaving spreads such spells over all of them.
    ours, vend = {n: [] for n, *_ in timing}, {n: [] for n, *_ in timing}
    for _ in range(3):
        for name, g, gv, _ in timing:
            ours[name].append(one_us(g))
            if not isinstance(gv, str):
                vend[name].append(one_us(gv))
    for name, g, gv, flops in timing:
        d = out[name]
        d["us"] = float(np.median(ours[name]))
        d["us_rounds"] = ours[name]
        d["tflops"] = flops / d["us"] / 1e6
        d["frac_of_fp32_mfma_peak"] = d["tflops"] / PEAK_FP32_MFMA_TFLOPS
        if isinstance(gv, str):
            d["vendor_error"] = gv
        else:
            d["vendor_torch_matmul_us"] = float(np.median(vend[name]))
    if all_ok:
        g = capture(lambda: [f(dA, dB, C=dC) for f, dA, dB, dC, _ in launches])

        def runb(i):
            if i is not None:
                g.replay()
                return 1
            for _ in range(steps):
                g.replay()
            return steps
        stream.synchronize()
        ms, n, _ = timed(runb, 4)
        us = 1e3 * ms / n
        total = sum(fl for *_, fl in launches)
        out["gpt2_block_9_products"] = {
            "us": us, "tflops": total / us / 1e6,
            "frac_of_fp32_mfma_peak": total / us / 1e6 / PEAK_FP32_MFMA_TFLOPS,
            "vendor_torch_matmul_us_sum": sum(out[o[0]].get("vendor_torch_matmul_us", float("nan"))
                                              for o in inputs.GPT2_OPS),
            "note": "F1..B3w back to back in one graph, 39,862,665,216 flop per block"}
    return out, all_ok


def host_cpu():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _short_name(kernel):
    k = kernel.replace("void gg::(anonymous namespace)::", "")
    return k.split("(")[0]


def _key(kernel, grid=None, wg=None):
    """A kernel's short name, and its workgroup count when the database gives
    the launch shape: one kernel launched at several shapes gets a row per
    shape."""
    k = _short_name(kernel)
    if grid and wg:
        k += " @%dwg" % (grid // wg)
    return k


def summarize_trace(db_path):
    """Per-kernel (and launch shape) count / total / average / min / max /
    median duration (us) from a rocprofv3 results database."""
    import sqlite3
    db = sqlite3.connect(db_path)
    try:
        rows = db.execute("select name, duration, grid_x * grid_y * grid_z, "
                          "workgroup_x * workgroup_y * workgroup_z from kernels").fetchall()
    except sqlite3.OperationalError:
        rows = [(n, d, None, None) for n, d in
                db.execute("select name, duration from kernels").fetchall()]
    by = {}
    for name, dur, grid, wg in rows:
        by.setdefault(_key(name, grid, wg), []).append(dur / 1e3)
    lines = ["| kernel | calls | total us | avg us | min us | max us | median us |",
             "|---|---|---|---|---|---|---|"]
    for k, d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        d = np.array(d)
        lines.append("| %s | %d | %.1f | %.3f | %.3f | %.3f | %.3f |" %
                     (k, len(d), d.sum(), d.mean(), d.min(), d.max(), np.median(d)))
    return "\n".join(lines)


def _counter_dispatches(db_path, counter):
    """Per kernel key: {dispatch id: the counter summed over its instances}."""
    import sqlite3
    db = sqlite3.connect(db_path)
    try:
        rows = db.execute("select kernel_name, dispatch_id, value, grid_size, workgroup_size "
                          "from counters_collection where counter_name = ?",
                          (counter,)).fetchall()
    except sqlite3.OperationalError:
        rows = [r + (None, None) for r in
                db.execute("select kernel_name, dispatch_id, value from counters_collection "
                           "where counter_name = ?", (counter,)).fetchall()]
    per = {}
    for name, disp, v, grid, wg in rows:
        k = _key(name, grid, wg)
        per.setdefault(k, {}).setdefault(disp, 0.0)
        per[k][disp] += v
    return per


def _median_per_kernel(per):
    return {k: float(np.median(list(v.values()))) for k, v in per.items()}


def write_traffic(fetch_db, write_db):
    """HBM bytes per launch of the GEMM and the 2-bit GEMV: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch, median over dispatches), each scaled by
    what the same counter reads for the calibration copy of known size."""
    fetch_d = _counter_dispatches(fetch_db, "FETCH_SIZE")
    write_d = _counter_dispatches(write_db, "WRITE_SIZE")
    fetch, write = _median_per_kernel(fetch_d), _median_per_kernel(write_d)
    copies = [(k, d) for k in write_d if "copyBuffer" in k for d in write_d[k]]
    if not copies:
        sys.exit("no copy kernel in the trace: run with --copy-calibration")
    nbytes = CALIBRATION_BYTES
    # The calibration copy is the copy dispatch that wrote closest to its
    # size (input uploads are smaller, the copy-rate context larger); both
    # runs execute the same program, so it has the same dispatch id in each.
    ck, disp = min(copies, key=lambda kd: abs(write_d[kd[0]][kd[1]] * 1024.0 - nbytes))
    if disp not in fetch_d.get(ck, {}):
        sys.exit("calibration copy (dispatch %d) missing from the FETCH_SIZE run" % disp)
    fetch[ck], write[ck] = fetch_d[ck][disp], write_d[ck][disp]
    f_scale = nbytes / (fetch[ck] * 1024.0)
    w_scale = nbytes / (write[ck] * 1024.0)
    out = []
    q2_srcs = ("gemv_packed.hip", "wave.hpp")
    for match, fname, srcs, alg in (
            (lambda n: n.startswith("gemm_f32_direct<64, 64, true, false, 2,")
             and ("@" not in n or n.endswith(" @%dwg" % (GEMM_N // 64) ** 2)),
             "traffic_gemm_f32_2048.json", ("gemm_f32.hip",), 3 * 4 * GEMM_N * GEMM_N),
            (lambda n: n.startswith("gemv_packed_flat<2, 1, 1,"),
             "traffic_gemv_q2_12288x1536.json", q2_srcs, Q2_ALG_BYTES),
            (lambda n: n.startswith("gemv_packed_flat<2, 8, 64,"),
             "traffic_gemv_q2_batched_12288x1536.json", q2_srcs,
             CALLS_PER_TOKEN * Q2_ALG_BYTES),
            (lambda n: n.startswith("gemv_packed_flat<4, 2, 1,"),
             "traffic_gemv_q4_12288x1536.json", q2_srcs, Q4_ALG_BYTES),
            (lambda n: n.startswith("gemv_packed_flat<4, 8, 64,"),
             "traffic_gemv_q4_batched_12288x1536.json", q2_srcs,
             CALLS_PER_TOKEN * Q4_ALG_BYTES),
            (lambda n: n.startswith("gemv_packed_kernel<2, 256, 6,")
             and n.split(" @")[0].endswith(", 1>"),
             "traffic_gemv_q2_1536x12288.json", q2_srcs, QT_ALG_BYTES),
            (lambda n: n.startswith("gemv_f32_kernel<1, 6, true>"),
             "traffic_gemv_f32_12288x1536.json", ("gemv_f32.hip", "wave.hpp"), F32_ALG_BYTES)):
        k = [n for n in fetch if match(n)]
        if not k:
            continue
        k = k[0]
        fb = fetch[k] * 1024.0 * f_scale
        wb = write[k] * 1024.0 * w_scale
        d = {"kernel": k, "kernel_src_sha": src_sha(*srcs),
             "fetch_kib_raw": fetch[k], "write_kib_raw": write[k],
             "copy_bytes": nbytes, "copy_fetch_kib_raw": fetch[ck],
             "copy_write_kib_raw": write[ck], "fetch_scale": f_scale,
             "write_scale": w_scale, "hbm_bytes_per_launch": fb + wb,
             "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
             "algorithmic_bytes_per_launch": alg,
             "traffic_over_algorithmic": (fb + wb) / alg}
        with open(os.path.join(PROFILES, fname), "w") as f:
            json.dump(d, f, indent=1)
            f.write("\n")
        out.append(d)
        print(json.dumps(d))
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="also run one device-to-device copy of BYTES before "
                         "timing, the reference for rocprofv3 byte counters")
    ap.add_argument("--summarize-trace", metavar="RESULTS_DB",
                    help="print the per-kernel summary of a rocprofv3 "
                         "--kernel-trace --stats database and exit")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="turn two rocprofv3 --pmc databases (FETCH_SIZE, "
                         "WRITE_SIZE) of a run made with --copy-calibration "
                         "into per-launch HBM bytes under profiles/, and exit")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return 0
    if args.traffic:
        return write_traffic(*args.traffic)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the products here are not "
              "sharded and no collective is built (asked for --gpus %d)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        sys.exit("need --steps >= 1 and --warmup >= 0")

    import torch
    from gemv_gemm_f32_amd import binding as bd
    from gemv_gemm_f32_amd import inputs

    bd.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    prop = torch.cuda.get_device_properties(dev)
    log("device: %s %s, %d CUs" % (prop.name, getattr(prop, "gcnArchName", "?"),
                                   prop.multi_processor_count))

    # ---- inputs, hashed, resident in HBM before timing
    t0 = time.perf_counter()
    A, B = inputs.large_square(3)
    dA, dB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    dC = torch.empty((GEMM_N, GEMM_N), dtype=torch.float32, device=dev)
    x = inputs.q2_x()
    dx = torch.from_numpy(x).to(dev)
    Qd, Sd, hq = [], [], hashlib.sha256()
    Q0 = S0 = None
    for r in range(Q2_ROTATION):
        Q, S = inputs.q2_weight(r)
        if r == 0:
            Q0, S0 = Q, S
        hq.update(Q.tobytes())
        hq.update(S.tobytes())
        Qd.append(torch.from_numpy(Q).to(dev))
        Sd.append(torch.from_numpy(S.view(np.int16)).to(dev))
    dy = torch.empty(Q2_M, dtype=torch.float32, device=dev)
    Q4d, S4d, h4 = [], [], hashlib.sha256()
    Q40 = S40 = None
    for r in range(Q4_ROTATION):
        Q, S = inputs.q4_weight(r)
        if r == 0:
            Q40, S40 = Q, S
        h4.update(Q.tobytes())
        h4.update(S.tobytes())
        Q4d.append(torch.from_numpy(Q).to(dev))
        S4d.append(torch.from_numpy(S.view(np.int16)).to(dev))
    # fp32 GEMV: 48 matrices of 12,288 x 1,536 (3.375 GiB), the same x
    # length; drawn on a few host threads, uploaded one by one
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=min(8, len(os.sched_getaffinity(0)))) as pool:
        Wf = [torch.from_numpy(W).to(dev)
              for W in pool.map(inputs.gemv_f32_weight, range(F32_ROTATION))]
    W0 = Wf[0].cpu().numpy()
    xf = inputs.gemv_f32_x()
    dxf = torch.from_numpy(xf).to(dev)
    # the transposed shape: 1,536 rows of 12,288 columns, same bytes per matrix
    xt = inputs.q2_x(QT_K)
    dxt = torch.from_numpy(xt).to(dev)
    QTd, STd, ht = [], [], hashlib.sha256()
    QT0 = ST0 = None
    for r in range(Q2_ROTATION):
        Q, S = inputs.q2_weight(r, QT_M, QT_K)
        if r == 0:
            QT0, ST0 = Q, S
        ht.update(Q.tobytes())
        ht.update(S.tobytes())
        QTd.append(torch.from_numpy(Q).to(dev))
        STd.append(torch.from_numpy(S.view(np.int16)).to(dev))
    dyt = torch.empty(QT_M, dtype=torch.float32, device=dev)
    dyts = [torch.empty(QT_M, dtype=torch.float32, device=dev) for _ in range(CALLS_PER_TOKEN)]
    torch.cuda.synchronize()
    hashes = {"gemm_A_B": inputs.sha256(A, B)[:16], "q2_x": inputs.sha256(x)[:16],
              "q2_set": hq.hexdigest()[:16], "q4_set": h4.hexdigest()[:16],
              "q2_transposed_set": ht.hexdigest()[:16], "q2_transposed_x": inputs.sha256(xt)[:16]}
    log("inputs ready in %.1f s" % (time.perf_counter() - t0))

    # ---- parity first: a wrong kernel reports no speed
    import oracle
    bd.gemm_f32(dA, dB, C=dC)
    bd.gemv_q2(Qd[0], Sd[0], dx, y=dy)
    C = dC.cpu().numpy()
    y = dy.cpu().numpy()
    rng = np.random.default_rng(2024)
    rows, cols = rng.integers(0, GEMM_N, 512), rng.integers(0, GEMM_N, 512)
    ref, bound = oracle.gemm_cells(A, B, rows, cols)
    gemm_ok, gemm_worst, _ = oracle.check(C[rows, cols], ref, bound)
    yref, ybound = oracle.gemv_q2(Q0, S0, x)
    q2_ok, q2_worst, _ = oracle.check(y, yref, ybound)
    # the batched entry point on token 0's 40 products, checked on 3 of them
    dys = [torch.empty(Q2_M, dtype=torch.float32, device=dev) for _ in range(CALLS_PER_TOKEN)]
    bd.gemv_q2_batched(Qd[:CALLS_PER_TOKEN], Sd[:CALLS_PER_TOKEN], [dx] * CALLS_PER_TOKEN, ys=dys)
    qb_ok, qb_worst = True, 0.0
    for b in (0, 17, CALLS_PER_TOKEN - 1):
        Qb, Sb = inputs.q2_weight(b)
        rb, bb = oracle.gemv_q2(Qb, Sb, x)
        ok, worst, _ = oracle.check(dys[b].cpu().numpy(), rb, bb)
        qb_ok, qb_worst = qb_ok and ok, max(qb_worst, worst)
    bd.gemv_q4(Q4d[0], S4d[0], dx, y=dy)
    y4ref, y4bound = oracle.gemv_q4(Q40, S40, x)
    q4_ok, q4_worst, _ = oracle.check(dy.cpu().numpy(), y4ref, y4bound)
    bd.gemv_q4_batched(Q4d[:CALLS_PER_TOKEN], S4d[:CALLS_PER_TOKEN], [dx] * CALLS_PER_TOKEN,
                       ys=dys)
    q4b_ok, q4b_worst = True, 0.0
    for b in (0, CALLS_PER_TOKEN - 1):
        Qb, Sb = inputs.q4_weight(b)
        rb, bb = oracle.gemv_q4(Qb, Sb, x)
        ok, worst, _ = oracle.check(dys[b].cpu().numpy(), rb, bb)
        q4b_ok, q4b_worst = q4b_ok and ok, max(q4b_worst, worst)
    bd.gemv_f32(Wf[0], dxf, y=dy)
    yfref, yfbound = oracle.gemv(W0, xf)
    gf_ok, gf_worst, _ = oracle.check(dy.cpu().numpy(), yfref, yfbound)
    bd.gemv_q2(QTd[0], STd[0], dxt, y=dyt)
    ytref, ytbound = oracle.gemv_q2(QT0, ST0, xt)
    qt_ok, qt_worst, _ = oracle.check(dyt.cpu().numpy(), ytref, ytbound)
    log("parity: gemm worst %.3g, q2 worst %.3g, q2 batched worst %.3g, q4 worst %.3g, "
        "q4 batched worst %.3g, q2 transposed worst %.3g, gemv_f32 worst %.3g (x 1e-4 bound)" %
        (gemm_worst / 1e-4, q2_worst / 1e-4, qb_worst / 1e-4, q4_worst / 1e-4,
         q4b_worst / 1e-4, qt_worst / 1e-4, gf_worst / 1e-4))

    if args.copy_calibration > 0:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: %d bytes" % (4 * n))
        del src, dst

    # ---- graphs.  A token is 40 q2 calls; 16 tokens cover the 128-matrix
    #      rotation (lcm(40, 128) = 640 calls), so call n uses matrix n mod 128.
    #      step_graphs[t]: one whole step (the GEMM, then token t).
    #      gemm_graph: GEMMS_PER_REPLAY back-to-back GEMMs; tok_graphs[t]:
    #      token t alone.  Those two time each kernel over runs of
    #      back-to-back launches, so a kernel's average launch duration
    #      carries no per-replay overhead.
    stream = torch.cuda.Stream(device=dev)
    n_tok = 16
    gemms_per_replay = 8
    with torch.cuda.stream(stream):
        for _ in range(3):
            bd.gemm_f32(dA, dB, C=dC)
            bd.gemv_q2(Qd[0], Sd[0], dx, y=dy)
    stream.synchronize()

    def token(t):
        for c in range(CALLS_PER_TOKEN):
            n = t * CALLS_PER_TOKEN + c
            bd.gemv_q2(Qd[n % Q2_ROTATION], Sd[n % Q2_ROTATION], dx, y=dy)

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        return g

    def token_batched(t):
        idx = [(t * CALLS_PER_TOKEN + c) % Q2_ROTATION for c in range(CALLS_PER_TOKEN)]
        bd.gemv_q2_batched([Qd[i] for i in idx], [Sd[i] for i in idx],
                           [dx] * CALLS_PER_TOKEN, ys=dys)

    step_graphs = [capture(lambda t=t: (bd.gemm_f32(dA, dB, C=dC), token(t)))
                   for t in range(n_tok)]
    btok_graphs = [capture(lambda t=t: token_batched(t)) for t in range(n_tok)]

    def token4(t):
        for c in range(CALLS_PER_TOKEN):
            n = (t * CALLS_PER_TOKEN + c) % Q4_ROTATION
            bd.gemv_q4(Q4d[n], S4d[n], dx, y=dy)

    def token4_batched(t):
        idx = [(t * CALLS_PER_TOKEN + c) % Q4_ROTATION for c in range(CALLS_PER_TOKEN)]
        bd.gemv_q4_batched([Q4d[i] for i in idx], [S4d[i] for i in idx],
                           [dx] * CALLS_PER_TOKEN, ys=dys)

    def tokent(t):
        for c in range(CALLS_PER_TOKEN):
            n = (t * CALLS_PER_TOKEN + c) % Q2_ROTATION
            bd.gemv_q2(QTd[n], STd[n], dxt, y=dyt)

    def tokent_batched(t):
        idx = [(t * CALLS_PER_TOKEN + c) % Q2_ROTATION for c in range(CALLS_PER_TOKEN)]
        bd.gemv_q2_batched([QTd[i] for i in idx], [STd[i] for i in idx],
                           [dxt] * CALLS_PER_TOKEN, ys=dyts)

    def tokenf(t):
        for c in range(CALLS_PER_TOKEN):
            bd.gemv_f32(Wf[(t * CALLS_PER_TOKEN + c) % F32_ROTATION], dxf, y=dy)

    tokf_graphs = [capture(lambda t=t: tokenf(t)) for t in range(n_tok)]
    tokt_graphs = [capture(lambda t=t: tokent(t)) for t in range(n_tok)]
    btokt_graphs = [capture(lambda t=t: tokent_batched(t)) for t in range(n_tok)]
    tok4_graphs = [capture(lambda t=t: token4(t)) for t in range(n_tok)]
    btok4_graphs = [capture(lambda t=t: token4_batched(t)) for t in range(n_tok)]
    tok_graphs = [capture(lambda t=t: token(t)) for t in range(n_tok)]
    gemm_graph = capture(lambda: [bd.gemm_f32(dA, dB, C=dC)
                                  for _ in range(gemms_per_replay)])
    torch.cuda.synchronize()

    def timed(replays, warm):
        """HIP events on the replay stream around back-to-back replays."""
        with torch.cuda.stream(stream):
            for i in range(warm):
                replays(i)
            stream.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            t = time.perf_counter()
            n = replays(None)
            e1.record(stream)
            stream.synchronize()
            t = time.perf_counter() - t
        return e0.elapsed_time(e1), n, t

    def spread(graphs, launches, n=16):
        """Per-launch durations over n single replays of graphs (run after the
        main timing, one event pair per replay): median, p10, p90, min in us."""
        with torch.cuda.stream(stream):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
            ev[0].record(stream)
            for k in range(n):
                graphs[k % len(graphs)].replay()
                ev[k + 1].record(stream)
            stream.synchronize()
        us = sorted(1e3 * ev[k].elapsed_time(ev[k + 1]) / launches for k in range(n))
        q = lambda f: us[min(n - 1, int(round(f * (n - 1))))]
        return {"median_us": q(0.5), "p10_us": q(0.1), "p90_us": q(0.9), "min_us": us[0],
                "replays": n, "launches_per_replay": launches,
                "note": ("an event pair per replay: medians run a few percent above "
                         "the uninterrupted back-to-back averages")}

    def run_steps(i):
        if i is not None:
            step_graphs[i % n_tok].replay()
            return 1
        for s in range(args.steps):
            step_graphs[(args.warmup + s) % n_tok].replay()
        return args.steps

    n_gemm_replays = max(1, (args.steps + gemms_per_replay - 1) // gemms_per_replay)

    def run_gemms(i):
        if i is not None:
            gemm_graph.replay()
            return 1
        for _ in range(n_gemm_replays):
            gemm_graph.replay()
        return n_gemm_replays * gemms_per_replay

    def run_tokens(i):
        if i is not None:
            tok_graphs[i % n_tok].replay()
            return 1
        for s in range(args.steps):
            tok_graphs[s % n_tok].replay()
        return args.steps * CALLS_PER_TOKEN

    def token_runner(graphs):
        def run(i):
            if i is not None:
                graphs[i % n_tok].replay()
                return 1
            for s in range(args.steps):
                graphs[s % n_tok].replay()
            return args.steps * CALLS_PER_TOKEN
        return run

    run_btokens = token_runner(btok_graphs)

    total_ms, _, t_wall = timed(run_steps, args.warmup)
    gemm_ms, n_gemm, _ = timed(run_gemms, max(1, args.warmup // gemms_per_replay))
    tok_ms, n_q2, _ = timed(run_tokens, args.warmup)
    btok_ms, n_qb, _ = timed(run_btokens, args.warmup)
    qb_us = 1e3 * btok_ms / n_qb
    qb_alg_gbs = Q2_ALG_BYTES / qb_us / 1e3
    tok4_ms, n_q4, _ = timed(token_runner(tok4_graphs), args.warmup)
    btok4_ms, n_q4b, _ = timed(token_runner(btok4_graphs), args.warmup)
    q4_us = 1e3 * tok4_ms / n_q4
    q4b_us = 1e3 * btok4_ms / n_q4b
    tokt_ms, n_qt, _ = timed(token_runner(tokt_graphs), args.warmup)
    btokt_ms, n_qtb, _ = timed(token_runner(btokt_graphs), args.warmup)
    qt_us = 1e3 * tokt_ms / n_qt
    tokf_ms, n_gf, _ = timed(token_runner(tokf_graphs), args.warmup)
    gf_us = 1e3 * tokf_ms / n_gf
    qtb_us = 1e3 * btokt_ms / n_qtb
    gemm_us = 1e3 * gemm_ms / n_gemm
    q2_us = 1e3 * tok_ms / n_q2

    # ---- context, after the main timing: the spread of per-launch times,
    #      the 2-bit GEMV with one cache-resident matrix ("hot"), and what a
    #      plain device-to-device copy streams on this GPU.
    spreads = {
        "gemm_f32": spread([gemm_graph], gemms_per_replay),
        "gemv_q2": spread(tok_graphs, CALLS_PER_TOKEN),
        "gemv_q2_batched": spread(btok_graphs, CALLS_PER_TOKEN),
        "gemv_q4": spread(tok4_graphs, CALLS_PER_TOKEN),
        "gemv_q4_batched": spread(btok4_graphs, CALLS_PER_TOKEN),
        "gemv_q2_transposed": spread(tokt_graphs, CALLS_PER_TOKEN),
        "gemv_q2_transposed_batched": spread(btokt_graphs, CALLS_PER_TOKEN),
        "gemv_f32": spread(tokf_graphs, CALLS_PER_TOKEN),
    }
    hot_graph = capture(lambda: [bd.gemv_q2(Qd[0], Sd[0], dx, y=dy)
                                 for _ in range(CALLS_PER_TOKEN)])
    hot_ms, n_hot, _ = timed(token_runner([hot_graph] * n_tok), args.warmup)
    q2_hot_us = 1e3 * hot_ms / n_hot
    del hot_graph
    copy_bytes = 1 << 30
    with torch.cuda.stream(stream):
        csrc = torch.empty(copy_bytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        cdst = torch.empty_like(csrc)
        cdst.copy_(csrc)
        stream.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            cdst.copy_(csrc)
        e1.record(stream)
        stream.synchronize()
    copy_gbs = 2 * copy_bytes * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del csrc, cdst
    vendor = vendor_context(torch, stream, capture, timed, token_runner, n_tok, gemms_per_replay,
                            dA, dB, Wf, dxf, A, B, args)
    configs, configs_ok = gemm_configs(torch, bd, inputs, oracle, dev, stream, capture, timed,
                                       args.steps)

    gemm_tflops = GEMM_FLOPS / gemm_us / 1e6
    q2_gbs = Q2_WEIGHT_BYTES / q2_us / 1e3
    q2_alg_gbs = Q2_ALG_BYTES / q2_us / 1e3

    gemm_traffic = traffic_from_profile("traffic_gemm_f32_2048.json",
                                        src_sha("gemm_f32.hip"))
    psha = src_sha("gemv_packed.hip", "wave.hpp")
    q2_traffic = traffic_from_profile("traffic_gemv_q2_12288x1536.json", psha)
    qb_traffic = traffic_from_profile("traffic_gemv_q2_batched_12288x1536.json", psha)
    q4_traffic = traffic_from_profile("traffic_gemv_q4_12288x1536.json", psha)
    q4b_traffic = traffic_from_profile("traffic_gemv_q4_batched_12288x1536.json", psha)
    qt_traffic = traffic_from_profile("traffic_gemv_q2_1536x12288.json", psha)
    gf_traffic = traffic_from_profile("traffic_gemv_f32_12288x1536.json",
                                      src_sha("gemv_f32.hip", "wave.hpp"))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(A, B, Q0, S0, x)

    out = {
        "metric": "fp32 GEMM TFLOP/s at 2048^3; 2-bit GEMV weight GB/s at 12288x1536",
        "value": gemm_tflops if gemm_ok else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (gemm_tflops / PAGE_GEMM_2048_TFLOPS) if gemm_ok else None,
        "vs_baseline_note": ("against the page's blocked4 WebGPU kernel at 2048^3 "
                             "(9.12 ms = 1.88 TFLOP/s) on an Apple M-series laptop: "
                             "context from other hardware, not a target"),
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": ("per step: gemm_f32 2048x2048x2048 (A, B uniform[-1,1), seed 3) "
                         "+ one token of 40 gemv_q2 12288x1536 calls rotating over 128 "
                         "seeded matrices (648 MiB of codes+scales)"),
            "gemm": "2048x2048x2048 NN",
            "q2_gemv": "12288x1536, 2-bit codes + fp16 scale per 64 columns",
            "rotation": Q2_ROTATION,
            "calls_per_token": CALLS_PER_TOKEN,
            "timing": ("HIP graph replay; HIP events on the replay stream around "
                       "K whole steps, and around runs of back-to-back GEMM and "
                       "q2 launches for each kernel's average launch duration"),
        },
        "roofline": {
            "kernel": "gemm_f32 (NN, 2048^3)",
            "bound": "mfma",
            "achieved": gemm_tflops,
            "peak": PEAK_FP32_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": gemm_tflops / PEAK_FP32_MFMA_TFLOPS,
            "traffic": gemm_traffic,
            "avg_launch_us": gemm_us,
        },
        "q2_gemv": {
            "metric": "2-bit GEMV effective weight-streaming GB/s at 12288x1536 (cold rotation)",
            "value": q2_gbs if q2_ok else None,
            "unit": "GB/s",
            "codes_only_gbs": Q2_CODE_BYTES / q2_us / 1e3 if q2_ok else None,
            "avg_launch_us": q2_us,
            "roofline": {
                "kernel": "gemv_q2 (12288x1536)",
                "bound": "hbm",
                "achieved": q2_alg_gbs,
                "peak": PEAK_HBM_GBS,
                "unit": "GB/s",
                "frac": q2_alg_gbs / PEAK_HBM_GBS,
                "traffic": q2_traffic,
            },
        },
        "q2_gemv_batched": {
            "metric": ("2-bit GEMV effective weight-streaming GB/s at 12288x1536, one "
                       "token's 40 products in one gemv_q2_batched launch (cold rotation)"),
            "value": Q2_WEIGHT_BYTES / qb_us / 1e3 if qb_ok else None,
            "unit": "GB/s",
            "us_per_gemv": qb_us,
            "us_per_token": qb_us * CALLS_PER_TOKEN,
            "roofline": {
                "kernel": "gemv_q2_batched (40 x 12288x1536 per launch)",
                "bound": "hbm",
                "achieved": qb_alg_gbs,
                "peak": PEAK_HBM_GBS,
                "unit": "GB/s",
                "frac": qb_alg_gbs / PEAK_HBM_GBS,
                "traffic": (qb_traffic / CALLS_PER_TOKEN) if qb_traffic else None,
                "traffic_note": "HBM bytes per product (launch total / 40)",
            },
        },
        "q4_gemv": {
            "metric": ("4-bit GEMV effective weight-streaming GB/s at 12288x1536 "
                       "(cold rotation over 64 matrices)"),
            "value": Q4_WEIGHT_BYTES / q4_us / 1e3 if q4_ok else None,
            "unit": "GB/s",
            "avg_launch_us": q4_us,
            "roofline": {
                "kernel": "gemv_q4 (12288x1536)",
                "bound": "hbm",
                "achieved": Q4_ALG_BYTES / q4_us / 1e3,
                "peak": PEAK_HBM_GBS,
                "unit": "GB/s",
                "frac": Q4_ALG_BYTES / q4_us / 1e3 / PEAK_HBM_GBS,
                "traffic": q4_traffic,
            },
            "batched": {
                "value": Q4_WEIGHT_BYTES / q4b_us / 1e3 if q4b_ok else None,
                "unit": "GB/s",
                "us_per_gemv": q4b_us,
                "roofline": {
                    "kernel": "gemv_q4_batched (40 x 12288x1536 per launch)",
                    "bound": "hbm",
                    "achieved": Q4_ALG_BYTES / q4b_us / 1e3,
                    "peak": PEAK_HBM_GBS,
                    "unit": "GB/s",
                    "frac": Q4_ALG_BYTES / q4b_us / 1e3 / PEAK_HBM_GBS,
                    "traffic": (q4b_traffic / CALLS_PER_TOKEN) if q4b_traffic else None,
                    "traffic_note": "HBM bytes per product (launch total / 40)",
                },
            },
        },
        "q2_gemv_transposed": {
            "metric": ("2-bit GEMV effective weight-streaming GB/s at the transposed shape "
                       "1536x12288 (12,288 inputs -> 1,536 outputs), cold rotation over 128 "
                       "matrices; rows split over 256 lanes"),
            "value": Q2_WEIGHT_BYTES / qt_us / 1e3 if qt_ok else None,
            "unit": "GB/s",
            "avg_launch_us": qt_us,
            "roofline": {
                "kernel": "gemv_q2 (1536x12288)",
                "bound": "hbm",
                "achieved": QT_ALG_BYTES / qt_us / 1e3,
                "peak": PEAK_HBM_GBS,
                "unit": "GB/s",
                "frac": QT_ALG_BYTES / qt_us / 1e3 / PEAK_HBM_GBS,
                "traffic": qt_traffic,
            },
            "batched": {
                "value": Q2_WEIGHT_BYTES / qtb_us / 1e3 if qt_ok else None,
                "unit": "GB/s",
                "us_per_gemv": qtb_us,
                "frac": QT_ALG_BYTES / qtb_us / 1e3 / PEAK_HBM_GBS,
            },
        },
        "gemv_f32": {
            "metric": "fp32 GEMV GB/s at 12288x1536 (cold rotation over 48 matrices, 3.375 GiB)",
            "value": F32_ALG_BYTES / gf_us / 1e3 if gf_ok else None,
            "unit": "GB/s",
            "avg_launch_us": gf_us,
            "roofline": {
                "kernel": "gemv_f32 (12288x1536)",
                "bound": "hbm",
                "achieved": F32_ALG_BYTES / gf_us / 1e3,
                "peak": PEAK_HBM_GBS,
                "unit": "GB/s",
                "frac": F32_ALG_BYTES / gf_us / 1e3 / PEAK_HBM_GBS,
                "traffic": gf_traffic,
            },
        },
        "gemm_configs": configs,
        "spread": spreads,
        "context": {
            "q2_gemv_hot_us": q2_hot_us,
            "q2_gemv_hot_note": ("gemv_q2 12288x1536 on one matrix, 40 back-to-back calls: "
                                 "weights resident in cache, the launch-and-compute floor"),
            "hbm_copy_gbs": copy_gbs,
            "hbm_copy_note": ("torch device-to-device copy of 1 GiB, 10 times, "
                              "read + write bytes / time: what plain streaming reaches"),
            "vendor_library": vendor,
        },
        "parity": {"gemm_f32_2048": "pass" if gemm_ok else "FAIL",
                   "gemm_configs": "pass" if configs_ok else "FAIL",
                   "gemv_f32": "pass" if gf_ok else "FAIL",
                   "gemv_f32_worst_err_over_bound": gf_worst,
                   "gemv_q2_transposed": "pass" if qt_ok else "FAIL",
                   "q2_transposed_worst_err_over_bound": qt_worst,
                   "gemv_q4": "pass" if q4_ok else "FAIL",
                   "gemv_q4_batched": "pass" if q4b_ok else "FAIL",
                   "q4_worst_err_over_bound": q4_worst,
                   "q4_batched_worst_err_over_bound": q4b_worst,
                   "gemv_q2": "pass" if q2_ok else "FAIL",
                   "gemv_q2_batched": "pass" if qb_ok else "FAIL",
                   "q2_batched_worst_err_over_bound": qb_worst,
                   "gemm_worst_err_over_bound": gemm_worst,
                   "q2_worst_err_over_bound": q2_worst},
        "cpu_baseline": cpu,
        "inputs_sha256": hashes,
        "device": {"name": prop.name, "arch": getattr(prop, "gcnArchName", None),
                   "cus": prop.multi_processor_count, "torch": torch.__version__,
                   "hip": getattr(torch.version, "hip", None), "host_cpu": host_cpu(),
                   "host_cores_usable": len(os.sched_getaffinity(0))},
        "wall_s_timed": t_wall,
    }
    print(json.dumps(out), flush=True)
    return 0 if (gemm_ok and q2_ok and qb_ok and q4_ok and q4b_ok and qt_ok and gf_ok
                 and configs_ok) else 1


if __name__ == "__main__":
    sys.exit(main())
