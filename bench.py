#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X: fp32 GEMM at 2048^3 and the
2-bit GEMV at 12,288 x 1,536.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

A step is one pass of the whole path over one batch of synthetic input:
  * one gemm_f32 of two 2048 x 2048 fp32 matrices (uniform [-1, 1), seed 3),
    the largest size of the kernel sweep in "I built a GPT-2 in the browser,
    then made it 2.6x-12.1x faster" (section "The kernel sweep");
  * one token of 2-bit GEMVs: the 40 products a token runs ("Kernel 0112",
    section "What is being measured") in one gemv_q2_batched launch, product n
    using weight matrix n mod 128 of a 128-matrix set (648 MiB of codes and
    scales, far above the 256 MB Infinity Cache, as the page's "cold"
    rotation keeps reuse between runs unlikely).
Every input is generated, hashed and copied to HBM before timing, and every
product is checked against the CPU oracle first -- on every matrix of each
rotation set -- so that a failing kernel reports no speed.  Launches are
captured into HIP graphs (torch.cuda.CUDAGraph) so timed regions replay
kernels back to back, without host launch gaps.

Timing.  `ms_per_step` is K whole steps (after W warm-up steps) between two
HIP events on the replay stream.  Each kernel's launch duration comes from a
fixed window that does not depend on K: one graph of L back-to-back launches
of that kernel alone (inputs rotating as above), replayed for at least
0.1 s of warm-up and then R times with a HIP event after each replay; `mean_us`
is the window's time over its R * L launches; `median_us`, `min_us`, `max_us`,
`p10_us` and `p90_us` are taken over the per-replay means.  The rooflines use
`mean_us`.

Output: one JSON line.  `value` is the GEMM's TFLOP/s (2 * 2048^3 flops per
launch over its mean launch duration).  `q2_gemv` and `q2_gemv_batched` give
the 2-bit GEMV's weight GB/s (codes + scales per product over its duration)
for one product per launch and for a token's 40 products per launch, each
with a roofline object; `q4_gemv`, `q2_gemv_transposed` and `gemv_f32` do the
same for the 4-bit product, the transposed 1,536 x 12,288 shape (batches
also through gemv_q2_batched_ws, rows cut into slices) and the fp32 product
(single calls and a token's 40 products per gemv_f32_batched launch).  `gemm_configs` checks and times the other GEMM configurations (the
nine products of a GPT-2-small block, the 346 x 768 x 768 classifier layer,
256^3).  `cpu_baseline` times the oracle on the host, on one core and on every
usable core.  `context` holds reference points measured in the same run.  The
last key, `summary`, repeats the headline figures in a few fields.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time
from concurrent.futures import ThreadPoolExecutor

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
N_TOK = 16                                         # 16 tokens x 40 = 640 = 5 x 128
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
# blocked4 at 2048^3 took 9.12 ms on an Apple M-series laptop (WebGPU): the
# pages' own figure for this metric and workload, on other hardware.
PAGE_GEMM_2048_TFLOPS = GEMM_FLOPS / 9.12e-3 / 1e12

# Fixed timing windows: (launches per graph, timed replays).
WIN_GEMM = (25, 8)                 # 200 launches of 2048^3
WIN_SINGLE = (N_TOK * CALLS_PER_TOKEN, 4)   # 2,560 single-product launches
WIN_BATCHED = (N_TOK, 8)           # 128 launches of 40 products
WIN_CONFIG = (8, 25)               # 200 launches per GEMM configuration
WARM_S = 0.1                       # time-based warm-up before each window

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


def usable_cores():
    return len(os.sched_getaffinity(0))


def oracle_product(oracle, layout, A, B):
    """The oracle's whole product op(A).op(B) ("nn", "tn" with A stored K x M,
    "nt" with B stored N x K), its output rows split into blocks over every
    usable core (threads calling the C oracle, which runs without the GIL;
    each cell is the same plain dot product as in one call)."""
    fn = {"nn": oracle.gemm_nn, "tn": oracle.gemm_tn, "nt": oracle.gemm_nt}[layout]
    M = A.shape[1] if layout == "tn" else A.shape[0]
    blocks = [b for b in np.array_split(np.arange(M), usable_cores()) if b.size]

    def part(r):
        return fn(A[:, r[0]:r[-1] + 1] if layout == "tn" else A[r[0]:r[-1] + 1], B)
    with ThreadPoolExecutor(max_workers=len(blocks)) as pool:
        parts = list(pool.map(part, blocks))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def cpu_baseline(A, B, Q, S, x):
    """The oracle as it stands, timed on the host: the whole 2048^3 product
    (about 3.5 s on one core) and 2-bit GEMVs on one rotation matrix, first
    on one core, then with its output rows split into blocks over every
    usable core (threads calling the C oracle, which runs without the GIL)."""
    import oracle
    oracle.build(force=False)
    cores = usable_cores()
    t0 = time.perf_counter()
    oracle.gemm_nn(A, B)
    t1 = time.perf_counter() - t0
    blocks = np.array_split(np.arange(GEMM_N), cores)
    with ThreadPoolExecutor(max_workers=cores) as pool:
        t0 = time.perf_counter()
        list(pool.map(lambda r: oracle.gemm_nn(A[r[0]:r[-1] + 1], B), blocks))
        tn = time.perf_counter() - t0
        reps = 8
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.gemv_q2(Q, S, x)
        tq1 = (time.perf_counter() - t0) / reps
        t0 = time.perf_counter()
        list(pool.map(lambda _: oracle.gemv_q2(Q, S, x), range(cores * 2)))
        tqn = (time.perf_counter() - t0) / (cores * 2)
    return {
        "value": GEMM_FLOPS / tn / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": ("fp64 triple-loop oracle on the whole 2048^3 product (%.2f s on %d cores, "
                   "%.2f s on 1); 2-bit unpack-then-dot oracle on one 12288x1536 matrix "
                   "(%d calls on 1 core, %d spread over %d cores)"
                   % (tn, cores, t1, reps, cores * 2, cores)),
        "value_1core": GEMM_FLOPS / t1 / 1e12,
        "q2_gemv_weight_gbs": Q2_WEIGHT_BYTES / tqn / 1e9,
        "q2_gemv_weight_gbs_1core": Q2_WEIGHT_BYTES / tq1 / 1e9,
        "cpu": host_cpu() or platform.processor() or platform.machine(),
    }


def vendor_context(torch, stream, capture, window, dA, dB, Wf, dx):
    """The vendor library on the same inputs, for context only (never part of
    the library's path): torch.matmul in fp32 with TF32 off at 2048^3 and
    torch.mv over the fp32 GEMV rotation set, in the same fixed windows."""
    out = {"note": ("torch.matmul / torch.mv in fp32 with TF32 off on the same operands, "
                    "timed like the library's kernels: context, not part of the library")}
    try:
        torch.backends.cuda.matmul.allow_tf32 = False
        C = torch.empty_like(dA)
        with torch.cuda.stream(stream):
            torch.matmul(dA, dB, out=C)
            stream.synchronize()
        g = capture(lambda: [torch.matmul(dA, dB, out=C) for _ in range(8)])
        w = window([g], 8, 25)
        out["matmul_2048_us"] = w["mean_us"]
        out["matmul_2048_tflops"] = GEMM_FLOPS / w["mean_us"] / 1e6
        y = torch.empty(Q2_M, dtype=torch.float32, device=dA.device)
        with torch.cuda.stream(stream):
            torch.mv(Wf[0], dx, out=y)
            stream.synchronize()
        # six graphs of 40 products: 240 calls, five turns of the 48-matrix set
        gs = [capture(lambda t=t: [torch.mv(Wf[(40 * t + c) % F32_ROTATION], dx, out=y)
                                   for c in range(40)]) for t in range(6)]
        w = window(gs, 240, 4)
        out["mv_12288x1536_us"] = w["mean_us"]
        out["mv_12288x1536_gbs"] = F32_ALG_BYTES / w["mean_us"] / 1e3
    except Exception as e:   # context only: report, never fail the bench
        out["error"] = "%s: %s" % (type(e).__name__, e)
        log("vendor context skipped: %s" % out["error"])
    return out


def gemm_configs(torch, bd, inputs, oracle, dev, capture, window):
    """The GEMM configurations besides 2048^3, each checked against the oracle
    on every cell before it is timed: the nine products of a GPT-2-small
    block at 1,024 tokens (three forward, six backward; "I built a GPT-2 in
    the browser...", section "The kernel sweep", where matmul is most of
    training time), the 346 x 768 x 768 classifier layer (the 346-token
    prompt of the polyomino classifier page) and 256^3.  Each product gets a
    fixed window of back-to-back launches (the median of three interleaved
    rounds), and the block's nine products also run as one graph.  A product
    that fails parity reports no time."""
    entry = {"nn": bd.gemm_f32, "tn": bd.gemm_f32_tn, "nt": bd.gemm_f32_nt}
    t = inputs.gpt2_tensors(2)
    ops = [(name, lay, M, N, K, t[an], t[bn]) for name, lay, M, N, K, (an, bn) in inputs.GPT2_OPS]
    A346, B346 = inputs.classifier(33)
    A256, B256 = inputs.small_square(0)
    ops += [("classifier_346x768x768", "nn", 346, 768, 768, A346, B346),
            ("square_256", "nn", 256, 256, 256, A256, B256)]
    out, launches, all_ok, timing = {}, [], True, []
    for name, lay, M, N, K, A, B in ops:
        dA, dB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
        dC = torch.empty((M, N), dtype=torch.float32, device=dev)
        f = entry[lay]
        f(dA, dB, C=dC)
        C = dC.cpu().numpy()
        ref, bound = oracle_product(oracle, lay, A, B)
        ok, worst, _ = oracle.check(C, ref, bound)
        all_ok = all_ok and ok
        out[name] = {"shape": "%s %dx%dx%d" % (lay.upper(), M, N, K),
                     "parity": "pass" if ok else "FAIL", "worst_err_over_bound": worst}
        flops = 2.0 * M * N * K
        if name in {o[0] for o in inputs.GPT2_OPS}:
            launches.append((f, dA, dB, dC, flops))
        if ok:
            g = capture(lambda f=f, dA=dA, dB=dB, dC=dC: [f(dA, dB, C=dC)
                                                          for _ in range(WIN_CONFIG[0])])
            timing.append((name, g, flops))
    # Three rounds over every product, the median per product: interleaving
    # spreads slow spells of a box over all of them.
    rounds = {n: [] for n, *_ in timing}
    for _ in range(3):
        for name, g, _ in timing:
            rounds[name].append(window(g, *WIN_CONFIG, warm_s=0.02)["mean_us"])
    for name, g, flops in timing:
        d = out[name]
        d["us"] = float(np.median(rounds[name]))
        d["us_rounds"] = rounds[name]
        d["launches_per_round"] = WIN_CONFIG[0] * WIN_CONFIG[1]
        d["tflops"] = flops / d["us"] / 1e6
        d["frac_of_fp32_mfma_peak"] = d["tflops"] / PEAK_FP32_MFMA_TFLOPS
    if all_ok:
        g = capture(lambda: [f(dA, dB, C=dC) for _ in range(2)
                             for f, dA, dB, dC, _ in launches])
        w = window(g, 2, 25)          # 25 replays of two blocks
        total = sum(fl for *_, fl in launches)
        out["gpt2_block_9_products"] = {
            "us": w["mean_us"], "tflops": total / w["mean_us"] / 1e6,
            "frac_of_fp32_mfma_peak": total / w["mean_us"] / 1e6 / PEAK_FP32_MFMA_TFLOPS,
            "note": "F1..B3w back to back in one graph, 39,862,665,216 flop per block"}
    return out, all_ok


PROBE_LIB = os.path.join(ROOT, "libbench_probes.so")
PROBE_SHAPES = ((1, 64), (512, 576))     # the 2-bit GEMV's single call: 512 x 576 lanes
# (shape, independent accumulators per wave, workgroups, lanes per workgroup)
PROBE_MFMA = ((32, 1, 256, 256), (32, 1, 1024, 256), (32, 4, 1024, 256), (16, 4, 1024, 256))
PROBE_CHAINS = (("l2_1mib", 1 << 20, 100000), ("infinity_cache_64mib", 64 << 20, 100000),
                ("hbm_4gib", 4 << 30, 20000))


def probe_context(torch, dev, stream, capture, window):
    """Physics reference points from bench_probes.hip: the per-launch floor of
    an empty kernel (back to back in one graph, at the single call's launch
    shape and at one wave), the fp32 MFMA rate with no memory traffic (one
    or four independent accumulators per wave, one or four waves per SIMD),
    and the load-to-use latency of one lane chasing
    random 256-byte-spaced links through 1 MiB (L2), 64 MiB (Infinity Cache)
    and 4 GiB (HBM, translation included; the chain starts where no earlier
    run went and a 1 GiB fill evicts the caches first)."""
    import ctypes
    if not os.path.exists(PROBE_LIB):
        log("probe library not built (%s): no probe context" % PROBE_LIB)
        return None
    lib = ctypes.CDLL(PROBE_LIB)
    lib.probe_empty.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.probe_chase.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int,
                                ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_mfma.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p, ctypes.c_void_p]
    sp = ctypes.c_void_p(stream.cuda_stream)
    out = {"empty_kernel_us": {}, "mfma_tflops": {}, "load_latency_ns": {}}
    for shape, nacc, grid, block in PROBE_MFMA:
        iters = 4000 if shape == 32 else 8000
        buf = torch.empty(grid * block, dtype=torch.float32, device=dev)
        with torch.cuda.stream(stream):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            for k in range(6):   # one warm-up launch, five timed
                if k == 1:
                    e0.record(stream)
                if lib.probe_mfma(shape, nacc, grid, block, iters, ctypes.c_void_p(buf.data_ptr()),
                                  sp) != 0:
                    raise RuntimeError("probe_mfma failed")
            e1.record(stream)
            stream.synchronize()
        flops = 5 * grid * block // 64 * iters * nacc * (4096 if shape == 32 else 2048)
        key = "%dx%d_%dacc_%dx%d" % (shape, shape, nacc, grid, block)
        out["mfma_tflops"][key] = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
        del buf
    for grid, block in PROBE_SHAPES:
        def launches():
            for _ in range(WIN_SINGLE[0]):
                rc = lib.probe_empty(grid, block, sp)
                if rc != 0:
                    raise RuntimeError("probe_empty failed: %d" % rc)
        g = capture(launches)
        out["empty_kernel_us"]["%dx%d" % (grid, block)] = window(g, WIN_SINGLE[0], 2)["mean_us"]
        del g
    res = torch.zeros(64, dtype=torch.int32, device=dev)
    for name, region, links in PROBE_CHAINS:
        slots = region // 256
        n = region // 4
        gen = torch.Generator(device=dev)
        gen.manual_seed(7)
        with torch.cuda.stream(stream):
            perm = torch.randperm(slots, device=dev, generator=gen) * 64
            nxt = torch.zeros(n, dtype=torch.int32, device=dev)
            nxt[perm] = torch.roll(perm, -1).to(torch.int32)
            lo, hi = int(nxt.min().item()), int(nxt.max().item())
            if lo < 0 or hi >= n:
                raise RuntimeError("chain index out of range")
            cold = region > (256 << 20)
            start = int(perm[slots // 2].item())
            if cold:
                flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
                flush.fill_(1.0)
                del flush
            else:   # one full pass first, so the chain is resident
                if lib.probe_chase(ctypes.c_void_p(nxt.data_ptr()), n, start, slots,
                                   ctypes.c_void_p(res.data_ptr()), sp) != 0:
                    raise RuntimeError("probe_chase failed")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if lib.probe_chase(ctypes.c_void_p(nxt.data_ptr()), n, start, links,
                               ctypes.c_void_p(res.data_ptr()), sp) != 0:
                raise RuntimeError("probe_chase failed")
            e1.record(stream)
            stream.synchronize()
        out["load_latency_ns"][name] = 1e6 * e0.elapsed_time(e1) / links
        del perm, nxt
    torch.cuda.synchronize()
    log("probes: empty kernel %s us; MFMA %s TFLOP/s; load latency %s ns" % (
        ", ".join("%s %.3f" % kv for kv in out["empty_kernel_us"].items()),
        ", ".join("%s %.1f" % kv for kv in out["mfma_tflops"].items()),
        ", ".join("%s %.0f" % kv for kv in out["load_latency_ns"].items())))
    return out


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
    k = kernel.replace("(anonymous namespace)::", "")
    for prefix in ("void gg::", "gg::", "void "):
        if k.startswith(prefix):
            k = k[len(prefix):]
            break
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


# Weights per dispatch of the GEMV kernels at the bench's shapes, for counts
# per weight: (kernel-name prefix, whole name suffix, weights per dispatch).
WEIGHTS_PER_DISPATCH = (
    ("gemv_q2_idot<3,", ", 64, false>", CALLS_PER_TOKEN * Q2_M * Q2_K),
    ("gemv_q2_idot<3,", ", 64, true>", CALLS_PER_TOKEN * QT_M * QT_K),
    ("gemv_packed_flat<2, 1, 1,", "", Q2_M * Q2_K),
    ("gemv_packed_flat<4, 2, 1,", "", Q2_M * Q2_K),
    ("gemv_packed_flat<4, 8, 64,", "", CALLS_PER_TOKEN * Q2_M * Q2_K),
    ("gemv_f32_kernel<1, 6, true, 1>", "", Q2_M * Q2_K),
    ("gemv_f32_kernel<1, 6, true, 64>", "", CALLS_PER_TOKEN * Q2_M * Q2_K),
)
N_SIMD = 1024                      # 256 CUs x 4 SIMDs
N_XCD = 8                          # GRBM_GUI_ACTIVE is summed over the 8 XCDs


def summarize_counters(db_paths):
    """Per kernel (and launch shape): the median per dispatch of every counter
    found in the rocprofv3 --pmc databases, then derived figures: VALU
    instructions per lane per weight (SQ_INSTS_VALU * 64 / weights), VALU
    issue share 4 * SQ_ACTIVE_INST_VALU / (SIMDs * GRBM_GUI_ACTIVE / XCDs),
    MFMA utilisation SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs * GRBM_GUI_ACTIVE /
    XCDs), LDS bank-conflict cycles per LDS instruction and the L2 hit rate."""
    import sqlite3
    med = {}
    for path in db_paths:
        db = sqlite3.connect(path)
        names = [r[0] for r in db.execute(
            "select distinct counter_name from counters_collection").fetchall()]
        db.close()
        for c in names:
            for k, v in _median_per_kernel(_counter_dispatches(path, c)).items():
                med.setdefault(k, {})[c] = v
    lines = []
    counters = sorted({c for d in med.values() for c in d})
    lines.append("| kernel | " + " | ".join(counters) + " |")
    lines.append("|---" * (len(counters) + 1) + "|")
    for k in sorted(med):
        lines.append("| %s | " % k + " | ".join(
            "%.0f" % med[k][c] if c in med[k] else "" for c in counters) + " |")
    lines.append("")
    lines.append("| kernel | VALU instr per lane per weight | VALU issue share | MFMA util | "
                 "LDS conflict cycles per LDS instr | L2 hit rate |")
    lines.append("|---|---|---|---|---|---|")
    for k in sorted(med):
        d = med[k]
        base = k.split(" @")[0]
        wts = [w for pre, suf, w in WEIGHTS_PER_DISPATCH
               if base.startswith(pre) and base.endswith(suf)]
        cyc = d.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD

        def f(v, fmt):
            return fmt % v if v is not None else ""
        vpw = d["SQ_INSTS_VALU"] * 64.0 / wts[0] if wts and "SQ_INSTS_VALU" in d else None
        busy = (4.0 * d["SQ_ACTIVE_INST_VALU"] / (N_SIMD * cyc)
                if cyc and "SQ_ACTIVE_INST_VALU" in d else None)
        mfma = (d["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * cyc)
                if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in d else None)
        lds = (d["SQ_LDS_BANK_CONFLICT"] / d["SQ_INSTS_LDS"]
               if d.get("SQ_INSTS_LDS") and "SQ_LDS_BANK_CONFLICT" in d else None)
        hits = (d["TCC_HIT_sum"] / (d["TCC_HIT_sum"] + d["TCC_MISS_sum"])
                if "TCC_HIT_sum" in d and d.get("TCC_HIT_sum", 0) + d.get("TCC_MISS_sum", 0)
                else None)
        if any(v is not None for v in (vpw, busy, mfma, lds, hits)):
            lines.append("| %s | %s | %s | %s | %s | %s |" % (
                k, f(vpw, "%.3f"), f(busy, "%.2f"), f(mfma, "%.2f"), f(lds, "%.2f"),
                f(hits, "%.3f")))
    return "\n".join(lines)


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
            (lambda n: n.startswith("gemv_q2_idot<3,") and n.split(" @")[0].endswith(", 64, false>"),
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
            (lambda n: n.startswith("gemv_f32_kernel<1, 6, true, 1>"),
             "traffic_gemv_f32_12288x1536.json", ("gemv_f32.hip", "wave.hpp"), F32_ALG_BYTES),
            (lambda n: n.startswith("gemv_f32_kernel<1, 6, true, 64>"),
             "traffic_gemv_f32_batched_12288x1536.json", ("gemv_f32.hip", "wave.hpp"),
             CALLS_PER_TOKEN * F32_ALG_BYTES),
            (lambda n: n.startswith("gemv_q2_idot<3,") and n.split(" @")[0].endswith(", 64, true>"),
             "traffic_gemv_q2_sliced_1536x12288.json", q2_srcs, CALLS_PER_TOKEN * QT_ALG_BYTES),
            (lambda n: n.startswith("gemv_slices_sum<64>"),
             "traffic_gemv_slices_sum_1536x12288.json", q2_srcs, CALLS_PER_TOKEN * QT_M * 4)):
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


def roofline(kernel, alg_bytes, us, traffic=None, note=None):
    achieved = alg_bytes / us / 1e3
    d = {"kernel": kernel, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
         "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": traffic}
    if note:
        d["traffic_note"] = note
    return d


def counters_run(torch, bd, inputs):
    """Each kernel of the path on the bench's inputs, a few launches each,
    eagerly, after one device-to-device copy of CALIBRATION_BYTES (the
    reference that scales rocprofv3's byte counters): 5 GEMMs at 2048^3, 128
    single 2-bit products and 4 batches of 40 over the 128-matrix set, the
    same for 4-bit over its 64 matrices, the transposed 1,536 x 12,288 2-bit
    products over its 128-matrix set one by one and in 4 batches of 40
    through gemv_q2_batched_ws (rows cut into slices), and 48 fp32 GEMVs and 4 batches of 40
    of them."""
    dev = torch.device("cuda:0")
    A, B = inputs.large_square(3)
    dA, dB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    dC = torch.empty((GEMM_N, GEMM_N), dtype=torch.float32, device=dev)
    dx = torch.from_numpy(inputs.q2_x()).to(dev)

    def packed_set(gen, n, M=Q2_M, K=Q2_K):
        out = []
        for r in range(n):
            Q, S = gen(r, M, K)
            out.append((torch.from_numpy(Q).to(dev), torch.from_numpy(S.view(np.int16)).to(dev)))
        return out
    q2, q4 = packed_set(inputs.q2_weight, Q2_ROTATION), packed_set(inputs.q4_weight, Q4_ROTATION)
    qt = packed_set(inputs.q2_weight, Q2_ROTATION, QT_M, QT_K)
    dxt = torch.from_numpy(inputs.q2_x(QT_K)).to(dev)
    dyts = [torch.empty(QT_M, dtype=torch.float32, device=dev) for _ in range(CALLS_PER_TOKEN)]
    wst = torch.empty(bd.gemv_q2_batched_ws_size(CALLS_PER_TOKEN, QT_M, QT_K), dtype=torch.uint8,
                      device=dev)
    Wf = [torch.from_numpy(inputs.gemv_f32_weight(r)).to(dev) for r in range(F32_ROTATION)]
    dxf = torch.from_numpy(inputs.gemv_f32_x()).to(dev)
    dy = torch.empty(Q2_M, dtype=torch.float32, device=dev)
    dys = [torch.empty(Q2_M, dtype=torch.float32, device=dev) for _ in range(CALLS_PER_TOKEN)]
    src = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    for _ in range(5):
        bd.gemm_f32(dA, dB, C=dC)
    for pset, rot, single, batched in ((q2, Q2_ROTATION, bd.gemv_q2, bd.gemv_q2_batched),
                                       (q4, Q4_ROTATION, bd.gemv_q4, bd.gemv_q4_batched)):
        for Q, S in pset:
            single(Q, S, dx, y=dy)
        for t in range(4):
            idx = [(t * CALLS_PER_TOKEN + c) % rot for c in range(CALLS_PER_TOKEN)]
            batched([pset[i][0] for i in idx], [pset[i][1] for i in idx],
                    [dx] * CALLS_PER_TOKEN, ys=dys)
    for Q, S in qt:
        bd.gemv_q2(Q, S, dxt, y=dyts[0])
    for t in range(4):
        idx = [(t * CALLS_PER_TOKEN + c) % Q2_ROTATION for c in range(CALLS_PER_TOKEN)]
        bd.gemv_q2_batched_ws([qt[i][0] for i in idx], [qt[i][1] for i in idx],
                              [dxt] * CALLS_PER_TOKEN, ys=dyts, workspace=wst)
    for W in Wf:
        bd.gemv_f32(W, dxf, y=dy)
    for t in range(4):
        idx = [(t * CALLS_PER_TOKEN + c) % F32_ROTATION for c in range(CALLS_PER_TOKEN)]
        bd.gemv_f32_batched([Wf[i] for i in idx], [dxf] * CALLS_PER_TOKEN, ys=dys)
    torch.cuda.synchronize()
    log("counters run done")
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
    ap.add_argument("--counters-run", action="store_true",
                    help="only launch each kernel of the path a few times on the bench's "
                         "inputs (for rocprofv3 --pmc passes, which serialise dispatches), "
                         "with the calibration copy, and exit")
    ap.add_argument("--summarize-trace", metavar="RESULTS_DB",
                    help="print the per-kernel summary of a rocprofv3 "
                         "--kernel-trace --stats database and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_DB",
                    help="print per-kernel medians of the counters in rocprofv3 --pmc "
                         "databases, with derived figures, and exit")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="turn two rocprofv3 --pmc databases (FETCH_SIZE, "
                         "WRITE_SIZE) of a run made with --copy-calibration "
                         "into per-launch HBM bytes under profiles/, and exit")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return 0
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters))
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
    if args.counters_run:
        return counters_run(torch, bd, inputs)
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

    def packed_set(gen, n, M=Q2_M, K=Q2_K):
        Qd, Sd, h = [], [], hashlib.sha256()
        for r in range(n):
            Q, S = gen(r, M, K)
            h.update(Q.tobytes())
            h.update(S.tobytes())
            Qd.append(torch.from_numpy(Q).to(dev))
            Sd.append(torch.from_numpy(S.view(np.int16)).to(dev))
        return Qd, Sd, h.hexdigest()[:16]

    Qd, Sd, hq = packed_set(inputs.q2_weight, Q2_ROTATION)
    Q4d, S4d, h4 = packed_set(inputs.q4_weight, Q4_ROTATION)
    QTd, STd, ht = packed_set(inputs.q2_weight, Q2_ROTATION, QT_M, QT_K)
    xt = inputs.q2_x(QT_K)
    dxt = torch.from_numpy(xt).to(dev)
    # fp32 GEMV: 48 matrices of 12,288 x 1,536 (3.375 GiB), drawn on a few
    # host threads, uploaded one by one
    with ThreadPoolExecutor(max_workers=min(8, usable_cores())) as pool:
        Wf = [torch.from_numpy(W).to(dev)
              for W in pool.map(inputs.gemv_f32_weight, range(F32_ROTATION))]
    xf = inputs.gemv_f32_x()
    dxf = torch.from_numpy(xf).to(dev)
    dy = torch.empty(Q2_M, dtype=torch.float32, device=dev)
    dyt = torch.empty(QT_M, dtype=torch.float32, device=dev)
    dys = [torch.empty(Q2_M, dtype=torch.float32, device=dev) for _ in range(CALLS_PER_TOKEN)]
    dyts = [torch.empty(QT_M, dtype=torch.float32, device=dev) for _ in range(CALLS_PER_TOKEN)]
    # the workspace of the transposed shape's sliced batches (64 products)
    wst = torch.empty(bd.gemv_q2_batched_ws_size(64, QT_M, QT_K), dtype=torch.uint8, device=dev)

    def q2_ws(Qs, Ss, xs, ys=None, stream=None):
        return bd.gemv_q2_batched_ws(Qs, Ss, xs, ys=ys, workspace=wst, stream=stream)
    torch.cuda.synchronize()
    hashes = {"gemm_A_B": inputs.sha256(A, B)[:16], "q2_x": inputs.sha256(x)[:16],
              "q2_set": hq, "q4_set": h4, "q2_transposed_set": ht,
              "q2_transposed_x": inputs.sha256(xt)[:16], "gemv_f32_x": inputs.sha256(xf)[:16]}
    log("inputs ready in %.1f s" % (time.perf_counter() - t0))

    # ---- parity first, on every matrix of every rotation set: a wrong
    #      kernel reports no speed
    import oracle
    t0 = time.perf_counter()
    bd.gemm_f32(dA, dB, C=dC)
    C = dC.cpu().numpy()
    ref, bound = oracle_product(oracle, "nn", A, B)
    gemm_ok, gemm_worst, _ = oracle.check(C, ref, bound)
    del C, ref, bound

    def packed_outputs(single, batched, Qs, Ss, xv, M):
        """Each matrix of a set through the single-product entry point and
        through batched launches of 64; both results on the host."""
        n = len(Qs)
        out_s = torch.empty((n, M), dtype=torch.float32, device=dev)
        out_b = torch.empty((n, M), dtype=torch.float32, device=dev)
        for r in range(n):
            single(Qs[r], Ss[r], xv, y=out_s[r])
        for b0 in range(0, n, 64):
            idx = range(b0, min(n, b0 + 64))
            batched([Qs[r] for r in idx], [Ss[r] for r in idx], [xv] * len(idx),
                    ys=[out_b[r] for r in idx])
        return out_s.cpu().numpy(), out_b.cpu().numpy()

    q2s, q2b = packed_outputs(bd.gemv_q2, bd.gemv_q2_batched, Qd, Sd, dx, Q2_M)

    def q2_ref(r):
        Q, S = inputs.q2_weight(r)
        return oracle.gemv_q2(Q, S, x)
    with ThreadPoolExecutor(max_workers=usable_cores()) as pool:
        q2_refs = list(pool.map(q2_ref, range(Q2_ROTATION)))

    def check_set(outs, refs, what):
        ok, worst = True, 0.0
        for r, (ref_r, bound_r) in enumerate(refs):
            good, w, idx = oracle.check(outs[r], ref_r, bound_r)
            if not good:
                log("parity FAIL: %s matrix %d at %s" % (what, r, idx))
            ok, worst = ok and good, max(worst, w)
        return ok, worst
    q2_ok, q2_worst = check_set(q2s, q2_refs, "gemv_q2")
    qb_ok, qb_worst = check_set(q2b, q2_refs, "gemv_q2_batched")
    del q2_refs

    q4s, q4b = packed_outputs(bd.gemv_q4, bd.gemv_q4_batched, Q4d, S4d, dx, Q2_M)

    def q4_ref(r):
        Q, S = inputs.q4_weight(r)
        return oracle.gemv_q4(Q, S, x)
    with ThreadPoolExecutor(max_workers=usable_cores()) as pool:
        q4_refs = list(pool.map(q4_ref, range(Q4_ROTATION)))
    q4_ok, q4_worst = check_set(q4s, q4_refs, "gemv_q4")
    q4b_ok, q4b_worst = check_set(q4b, q4_refs, "gemv_q4_batched")
    del q4_refs

    qts, qtb = packed_outputs(bd.gemv_q2, bd.gemv_q2_batched, QTd, STd, dxt, QT_M)
    _, qtw = packed_outputs(bd.gemv_q2, q2_ws, QTd, STd, dxt, QT_M)

    def qt_ref(r):
        Q, S = inputs.q2_weight(r, QT_M, QT_K)
        return oracle.gemv_q2(Q, S, xt)
    with ThreadPoolExecutor(max_workers=usable_cores()) as pool:
        qt_refs = list(pool.map(qt_ref, range(Q2_ROTATION)))
    qt_ok, qt_worst = check_set(qts, qt_refs, "gemv_q2 1536x12288")
    qtb_ok, qtb_worst = check_set(qtb, qt_refs, "gemv_q2_batched 1536x12288")
    qtw_ok, qtw_worst = check_set(qtw, qt_refs, "gemv_q2_batched_ws 1536x12288")
    del qt_refs

    gf = torch.empty((F32_ROTATION, Q2_M), dtype=torch.float32, device=dev)
    gfb = torch.full((F32_ROTATION, Q2_M), float("nan"), dtype=torch.float32, device=dev)
    for r in range(F32_ROTATION):
        bd.gemv_f32(Wf[r], dxf, y=gf[r])
    for b0 in range(0, F32_ROTATION, CALLS_PER_TOKEN):
        idx = range(b0, min(F32_ROTATION, b0 + CALLS_PER_TOKEN))
        bd.gemv_f32_batched([Wf[r] for r in idx], [dxf] * len(idx), ys=[gfb[r] for r in idx])
    gf, gfb = gf.cpu().numpy(), gfb.cpu().numpy()
    # each batched product runs the single call's arithmetic: equal bit for bit
    gfb_ok = bool(np.array_equal(gfb, gf))
    if not gfb_ok:
        log("parity FAIL: gemv_f32_batched differs from gemv_f32")
    with ThreadPoolExecutor(max_workers=usable_cores()) as pool:
        gf_refs = list(pool.map(lambda r: oracle.gemv(inputs.gemv_f32_weight(r), xf),
                                range(F32_ROTATION)))
    gf_ok, gf_worst = check_set(gf, gf_refs, "gemv_f32")
    gfb_ok = gfb_ok and gf_ok
    del gf_refs
    parity = {
        "gemm_f32_2048": "pass" if gemm_ok else "FAIL", "gemm_worst_err_over_bound": gemm_worst,
        "gemv_q2": "pass" if q2_ok else "FAIL", "gemv_q2_worst": q2_worst,
        "gemv_q2_batched": "pass" if qb_ok else "FAIL", "gemv_q2_batched_worst": qb_worst,
        "gemv_q4": "pass" if q4_ok else "FAIL", "gemv_q4_worst": q4_worst,
        "gemv_q4_batched": "pass" if q4b_ok else "FAIL", "gemv_q4_batched_worst": q4b_worst,
        "gemv_q2_transposed": "pass" if qt_ok else "FAIL", "gemv_q2_transposed_worst": qt_worst,
        "gemv_q2_transposed_batched": "pass" if qtb_ok else "FAIL",
        "gemv_q2_transposed_batched_worst": qtb_worst,
        "gemv_q2_transposed_batched_ws": "pass" if qtw_ok else "FAIL",
        "gemv_q2_transposed_batched_ws_worst": qtw_worst,
        "gemv_f32": "pass" if gf_ok else "FAIL", "gemv_f32_worst": gf_worst,
        "gemv_f32_batched": "pass" if gfb_ok else "FAIL",
        "note": ("worst |gpu - oracle| / sum|a*b| per element (bound 1e-4); the packed and "
                 "fp32 GEMVs on every matrix of their rotation sets, through the single and "
                 "the batched entry points (the fp32 batch must also equal the single calls "
                 "bit for bit); the 2048^3 GEMM and the other GEMM configurations on every cell"),
    }
    log("parity in %.1f s: gemm %.3g, q2 %.3g, q2 batched %.3g, q4 %.3g, q4 batched %.3g, "
        "q2 transposed %.3g / %.3g, gemv_f32 %.3g (x 1e-4 bound)" %
        (time.perf_counter() - t0, gemm_worst / 1e-4, q2_worst / 1e-4, qb_worst / 1e-4,
         q4_worst / 1e-4, q4b_worst / 1e-4, qt_worst / 1e-4, qtb_worst / 1e-4,
         gf_worst / 1e-4))
    del q2s, q2b, q4s, q4b, qts, qtb, qtw, gf, gfb

    if args.copy_calibration > 0:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: %d bytes" % (4 * n))
        del src, dst

    # ---- graphs
    stream = torch.cuda.Stream(device=dev)

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        return g

    def window(graph, launches, replays, warm_s=WARM_S):
        """A fixed window: `replays` replays of `graph` (a graph, or a list of
        graphs replayed in turn, holding `launches` back-to-back launches in
        all) after `warm_s` seconds of warm-up replays, a HIP event on the
        replay stream after each replay."""
        graphs = graph if isinstance(graph, list) else [graph]

        def replay():
            for g in graphs:
                g.replay()
        with torch.cuda.stream(stream):
            t0 = time.perf_counter()
            while True:
                for _ in range(2):
                    replay()
                stream.synchronize()
                if time.perf_counter() - t0 >= warm_s:
                    break
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
            ev[0].record(stream)
            for k in range(replays):
                replay()
                ev[k + 1].record(stream)
            stream.synchronize()
        per = sorted(1e3 * ev[k].elapsed_time(ev[k + 1]) / launches for k in range(replays))
        total_us = 1e3 * ev[0].elapsed_time(ev[-1])
        return {"mean_us": total_us / (launches * replays),
                "median_us": per[len(per) // 2] if replays % 2 else
                0.5 * (per[replays // 2 - 1] + per[replays // 2]),
                "min_us": per[0], "max_us": per[-1],
                "p10_us": float(np.percentile(per, 10)), "p90_us": float(np.percentile(per, 90)),
                "launches": launches * replays,
                "launches_per_replay": launches, "replays": replays, "warmup_s": warm_s}

    def tok_idx(t, rot):
        return [(t * CALLS_PER_TOKEN + c) % rot for c in range(CALLS_PER_TOKEN)]

    def singles(fn, Qs, Ss, xv, y, rot):
        return lambda: [fn(Qs[n % rot], Ss[n % rot], xv, y=y) for n in range(WIN_SINGLE[0])]

    def batches(fn, Qs, Ss, xv, ys, rot):
        def run():
            for t in range(N_TOK):
                idx = tok_idx(t, rot)
                fn([Qs[i] for i in idx], [Ss[i] for i in idx], [xv] * CALLS_PER_TOKEN, ys=ys)
        return run

    with torch.cuda.stream(stream):
        for _ in range(3):
            bd.gemm_f32(dA, dB, C=dC)
            batches(bd.gemv_q2_batched, Qd, Sd, dx, dys, Q2_ROTATION)()
    stream.synchronize()

    # whole steps: the GEMM, then token t's 40 products in one launch
    step_graphs = []
    for t in range(N_TOK):
        idx = tok_idx(t, Q2_ROTATION)
        step_graphs.append(capture(lambda idx=idx: (
            bd.gemm_f32(dA, dB, C=dC),
            bd.gemv_q2_batched([Qd[i] for i in idx], [Sd[i] for i in idx],
                               [dx] * CALLS_PER_TOKEN, ys=dys))))
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step_graphs[i % N_TOK].replay()
        stream.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        t_wall = time.perf_counter()
        for s in range(args.steps):
            step_graphs[(args.warmup + s) % N_TOK].replay()
        e1.record(stream)
        stream.synchronize()
        t_wall = time.perf_counter() - t_wall
    total_ms = e0.elapsed_time(e1)
    del step_graphs

    # per-kernel windows
    win = {}
    g = capture(lambda: [bd.gemm_f32(dA, dB, C=dC) for _ in range(WIN_GEMM[0])])
    win["gemm_f32"] = window(g, *WIN_GEMM)
    del g
    for name, mk, gw in (
            ("gemv_q2_batched", batches(bd.gemv_q2_batched, Qd, Sd, dx, dys, Q2_ROTATION),
             WIN_BATCHED),
            ("gemv_q2", singles(bd.gemv_q2, Qd, Sd, dx, dy, Q2_ROTATION), WIN_SINGLE),
            ("gemv_q4_batched", batches(bd.gemv_q4_batched, Q4d, S4d, dx, dys, Q4_ROTATION),
             WIN_BATCHED),
            ("gemv_q4", singles(bd.gemv_q4, Q4d, S4d, dx, dy, Q4_ROTATION), WIN_SINGLE),
            ("gemv_q2_transposed_batched",
             batches(bd.gemv_q2_batched, QTd, STd, dxt, dyts, Q2_ROTATION), WIN_BATCHED),
            ("gemv_q2_transposed", singles(bd.gemv_q2, QTd, STd, dxt, dyt, Q2_ROTATION),
             WIN_SINGLE),
            ("gemv_q2_transposed_batched_ws",
             batches(q2_ws, QTd, STd, dxt, dyts, Q2_ROTATION), WIN_BATCHED),
            ("gemv_f32", lambda: [bd.gemv_f32(Wf[n % F32_ROTATION], dxf, y=dy)
                                  for n in range(WIN_SINGLE[0])], WIN_SINGLE),
            ("gemv_f32_batched",
             lambda: [bd.gemv_f32_batched([Wf[i] for i in tok_idx(t, F32_ROTATION)],
                                          [dxf] * CALLS_PER_TOKEN, ys=dys)
                      for t in range(N_TOK)], WIN_BATCHED)):
        g = capture(mk)
        win[name] = window(g, *gw)
        del g
        log("%-28s mean %.3f us, median %.3f us per launch" %
            (name, win[name]["mean_us"], win[name]["median_us"]))
    per_product = {k: (win[k]["mean_us"] / CALLS_PER_TOKEN if "_batched" in k
                       else win[k]["mean_us"]) for k in win}

    # ---- context, after the main timing
    #  * the 2-bit GEMV on one cache-resident matrix ("hot");
    #  * a near-empty kernel back to back: the per-launch floor of the queue;
    #  * what a plain device-to-device copy streams.
    g = capture(lambda: [bd.gemv_q2(Qd[0], Sd[0], dx, y=dy) for _ in range(WIN_SINGLE[0])])
    q2_hot_us = window(g, WIN_SINGLE[0], 2)["mean_us"]
    small = torch.zeros(256 * 256, dtype=torch.float32, device=dev)
    g = capture(lambda: [small.fill_(1.0) for _ in range(WIN_SINGLE[0])])
    floor_us = window(g, WIN_SINGLE[0], 2)["mean_us"]
    del g, small
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
    probes = probe_context(torch, dev, stream, capture, window)
    vendor = vendor_context(torch, stream, capture, window, dA, dB, Wf, dxf)
    torch.cuda.synchronize()
    configs, configs_ok = gemm_configs(torch, bd, inputs, oracle, dev, capture, window)

    gemm_us = win["gemm_f32"]["mean_us"]
    gemm_tflops = GEMM_FLOPS / gemm_us / 1e6
    psha = src_sha("gemv_packed.hip", "wave.hpp")
    gemm_traffic = traffic_from_profile("traffic_gemm_f32_2048.json", src_sha("gemm_f32.hip"))
    q2_traffic = traffic_from_profile("traffic_gemv_q2_12288x1536.json", psha)
    qb_traffic = traffic_from_profile("traffic_gemv_q2_batched_12288x1536.json", psha)
    q4_traffic = traffic_from_profile("traffic_gemv_q4_12288x1536.json", psha)
    q4b_traffic = traffic_from_profile("traffic_gemv_q4_batched_12288x1536.json", psha)
    qt_traffic = traffic_from_profile("traffic_gemv_q2_1536x12288.json", psha)
    qtw_traffic = traffic_from_profile("traffic_gemv_q2_sliced_1536x12288.json", psha)
    qts_traffic = traffic_from_profile("traffic_gemv_slices_sum_1536x12288.json", psha)
    gf_traffic = traffic_from_profile("traffic_gemv_f32_12288x1536.json",
                                      src_sha("gemv_f32.hip", "wave.hpp"))
    gfb_traffic = traffic_from_profile("traffic_gemv_f32_batched_12288x1536.json",
                                       src_sha("gemv_f32.hip", "wave.hpp"))
    per_prod_note = "HBM bytes per product (launch total / 40)"

    cpu = None
    if not args.no_cpu_baseline:
        Q0, S0 = inputs.q2_weight(0)
        cpu = cpu_baseline(A, B, Q0, S0, x)

    all_ok = (gemm_ok and q2_ok and qb_ok and q4_ok and q4b_ok and qt_ok and qtb_ok and qtw_ok
              and gf_ok and gfb_ok and configs_ok)
    qb_us, q2_us = per_product["gemv_q2_batched"], per_product["gemv_q2"]
    q4b_us, q4_us = per_product["gemv_q4_batched"], per_product["gemv_q4"]
    qtb_us, qt_us = per_product["gemv_q2_transposed_batched"], per_product["gemv_q2_transposed"]
    qtw_us = per_product["gemv_q2_transposed_batched_ws"]
    gf_us, gfb_us = per_product["gemv_f32"], per_product["gemv_f32_batched"]
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
        "vs_baseline_note": ("the pages' own figure for this metric and workload: the blocked4 "
                             "WebGPU kernel at 2048^3 (9.12 ms = 1.88 TFLOP/s) on an Apple "
                             "M-series laptop -- other hardware, context and not a target; "
                             "vs_cpu_baseline is the ratio to the oracle timed here"),
        "vs_cpu_baseline": (gemm_tflops / cpu["value"]) if (gemm_ok and cpu) else None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": ("per step: gemm_f32 2048x2048x2048 (A, B uniform[-1,1), seed 3) "
                         "+ one token of 40 2-bit 12288x1536 products in one gemv_q2_batched "
                         "launch, rotating over 128 seeded matrices (648 MiB of codes+scales)"),
            "gemm": "2048x2048x2048 NN",
            "q2_gemv": "12288x1536, 2-bit codes + fp16 scale per 64 columns",
            "rotation": Q2_ROTATION,
            "calls_per_token": CALLS_PER_TOKEN,
            "timing": ("HIP graph replay; ms_per_step: HIP events around K whole steps; each "
                       "kernel: a fixed window of back-to-back launches (launches per graph x "
                       "replays, after %.1f s of warm-up), mean over the window" % WARM_S),
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
            "median_launch_us": win["gemm_f32"]["median_us"],
            "launches": win["gemm_f32"]["launches"],
        },
        "q2_gemv_batched": {
            "metric": ("2-bit GEMV effective weight-streaming GB/s at 12288x1536, one "
                       "token's 40 products in one gemv_q2_batched launch (cold rotation)"),
            "value": Q2_WEIGHT_BYTES / qb_us / 1e3 if qb_ok else None,
            "unit": "GB/s",
            "codes_only_gbs": Q2_CODE_BYTES / qb_us / 1e3,
            "us_per_gemv": qb_us,
            "us_per_token": win["gemv_q2_batched"]["mean_us"],
            "roofline": roofline("gemv_q2_batched (40 x 12288x1536 per launch)", Q2_ALG_BYTES,
                                 qb_us, qb_traffic / CALLS_PER_TOKEN if qb_traffic else None,
                                 per_prod_note),
        },
        "q2_gemv": {
            "metric": "2-bit GEMV effective weight-streaming GB/s at 12288x1536 (cold rotation)",
            "value": Q2_WEIGHT_BYTES / q2_us / 1e3 if q2_ok else None,
            "unit": "GB/s",
            "codes_only_gbs": Q2_CODE_BYTES / q2_us / 1e3,
            "avg_launch_us": q2_us,
            "roofline": roofline("gemv_q2 (12288x1536)", Q2_ALG_BYTES, q2_us, q2_traffic),
        },
        "q4_gemv": {
            "metric": ("4-bit GEMV effective weight-streaming GB/s at 12288x1536 "
                       "(cold rotation over 64 matrices)"),
            "value": Q4_WEIGHT_BYTES / q4_us / 1e3 if q4_ok else None,
            "unit": "GB/s",
            "avg_launch_us": q4_us,
            "roofline": roofline("gemv_q4 (12288x1536)", Q4_ALG_BYTES, q4_us, q4_traffic),
            "batched": {
                "value": Q4_WEIGHT_BYTES / q4b_us / 1e3 if q4b_ok else None,
                "unit": "GB/s",
                "us_per_gemv": q4b_us,
                "roofline": roofline("gemv_q4_batched (40 x 12288x1536 per launch)",
                                     Q4_ALG_BYTES, q4b_us,
                                     q4b_traffic / CALLS_PER_TOKEN if q4b_traffic else None,
                                     per_prod_note),
            },
        },
        "q2_gemv_transposed": {
            "metric": ("2-bit GEMV effective weight-streaming GB/s at the transposed shape "
                       "1536x12288 (12,288 inputs -> 1,536 outputs), cold rotation over 128 "
                       "matrices; rows split over 256 lanes"),
            "value": Q2_WEIGHT_BYTES / qt_us / 1e3 if qt_ok else None,
            "unit": "GB/s",
            "avg_launch_us": qt_us,
            "roofline": roofline("gemv_q2 (1536x12288)", QT_ALG_BYTES, qt_us, qt_traffic),
            "batched": {
                "value": Q2_WEIGHT_BYTES / qtb_us / 1e3 if qtb_ok else None,
                "unit": "GB/s",
                "us_per_gemv": qtb_us,
                "frac": QT_ALG_BYTES / qtb_us / 1e3 / PEAK_HBM_GBS,
            },
            "batched_ws": {
                "metric": ("the same, a token's 40 products per gemv_q2_batched_ws launch: "
                           "rows cut into 8 slices of 1,536 columns, partial sums in a "
                           "workspace, added by a second kernel (both timed)"),
                "value": Q2_WEIGHT_BYTES / qtw_us / 1e3 if qtw_ok else None,
                "unit": "GB/s",
                "us_per_gemv": qtw_us,
                "frac": QT_ALG_BYTES / qtw_us / 1e3 / PEAK_HBM_GBS,
                "roofline": roofline(
                    "gemv_q2_idot sliced + gemv_slices_sum (40 x 1536x12288 per launch pair)",
                    QT_ALG_BYTES, qtw_us,
                    (qtw_traffic + qts_traffic) / CALLS_PER_TOKEN
                    if qtw_traffic and qts_traffic else None,
                    per_prod_note + "; both kernels, the partial sums included"),
            },
        },
        "gemv_f32": {
            "metric": "fp32 GEMV GB/s at 12288x1536 (cold rotation over 48 matrices, 3.375 GiB)",
            "value": F32_ALG_BYTES / gf_us / 1e3 if gf_ok else None,
            "unit": "GB/s",
            "avg_launch_us": gf_us,
            "roofline": roofline("gemv_f32 (12288x1536)", F32_ALG_BYTES, gf_us, gf_traffic),
            "batched": {
                "metric": ("the same, one token's 40 products in one gemv_f32_batched launch"),
                "value": F32_ALG_BYTES / gfb_us / 1e3 if gfb_ok else None,
                "unit": "GB/s",
                "us_per_gemv": gfb_us,
                "us_per_token": win["gemv_f32_batched"]["mean_us"],
                "roofline": roofline("gemv_f32_batched (40 x 12288x1536 per launch)",
                                     F32_ALG_BYTES, gfb_us,
                                     gfb_traffic / CALLS_PER_TOKEN if gfb_traffic else None,
                                     per_prod_note),
            },
        },
        "windows": win,
        "gemm_configs": configs,
        "context": {
            "q2_gemv_hot_us": q2_hot_us,
            "q2_gemv_hot_note": ("gemv_q2 12288x1536 on one matrix, back to back: weights "
                                 "resident in cache, the launch-and-compute floor"),
            "launch_floor_us": floor_us,
            "launch_floor_note": ("a fill of 256 KiB (a near-empty kernel) back to back in "
                                  "one graph: the queue's per-launch floor"),
            "probes": probes,
            "probes_note": ("bench_probes.hip: empty_kernel_us is an empty kernel back to back "
                            "in one graph at grid x workgroup lanes (512x576 is the 2-bit "
                            "GEMV's single call); mfma_tflops is back-to-back fp32 MFMAs of "
                            "that shape with that many independent accumulators per wave on "
                            "workgroups x lanes; load_latency_ns is one lane chasing random "
                            "links through a region of that size"),
            "hbm_copy_gbs": copy_gbs,
            "hbm_copy_note": ("torch device-to-device copy of 1 GiB, 10 times, "
                              "read + write bytes / time: what plain streaming reaches"),
            "vendor_library": vendor,
        },
        "parity": parity,
        "cpu_baseline": cpu,
        "inputs_sha256": hashes,
        "device": {"name": prop.name, "arch": getattr(prop, "gcnArchName", None),
                   "cus": prop.multi_processor_count, "torch": torch.__version__,
                   "hip": getattr(torch.version, "hip", None), "host_cpu": host_cpu(),
                   "host_cores_usable": usable_cores()},
        "wall_s_timed": t_wall,
    }
    ok_s = lambda b: "pass" if b else "FAIL"
    out["summary"] = {
        "gemm_2048": {"us": round(gemm_us, 2), "tflops": round(gemm_tflops, 1),
                      "frac": round(gemm_tflops / PEAK_FP32_MFMA_TFLOPS, 3),
                      "parity": ok_s(gemm_ok)},
        "q2_batched": {"us_per_product": round(qb_us, 3),
                       "weight_gbs": round(Q2_WEIGHT_BYTES / qb_us / 1e3, 0),
                       "frac": round(Q2_ALG_BYTES / qb_us / 1e3 / PEAK_HBM_GBS, 3),
                       "parity": ok_s(qb_ok)},
        "q2_single": {"us": round(q2_us, 3),
                      "weight_gbs": round(Q2_WEIGHT_BYTES / q2_us / 1e3, 0),
                      "frac": round(Q2_ALG_BYTES / q2_us / 1e3 / PEAK_HBM_GBS, 3),
                      "empty_kernel_us": (round(probes["empty_kernel_us"]["512x576"], 3)
                                          if probes else None),
                      "parity": ok_s(q2_ok)},
        "q4_batched_frac": round(Q4_ALG_BYTES / q4b_us / 1e3 / PEAK_HBM_GBS, 3),
        "gemv_f32_frac": round(F32_ALG_BYTES / gf_us / 1e3 / PEAK_HBM_GBS, 3),
        "gemv_f32_batched_frac": round(F32_ALG_BYTES / gfb_us / 1e3 / PEAK_HBM_GBS, 3),
        "q2_transposed_batched_frac": round(QT_ALG_BYTES / min(qtb_us, qtw_us) / 1e3
                                            / PEAK_HBM_GBS, 3),
        "gpt2_block_frac": round(configs.get("gpt2_block_9_products", {})
                                 .get("frac_of_fp32_mfma_peak", float("nan")), 3),
        "parity_all": ok_s(all_ok),
        "cpu_oracle_tflops": round(cpu["value"], 5) if cpu else None,
        "cpu_cores": cpu["cores"] if cpu else None,
    }
    print(json.dumps(out), flush=True)
    return 0 if all_ok else 1


if __name__ == "__main__":
    sys.exit(main())
