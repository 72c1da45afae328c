"""GPU check of the header's statement that every entry point but the
allocation-free one may be called from several host threads.  Eight
threads, each with its own stream (and its own workspace for the sliced
2-bit batch), call a mix of the entry points at once for several rounds; the ctypes calls release
the interpreter lock, so argument checks, the per-device cache and the
launches overlap.  All operands and outputs are allocated and filled before
the threads start, so the threads make no call but the library's.  The
kernels are deterministic, so every result must equal, bit for bit, the same
call made alone beforehand: any difference would be interference between
concurrent calls."""
import threading

import numpy as np
import pytest

from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs
from gpu_util import dev, host, torch

pytestmark = pytest.mark.gpu

THREADS = 8
ROUNDS = 4


def _operands(rng):
    d = {
        "A": dev(inputs.uniform(rng, (300, 500))),
        "B": dev(inputs.uniform(rng, (500, 260))),
        "Bt": dev(inputs.uniform(rng, (260, 500))),
        "C0": dev(inputs.uniform(rng, (300, 260))),
        "W": dev(inputs.normal(rng, (1000, 1536), 0.02)),
        "xv": dev(inputs.normal(rng, (1536,))),
    }
    d["q"] = []
    for _ in range(3):
        Q = rng.integers(0, 256, (1200, 1536 // 4), dtype=np.uint8)
        S = rng.uniform(0.01, 0.05, (1200, 1536 // 64)).astype(np.float16).view(np.int16)
        d["q"].append((dev(Q), dev(S), dev(inputs.normal(rng, (1536,)))))
    # a batch whose rows are cut into slices (workspace per call)
    d["sl"] = []
    for _ in range(8):
        Q = rng.integers(0, 256, (100, 6144 // 4), dtype=np.uint8)
        S = rng.uniform(0.01, 0.05, (100, 6144 // 64)).astype(np.float16).view(np.int16)
        d["sl"].append((dev(Q), dev(S), dev(inputs.normal(rng, (6144,)))))
    return d


def _outputs(d):
    """Fresh outputs for one run of every job; C of the accumulating product
    starts as C0."""
    t = torch()
    f32 = dict(dtype=t.float32, device="cuda")
    return {"gemm": t.empty((300, 260), **f32), "nt": t.empty((300, 260), **f32),
            "ex": d["C0"].clone(), "gemv": t.empty(1000, **f32), "q2": t.empty(1200, **f32),
            "q2b": [t.empty(1200, **f32) for _ in range(3)],
            "gemvb": [t.empty(1000, **f32) for _ in range(2)],
            "q2ws": [t.empty(100, **f32) for _ in range(8)]}


def _workspace():
    t = torch()
    return t.empty(bd.gemv_q2_batched_ws_size(8, 100, 6144), dtype=t.uint8, device="cuda")


def _run(d, o, ws, stream):
    bd.gemm_f32(d["A"], d["B"], o["gemm"], stream=stream)
    bd.gemm_f32_nt(d["A"], d["Bt"], o["nt"], stream=stream)
    bd.gemm_f32_ex(d["A"], d["B"], o["ex"], 0.5, 1.5, stream=stream)
    bd.gemv_f32(d["W"], d["xv"], o["gemv"], stream=stream)
    Q, S, x = d["q"][0]
    bd.gemv_q2(Q, S, x, o["q2"], stream=stream)
    bd.gemv_q2_batched([q[0] for q in d["q"]], [q[1] for q in d["q"]], [q[2] for q in d["q"]],
                       o["q2b"], stream=stream)
    bd.gemv_f32_batched([d["W"], d["W"]], [d["xv"], d["xv"]], o["gemvb"], stream=stream)
    bd.gemv_q2_batched_ws([q[0] for q in d["sl"]], [q[1] for q in d["sl"]],
                          [q[2] for q in d["sl"]], o["q2ws"], workspace=ws, stream=stream)


def _flat(o):
    return [host(v) for k in sorted(o) for v in (o[k] if isinstance(o[k], list) else [o[k]])]


def test_concurrent_calls_from_threads():
    t = torch()
    d = _operands(np.random.default_rng(808))
    ref_out = _outputs(d)
    t.cuda.synchronize()
    _run(d, ref_out, _workspace(), t.cuda.current_stream())
    ref = _flat(ref_out)

    streams = [t.cuda.Stream() for _ in range(THREADS)]
    outs = [[_outputs(d) for _ in range(ROUNDS)] for _ in range(THREADS)]
    wss = [_workspace() for _ in range(THREADS)]   # one per thread: calls on a stream reuse it
    t.cuda.synchronize()
    errors = []
    start = threading.Barrier(THREADS)

    def worker(i):
        try:
            start.wait()
            for r in range(ROUNDS):
                _run(d, outs[i][r], wss[i], streams[i])
        except Exception as e:   # reported after the join
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    assert not errors, errors
    t.cuda.synchronize()
    for i in range(THREADS):
        for r in range(ROUNDS):
            got = _flat(outs[i][r])
            for k, (g, e) in enumerate(zip(got, ref)):
                assert np.array_equal(g, e), "thread %d round %d output %d differs" % (i, r, k)
