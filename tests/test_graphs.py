"""GPU check that the entry points can be captured in a HIP graph and
replayed: they allocate nothing, clear nothing with memsets and keep no state
between calls, so a replay must redo exactly what an eager call does.  One
graph holds the GEMM (plain, TN, NT and accumulating), the single and batched
fp32 GEMV, the single and batched 2-bit and 4-bit GEMVs, and a 2-bit batch
whose rows are cut into slices through a workspace.  It is replayed five times, with
eager library calls and torch work on the same buffers' neighbours in
between, and after every replay each output is compared bit for bit with
eager calls.  The accumulating product (beta = 1) grows by one term per
replay, so it also shows that every replay reran its kernel."""
import numpy as np
import pytest

from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs
from gpu_util import dev, host, torch

pytestmark = pytest.mark.gpu

REPLAYS = 5


def _packed(rng, M, K, bits):
    Q = rng.integers(0, 256, (M, K * bits // 8), dtype=np.uint8)
    S = rng.uniform(0.01, 0.05, (M, K // 64)).astype(np.float16).view(np.int16)
    return dev(Q), dev(S), dev(inputs.normal(rng, (K,)))


def test_capture_and_replay():
    t = torch()
    rng = np.random.default_rng(909)
    A = dev(inputs.uniform(rng, (520, 700)))
    At = dev(inputs.uniform(rng, (700, 520)))
    B = dev(inputs.uniform(rng, (700, 330)))
    Bt = dev(inputs.uniform(rng, (330, 700)))
    C0 = dev(inputs.uniform(rng, (520, 330)))
    W = dev(inputs.normal(rng, (2000, 1536), 0.02))
    xv = dev(inputs.normal(rng, (1536,)))
    q2 = [_packed(rng, 3000, 1536, 2) for _ in range(3)]
    q4 = _packed(rng, 3000, 1536, 4)
    sl = [_packed(rng, 100, 6144, 2) for _ in range(16)]           # rows cut into slices
    ws = t.empty(bd.gemv_q2_batched_ws_size(16, 100, 6144), dtype=t.uint8, device="cuda")
    f32 = dict(dtype=t.float32, device="cuda")

    def outputs():
        return {"nn": t.empty((520, 330), **f32), "tn": t.empty((520, 330), **f32),
                "nt": t.empty((520, 330), **f32), "gemv": t.empty(2000, **f32),
                "q2": t.empty(3000, **f32), "q4": t.empty(3000, **f32),
                "q2b": [t.empty(3000, **f32) for _ in range(3)],
                "gemvb": [t.empty(2000, **f32) for _ in range(2)],
                "q2ws": [t.empty(100, **f32) for _ in range(16)]}

    def run(o, acc, stream):
        bd.gemm_f32(A, B, o["nn"], stream=stream)
        bd.gemm_f32_tn(At, B, o["tn"], stream=stream)
        bd.gemm_f32_nt(A, Bt, o["nt"], stream=stream)
        bd.gemm_f32_ex(A, B, acc, 0.25, 1.0, stream=stream)
        bd.gemv_f32(W, xv, o["gemv"], stream=stream)
        bd.gemv_q2(*q2[0], o["q2"], stream=stream)
        bd.gemv_q4(*q4, o["q4"], stream=stream)
        bd.gemv_q2_batched([q[0] for q in q2], [q[1] for q in q2], [q[2] for q in q2],
                           o["q2b"], stream=stream)
        bd.gemv_f32_batched([W, W], [xv, xv], o["gemvb"], stream=stream)
        bd.gemv_q2_batched_ws([q[0] for q in sl], [q[1] for q in sl], [q[2] for q in sl],
                              o["q2ws"], workspace=ws, stream=stream)

    def flat(o):
        return [host(v) for k in sorted(o) for v in (o[k] if isinstance(o[k], list) else [o[k]])]

    # eager reference, and the accumulator's value after each of REPLAYS terms
    eager, acc_e = outputs(), C0.clone()
    acc_ref = []
    for _ in range(REPLAYS):
        run(eager, acc_e, t.cuda.current_stream())
        acc_ref.append(host(acc_e))
    ref = flat(eager)

    side = t.cuda.Stream()
    got, acc_g = outputs(), C0.clone()
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g, stream=side):
        run(got, acc_g, side)
    # capture records without running: the accumulator still holds C0
    t.cuda.synchronize()
    assert np.array_equal(host(acc_g), host(C0))

    scratch = outputs()
    for k in range(REPLAYS):
        for v in got.values():   # clobber the outputs so that stale values cannot pass
            for x in (v if isinstance(v, list) else [v]):
                x.fill_(float("nan"))
        g.replay()
        # eager work between replays: library calls on other buffers, torch ops
        run(scratch, C0.clone(), t.cuda.current_stream())
        _ = (W * 2.0).sum()
        t.cuda.synchronize()
        for i, (a, b) in enumerate(zip(flat(got), ref)):
            assert np.array_equal(a, b), "replay %d output %d differs from the eager call" % (k, i)
        assert np.array_equal(host(acc_g), acc_ref[k]), "replay %d accumulator" % k
