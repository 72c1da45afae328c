"""Every matrix of every rotation set the benchmark streams, element by element
against the oracle: the 128 2-bit matrices at 12,288 x 1,536 and at the
transposed 1,536 x 12,288, the 64 4-bit matrices and the 48 fp32 matrices,
each through the single-product entry point and through batched launches of
up to 64 products (the fp32 batch must equal the single calls bit for bit).
The oracle runs on all host cores."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs
from gpu_util import assert_close, torch

pytestmark = pytest.mark.gpu

CORES = len(os.sched_getaffinity(0))


def _refs(fn, n):
    with ThreadPoolExecutor(max_workers=CORES) as pool:
        return list(pool.map(fn, range(n)))


def _packed(bits, n, M, K, x):
    t = torch()
    gen = inputs.q2_weight if bits == 2 else inputs.q4_weight
    single = bd.gemv_q2 if bits == 2 else bd.gemv_q4
    batched = bd.gemv_q2_batched if bits == 2 else bd.gemv_q4_batched
    ref_fn = oracle.gemv_q2 if bits == 2 else oracle.gemv_q4
    dx = t.from_numpy(x).cuda()
    mats = [gen(r, M, K) for r in range(n)]
    dQ = [t.from_numpy(Q).cuda() for Q, _ in mats]
    dS = [t.from_numpy(S.view(np.int16)).cuda() for _, S in mats]
    ys = t.empty((n, M), dtype=t.float32, device="cuda")
    yb = t.empty((n, M), dtype=t.float32, device="cuda")
    for r in range(n):
        single(dQ[r], dS[r], dx, y=ys[r])
    for b0 in range(0, n, 64):
        idx = range(b0, min(n, b0 + 64))
        batched([dQ[r] for r in idx], [dS[r] for r in idx], [dx] * len(idx),
                ys=[yb[r] for r in idx])
    t.cuda.synchronize()
    ys, yb = ys.cpu().numpy(), yb.cpu().numpy()
    refs = _refs(lambda r: ref_fn(mats[r][0], mats[r][1], x), n)
    for r in range(n):
        assert_close(ys[r], refs[r][0], refs[r][1], "%d-bit %dx%d matrix %d, single" % (bits, M, K, r))
        assert_close(yb[r], refs[r][0], refs[r][1], "%d-bit %dx%d matrix %d, batched" % (bits, M, K, r))


def test_q2_set():
    _packed(2, inputs.GEMV_Q2_ROTATION, inputs.GEMV_M, inputs.GEMV_K, inputs.q2_x())


def test_q2_transposed_set():
    _packed(2, inputs.GEMV_Q2_ROTATION, inputs.GEMV_K, inputs.GEMV_M, inputs.q2_x(inputs.GEMV_M))


def test_q4_set():
    _packed(4, 64, inputs.GEMV_M, inputs.GEMV_K, inputs.q2_x())


def test_f32_set():
    t = torch()
    x = inputs.gemv_f32_x()
    dx = t.from_numpy(x).cuda()
    n = inputs.GEMV_F32_ROTATION
    y = t.empty((n, inputs.GEMV_M), dtype=t.float32, device="cuda")
    yb = t.full((n, inputs.GEMV_M), float("nan"), dtype=t.float32, device="cuda")
    Ws = []
    for r in range(n):
        Ws.append(t.from_numpy(inputs.gemv_f32_weight(r)).cuda())
        bd.gemv_f32(Ws[r], dx, y=y[r])
    bd.gemv_f32_batched(Ws, [dx] * n, ys=[yb[r] for r in range(n)])
    t.cuda.synchronize()
    del Ws
    y, yb = y.cpu().numpy(), yb.cpu().numpy()
    assert np.array_equal(yb, y), "fp32 batch differs from single calls"
    refs = _refs(lambda r: oracle.gemv(inputs.gemv_f32_weight(r), x), n)
    for r in range(n):
        assert_close(y[r], refs[r][0], refs[r][1], "fp32 matrix %d" % r)
