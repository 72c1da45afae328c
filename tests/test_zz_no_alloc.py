"""gemv_q2_batched_noalloc, the allocation-free form of gemv_q2_batched_ws:
the partial sums of sliced rows go to the library's fixed per-GPU scratch
buffer instead of a caller's workspace.  Through the C ABI, against
gemv_q2_batched_ws on the same inputs (the same kernels: equal bit for bit)
and against the oracle, on two calls in a row, the second smaller (its
slices then meet the first call's stale partial sums in the buffer); a batch
that does not cut its rows; and a batch whose partial sums would not fit."""
import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs

from gpu_util import assert_close, dev, host, torch

pytestmark = pytest.mark.gpu


def _mats(n, M, K, seed):
    rng = np.random.default_rng(seed)
    return [(rng.integers(0, 256, (M, K // 4), dtype=np.uint8),
             rng.uniform(0.01, 0.05, (M, K // 64)).astype(np.float16).view(np.uint16))
            for _ in range(n)]


def _both(mats, xs):
    t = torch()
    dQ = [dev(Q) for Q, _ in mats]
    dS = [dev(S.view(np.int16)) for _, S in mats]
    dx = [dev(x) for x in xs]
    M, K = mats[0][0].shape[0], xs[0].shape[0]
    ws = t.empty(bd.gemv_q2_batched_ws_size(len(mats), M, K), dtype=t.uint8, device="cuda")
    yw = [host(y) for y in bd.gemv_q2_batched_ws(dQ, dS, dx, workspace=ws)]
    yn = [host(y) for y in bd.gemv_q2_batched_noalloc(dQ, dS, dx)]
    return yw, yn


def test_two_calls_in_a_row_second_smaller():
    for n, M, K, seed, step in ((40, 1536, 12288, 1, 7), (16, 700, 6144, 2, 5)):
        mats = _mats(n, M, K, seed)
        rng = np.random.default_rng(seed + 100)
        xs = [inputs.normal(rng, (K,)) for _ in range(n)]
        yw, yn = _both(mats, xs)
        for b in range(n):
            assert np.array_equal(yn[b], yw[b]), "%dx%d, product %d" % (M, K, b)
        for b in range(0, n, step):
            ref, bound = oracle.gemv_q2(mats[b][0], mats[b][1], xs[b])
            assert_close(yn[b], ref, bound, "%dx%d, product %d" % (M, K, b))


def test_batch_that_does_not_cut_rows():
    """Fewer than 8 products: no slices, the scratch buffer is not used,
    and the result equals gemv_q2_batched's."""
    n, M, K = 5, 300, 12288
    mats = _mats(n, M, K, 3)
    xs = [inputs.normal(np.random.default_rng(4), (K,))] * n
    yw, yn = _both(mats, xs)
    dQ = [dev(Q) for Q, _ in mats]
    dS = [dev(S.view(np.int16)) for _, S in mats]
    yb = [host(y) for y in bd.gemv_q2_batched(dQ, dS, [dev(x) for x in xs])]
    for a, b, c in zip(yn, yw, yb):
        assert np.array_equal(a, b) and np.array_equal(a, c)
    ref, bound = oracle.gemv_q2(mats[0][0], mats[0][1], xs[0])
    assert_close(yn[0], ref, bound, "unsliced batch")


def test_batch_beyond_the_scratch_is_rejected():
    """64 products of 2,049 x 12,288 need 64 x 8 x 2,049 x 4 bytes of partial
    sums, more than the 4 MiB buffer: rejected before anything runs (the
    outputs keep their contents)."""
    t = torch()
    n, M, K = 64, 2049, 12288
    Q = t.zeros((M, K // 4), dtype=t.uint8, device="cuda")
    S = t.zeros((M, K // 64), dtype=t.int16, device="cuda")
    x = t.zeros(K, dtype=t.float32, device="cuda")
    ys = [t.full((M,), 7.0, dtype=t.float32, device="cuda") for _ in range(n)]
    with pytest.raises(bd.GGError) as e:
        bd.gemv_q2_batched_noalloc([Q] * n, [S] * n, [x] * n, ys=ys)
    assert e.value.status == bd.GG_ERR_SCRATCH
    t.cuda.synchronize()
    assert all(bool((y == 7.0).all()) for y in ys)
