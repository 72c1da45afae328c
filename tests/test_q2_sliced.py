"""gemv_q2_batched_ws: batches of 2-bit products whose long rows (K a
multiple of 1,536, at least 6,144) are cut into slices of 1,536 columns, each
slice's partial row sums going to the caller's workspace and a second kernel
adding them in slice order.  Element by element against the oracle, through
the C ABI: the transposed 1,536 x 12,288 shape of the rotation set, ragged
row counts, several slice counts, more than 64 products (the workspace reused
by a second launch), x far from 1 and chunks of different magnitudes, exact
integer sums, non-finite x in one slice, a NaN scale, padded rows, batches
that do not cut their rows (fewer than 8 products, short rows, misaligned
operands: same bits as gemv_q2_batched, workspace untouched), and the
workspace checks.
"""
import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs

from gpu_util import assert_close, dev, host, torch

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A


def _mats(n, M, K, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        Q = rng.integers(0, 256, (M, K // 4), dtype=np.uint8)
        S = rng.uniform(0.01, 0.05, (M, K // 64)).astype(np.float16).view(np.uint16)
        out.append((Q, S))
    return out


def _workspace(n, M, K, extra=0):
    t = torch()
    size = bd.gemv_q2_batched_ws_size(n, M, K)
    return t.full((size + extra,), SENTINEL, dtype=t.uint8, device="cuda"), size


def _run(mats, xs, ws=None):
    dQ = [dev(Q) for Q, _ in mats]
    dS = [dev(S.view(np.int16)) for _, S in mats]
    dx = [dev(x) for x in xs]
    if ws is None:
        ws, _ = _workspace(len(mats), mats[0][0].shape[0], xs[0].shape[0])
    ys = bd.gemv_q2_batched_ws(dQ, dS, dx, workspace=ws)
    return [host(y) for y in ys]


def _check_all(mats, xs, ys, what, step=1):
    for b in range(0, len(mats), step):
        (Q, S), x, y = mats[b], xs[b], ys[b]
        ref, bound = oracle.gemv_q2(Q, S, x)
        assert_close(y, ref, bound, "%s, product %d" % (what, b))


def test_workspace_size_rule():
    assert bd.gemv_q2_batched_ws_size(40, 1536, 12288) == 40 * 8 * 1536 * 4
    assert bd.gemv_q2_batched_ws_size(130, 1536, 12288) == 64 * 8 * 1536 * 4
    assert bd.gemv_q2_batched_ws_size(8, 100, 6144) == 8 * 4 * 100 * 4
    assert bd.gemv_q2_batched_ws_size(7, 1536, 12288) == 0       # too few products
    assert bd.gemv_q2_batched_ws_size(40, 12288, 1536) == 0      # short rows
    assert bd.gemv_q2_batched_ws_size(40, 1536, 4608) == 0       # three slices
    assert bd.gemv_q2_batched_ws_size(40, 1536, 12800) == 0      # not a multiple of 1,536
    assert bd.gemv_q2_batched_ws_size(40, 0, 12288) == 0


def test_transposed_rotation_shape():
    """The 1,536 x 12,288 shape of the transposed rotation set, 40 products
    (a token), against the oracle; repeated launches give the same bits."""
    M, K, n = inputs.GEMV_K, inputs.GEMV_M, 40
    mats = [inputs.q2_weight(r, M, K) for r in range(n)]
    xs = [inputs.q2_x(K)] * n
    ys = _run(mats, xs)
    _check_all(mats, xs, ys, "1536x12288", step=3)
    again = _run(mats, xs)
    for a, b in zip(ys, again):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("M,K", [(1, 6144), (127, 6144), (128, 7680), (129, 12288),
                                 (1000, 9216), (300, 24576)])
def test_shapes_distinct_x(M, K):
    n = 17
    mats = _mats(n, M, K, M + K)
    rng = np.random.default_rng(3 * M + K)
    xs = [inputs.normal(rng, (K,)) for _ in range(n)]
    _check_all(mats, xs, _run(mats, xs), "%dx%d" % (M, K))


@pytest.mark.parametrize("n", [8, 64, 65, 130])
def test_batch_sizes(n):
    """Up to two full launches and a partial third, which reuse the workspace
    in stream order."""
    M, K = 200, 6144
    base = _mats(5, M, K, 40 + n)
    mats = [base[b % 5] for b in range(n)]
    rng = np.random.default_rng(n)
    xs = [inputs.normal(rng, (K,)) for _ in range(n)]
    ys = _run(mats, xs)
    _check_all(mats, xs, ys, "batch of %d" % n)


@pytest.mark.parametrize("scale", [2.0 ** 100, 2.0 ** -100, 2.0 ** -120])
def test_x_far_from_one(scale):
    M, K, n = 300, 6144, 16
    mats = _mats(n, M, K, 50)
    rng = np.random.default_rng(51)
    xs = [(inputs.normal(rng, (K,)).astype(np.float64) * scale).astype(np.float32)
          for _ in range(n)]
    ys = _run(mats, xs)
    assert all(np.all(np.isfinite(y)) for y in ys)
    _check_all(mats, xs, ys, "x scaled by 2^%d" % int(np.log2(scale)), step=5)


def test_slices_of_different_magnitudes():
    """Each slice at its own scale, 2^-80 .. 2^80: every slice is quantised
    on its own chunks, and the partials of different sizes still add within
    the bound."""
    M, K, n = 400, 12288, 16
    mats = _mats(n, M, K, 52)
    rng = np.random.default_rng(53)
    xs = []
    for _ in range(n):
        x = inputs.normal(rng, (K,)).astype(np.float64)
        for s in range(K // 1536):
            x[1536 * s:1536 * (s + 1)] *= 2.0 ** (20 * (s % 9) - 80)
        xs.append(x.astype(np.float32))
    _check_all(mats, xs, _run(mats, xs), "slices of different magnitudes", step=5)


def test_integer_sums_are_exact():
    """Scales 2.0 and integer x in [-8, 8]: every partial and the row sum are
    integers below 2^24, so the result equals the oracle bit for bit."""
    M, K, n = 333, 6144, 16
    rng = np.random.default_rng(54)
    mats = [(rng.integers(0, 256, (M, K // 4), dtype=np.uint8),
             np.full((M, K // 64), 0x4000, np.uint16)) for _ in range(n)]
    xs = [rng.integers(-8, 9, K).astype(np.float32) for _ in range(n)]
    for (Q, S), x, y in zip(mats, xs, _run(mats, xs)):
        ref, _ = oracle.gemv_q2(Q, S, x)
        assert np.array_equal(y.astype(np.float64), ref)


def test_non_finite_x_in_one_slice():
    """A NaN or an infinity in one slice of one product's x makes every
    output of that product NaN; the other products are unaffected."""
    M, K, n = 300, 9216, 16
    mats = _mats(n, M, K, 55)
    rng = np.random.default_rng(56)
    for bad in (np.inf, -np.inf, np.nan):
        xs = [inputs.normal(rng, (K,)) for _ in range(n)]
        xs[3][5000] = bad
        ys = _run(mats, xs)
        assert np.all(np.isnan(ys[3])), bad
        _check_all([mats[0]], [xs[0]], [ys[0]], "finite neighbour")


def test_nan_scale_makes_its_row_nan():
    M, K, n = 300, 6144, 16
    mats = _mats(n, M, K, 57)
    Q, S = mats[2]
    S = S.copy()
    S[17, 70] = np.float16(np.nan).view(np.uint16)
    mats[2] = (Q, S)
    x = inputs.normal(np.random.default_rng(58), (K,))
    y = _run(mats, [x] * n)[2]
    assert np.isnan(y[17])
    rows = np.arange(M) != 17
    ref, bound = oracle.gemv_q2(Q, S, x)
    assert_close(y[rows], ref[rows], bound[rows], "rows beside a NaN scale")


def test_padded_rows_are_ignored():
    M, K, n = 250, 6144, 16
    rng = np.random.default_rng(59)
    Qp = rng.integers(0, 256, (M, K // 4 + 64), dtype=np.uint8)
    Sp = rng.uniform(0.01, 0.05, (M, K // 64 + 8)).astype(np.float16)
    Sp[:, K // 64:] = np.float16(np.nan)
    x = inputs.normal(rng, (K,))
    dQ, dS = dev(Qp)[:, :K // 4], dev(Sp.view(np.int16))[:, :K // 64]
    ws, _ = _workspace(n, M, K)
    ys = bd.gemv_q2_batched_ws([dQ] * n, [dS] * n, [dev(x)] * n, workspace=ws)
    ref, bound = oracle.gemv_q2(np.ascontiguousarray(Qp[:, :K // 4]),
                                np.ascontiguousarray(Sp[:, :K // 64]).view(np.uint16), x)
    for y in ys:
        assert_close(host(y), ref, bound, "padded rows")


@pytest.mark.parametrize("case", ["few", "short", "misaligned_x"])
def test_batches_that_do_not_cut_rows(case):
    """Fewer than 8 products, rows below 6,144 columns, or an x off 16 bytes:
    the batch runs gemv_q2_batched's kernels (same bits) and leaves the
    workspace as it was."""
    t = torch()
    M, K, n = {"few": (500, 12288, 7), "short": (500, 3072, 16),
               "misaligned_x": (500, 6144, 16)}[case]
    mats = _mats(n, M, K, 60)
    rng = np.random.default_rng(61)
    xs = [inputs.normal(rng, (K + 1,)) for _ in range(n)]
    dQ = [dev(Q) for Q, _ in mats]
    dS = [dev(S.view(np.int16)) for _, S in mats]
    off = 1 if case == "misaligned_x" else 0
    dx = [dev(x)[off:off + K] for x in xs]
    ws = t.full((max(bd.gemv_q2_batched_ws_size(n, M, K), 1 << 16),), SENTINEL,
                dtype=t.uint8, device="cuda")
    ya = [host(y) for y in bd.gemv_q2_batched_ws(dQ, dS, dx, workspace=ws)]
    yb = [host(y) for y in bd.gemv_q2_batched(dQ, dS, dx)]
    for a, b in zip(ya, yb):
        assert np.array_equal(a, b)
    assert bool((ws == SENTINEL).all())
    _check_all(mats[:1], [np.ascontiguousarray(xs[0][off:off + K])], ya[:1], case)


def test_workspace_checks():
    t = torch()
    M, K, n = 64, 6144, 16
    mats = _mats(n, M, K, 62)
    dQ = [dev(Q) for Q, _ in mats]
    dS = [dev(S.view(np.int16)) for _, S in mats]
    dx = [dev(inputs.normal(np.random.default_rng(63), (K,)))] * n
    size = bd.gemv_q2_batched_ws_size(n, M, K)
    ws = t.empty(size + 64, dtype=t.uint8, device="cuda")
    with pytest.raises(bd.GGError) as e:
        bd.gemv_q2_batched_ws(dQ, dS, dx, workspace=ws[:size - 4])
    assert e.value.status == bd.GG_ERR_INVALID_ARG
    with pytest.raises(bd.GGError) as e:
        bd.gemv_q2_batched_ws(dQ, dS, dx, workspace=ws[4:size + 4])      # not 16-byte aligned
    assert e.value.status == bd.GG_ERR_INVALID_ARG
    ys = [t.empty(M, dtype=t.float32, device="cuda") for _ in range(n)]
    over = ws[:size].view(t.float32)
    ys[5] = over[16:16 + M]                                               # y inside the workspace
    with pytest.raises(bd.GGError) as e:
        bd.gemv_q2_batched_ws(dQ, dS, dx, ys=ys, workspace=ws[:size])
    assert e.value.status == bd.GG_ERR_ALIAS
