"""GPU parity of the GEMM on wide grids (M, N >= 2048, the direct-load path
with more tiles than compute units): ragged tile edges, a K tail inside the
last slab, all four transpose pairs, alpha/beta, padded leading dimensions
with NaN in the padding, exact integer sums and determinism, against the
oracle."""
import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs
from gpu_util import assert_close, dev, host, torch

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(128)
PAIRS = [(0, 0), (1, 0), (0, 1), (1, 1)]


def _ops(ta, tb, M, N, K, gen):
    return gen((K, M) if ta else (M, K)), gen((N, K) if tb else (K, N))


def _sample(M, N, n=600):
    rows = np.concatenate([RNG.integers(0, M, n), [0, M - 1, M - 1, 0, 2048 % M, M - 3]])
    cols = np.concatenate([RNG.integers(0, N, n), [0, N - 1, 0, N - 1, N - 5, 2047 % N]])
    return rows, cols


@pytest.mark.parametrize("ta,tb", PAIRS)
def test_ragged_grid_with_k_tail(ta, tb):
    """M, N one partial tile past 16 x 128, K = 4 slabs + 4: against the
    oracle on every element, with alpha and beta."""
    M, N, K = 2052, 2056, 132
    A, B = _ops(ta, tb, M, N, K, lambda s: inputs.uniform(RNG, s))
    C = inputs.uniform(RNG, (M, N))
    ref, bound = oracle.gemm_ex(A, B, C, 1.5, -0.5, trans_a=bool(ta), trans_b=bool(tb))
    dC = dev(C)
    bd.gemm_f32_ex(dev(A), dev(B), dC, 1.5, -0.5, trans_a=bool(ta), trans_b=bool(tb))
    assert_close(host(dC), ref, bound, "wide t%d%d %dx%dx%d" % (ta, tb, M, N, K))


@pytest.mark.parametrize("ta,tb", PAIRS)
def test_integer_exact_sampled(ta, tb):
    """Integer inputs in [-8, 8] with K = 1028: every partial sum is an
    integer below 2^24, so sampled cells equal the oracle bit for bit."""
    M, N, K = 2176, 2304, 1028
    A, B = _ops(ta, tb, M, N, K, lambda s: inputs.integers(RNG, s))
    dC = bd.gemm_f32_ex(dev(A), dev(B), None, 1.0, 0.0, trans_a=bool(ta), trans_b=bool(tb))
    C = host(dC)
    rows, cols = _sample(M, N)
    ref, _ = oracle.gemm_cells(A, B, rows, cols, trans_a=bool(ta), trans_b=bool(tb))
    assert np.array_equal(C[rows, cols].astype(np.float64), ref)


def test_padded_leading_dimensions_nan():
    """lda, ldb and ldc padded by 4 and 8 floats (still 16-byte rows, so the
    direct loads apply) with NaN in the padding of A and B."""
    M, N, K = 2048, 2048, 256
    t = torch()
    A = inputs.uniform(RNG, (M, K))
    B = inputs.uniform(RNG, (K, N))
    Ap = np.full((M, K + 4), np.nan, np.float32)
    Ap[:, :K] = A
    Bp = np.full((K, N + 8), np.nan, np.float32)
    Bp[:, :N] = B
    dA = dev(Ap)[:, :K]
    dB = dev(Bp)[:, :N]
    Cbuf = t.full((M, N + 4), 7.0, dtype=t.float32, device="cuda")
    dC = Cbuf[:, :N]
    bd.gemm_f32(dA, dB, C=dC)
    got = host(Cbuf)
    assert np.all(got[:, N:] == 7.0)
    rows, cols = _sample(M, N)
    ref, bound = oracle.gemm_cells(A, B, rows, cols)
    assert_close(got[rows, cols], ref, bound, "padded wide")


def test_full_size_2048_cube_sampled_and_deterministic():
    A, B = inputs.large_square(3)
    dA, dB = dev(A), dev(B)
    C1 = host(bd.gemm_f32(dA, dB))
    C2 = host(bd.gemm_f32(dA, dB))
    assert np.array_equal(C1, C2)
    rows, cols = _sample(2048, 2048, 2000)
    ref, bound = oracle.gemm_cells(A, B, rows, cols)
    assert_close(C1[rows, cols], ref, bound, "2048^3")
