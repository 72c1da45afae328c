"""GPU checks of what the header states for non-finite inputs.  The GEMM and
the fp32 GEMV follow IEEE arithmetic: a NaN operand makes exactly the output
cells whose sums contain it NaN, and an infinity meeting finite non-zero
operands gives an infinity of the product's sign, as in the exact sum.  The
packed GEMVs apply the zero point through the sum of x, so any NaN or
infinity in x makes every output NaN (the exact sum would give +-inf for an
infinity), while a NaN scale affects only its own row.  Every other output
still meets the usual bound against the oracle."""
import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs
from gpu_util import assert_close, dev, host

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(4242)


@pytest.mark.parametrize("M,N,K", [(300, 260, 500), (2048, 256, 512)])
def test_gemm_nan_and_inf(M, N, K):
    A = inputs.uniform(RNG, (M, K))
    B = inputs.uniform(RNG, (K, N))
    A[np.abs(A) < 1e-3] = 0.5           # no zero meets the infinity
    i0, k0, k1, j1 = M // 3, K // 5, K - 2, N - 3
    A[i0, k0] = np.nan
    B[k1, j1] = np.inf
    C = host(bd.gemm_f32(dev(A), dev(B)))
    assert np.all(np.isnan(C[i0]))
    rows = np.arange(M) != i0
    col = C[rows, j1]
    assert np.array_equal(col, np.where(A[rows, k1] > 0, np.inf, -np.inf).astype(np.float32))
    cols = np.arange(N) != j1
    Af, Bf = A[rows], B[:, cols]
    ref, bound = oracle.gemm_nn(Af, Bf)
    assert_close(C[np.ix_(rows, cols)], ref, bound, "finite cells %dx%dx%d" % (M, N, K))


def test_gemv_f32_nan_row():
    W = inputs.normal(RNG, (1000, 1536), 0.02)
    x = inputs.normal(RNG, (1536,))
    W[17, 900] = np.nan
    y = host(bd.gemv_f32(dev(W), dev(x)))
    assert np.isnan(y[17])
    keep = np.arange(1000) != 17
    ref, bound = oracle.gemv(W[keep], x)
    assert_close(y[keep], ref, bound, "gemv_f32 finite rows")


def _packed(M, K, bits):
    Q = RNG.integers(0, 256, (M, -(-K * bits // 8)), dtype=np.uint8)
    S = RNG.uniform(0.01, 0.05, (M, -(-K // 64))).astype(np.float16).view(np.uint16)
    return Q, S


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("M,K", [(12288, 1536), (300, 1000), (1536, 12288)])
def test_packed_nonfinite(bits, M, K):
    Q, S = _packed(M, K, bits)
    f = bd.gemv_q2 if bits == 2 else bd.gemv_q4
    ref_fn = oracle.gemv_q2 if bits == 2 else oracle.gemv_q4
    x = inputs.normal(RNG, (K,))
    # a NaN scale: only its row
    S2 = S.copy()
    S2[M // 2, 0] = 0x7E00
    y = host(f(dev(Q), dev(S2.view(np.int16)), dev(x)))
    assert np.isnan(y[M // 2])
    keep = np.arange(M) != M // 2
    ref, bound = ref_fn(Q, S2, x)
    assert_close(y[keep], ref[keep], bound[keep], "%d-bit NaN scale, other rows" % bits)
    # a NaN or an infinity in x: every row
    for bad in (np.nan, np.inf, -np.inf):
        xb = x.copy()
        xb[K // 3] = bad
        y = host(f(dev(Q), dev(S.view(np.int16)), dev(xb)))
        assert np.all(np.isnan(y)), "%d-bit x[%d] = %r" % (bits, K // 3, bad)
