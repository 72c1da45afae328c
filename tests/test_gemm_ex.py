"""GPU parity of gemm_f32_ex, C = alpha * op(A).op(B) + beta * C, against the
CPU oracle, through the C ABI, for all four transpose pairs on both load paths
(aligned operands load straight into LDS, others through registers)."""
import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs
from gpu_util import assert_close, canaries_intact, dev, guarded, host, torch

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(31)
PAIRS = [(0, 0), (1, 0), (0, 1), (1, 1)]


def _ops(ta, tb, M, N, K, gen):
    return gen((K, M) if ta else (M, K)), gen((N, K) if tb else (K, N))


def _ex(A, B, C, alpha, beta, ta, tb):
    dC = dev(C)
    bd.gemm_f32_ex(dev(A), dev(B), dC, alpha, beta, trans_a=bool(ta), trans_b=bool(tb))
    return host(dC)


@pytest.mark.parametrize("ta,tb", PAIRS)
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (2.5, -0.5), (-1.0, 1.0), (0.75, 3.0)])
@pytest.mark.parametrize("M,N,K", [(196, 132, 100), (129, 67, 33)])
def test_matches_oracle(ta, tb, alpha, beta, M, N, K):
    A, B = _ops(ta, tb, M, N, K, lambda s: inputs.uniform(RNG, s))
    C = inputs.uniform(RNG, (M, N))
    ref, bound = oracle.gemm_ex(A, B, C, alpha, beta, trans_a=bool(ta), trans_b=bool(tb))
    assert_close(_ex(A, B, C, alpha, beta, ta, tb), ref, bound,
                 "t%d%d a=%g b=%g %dx%dx%d" % (ta, tb, alpha, beta, M, N, K))


@pytest.mark.parametrize("ta,tb", PAIRS)
@pytest.mark.parametrize("M,N,K", [(132, 68, 36), (2048, 2048, 100), (33, 5, 7)])
def test_integer_exact(ta, tb, M, N, K):
    A, B = _ops(ta, tb, M, N, K, lambda s: inputs.integers(RNG, s))
    C = inputs.integers(RNG, (M, N))
    ref, _ = oracle.gemm_ex(A, B, C, 2.0, -1.0, trans_a=bool(ta), trans_b=bool(tb))
    assert np.array_equal(_ex(A, B, C, 2.0, -1.0, ta, tb).astype(np.float64), ref)


@pytest.mark.parametrize("ta,tb", PAIRS)
def test_beta_zero_does_not_read_c(ta, tb):
    A, B = _ops(ta, tb, 100, 72, 64, lambda s: inputs.uniform(RNG, s))
    C = np.full((100, 72), np.nan, np.float32)
    got = _ex(A, B, C, 1.5, 0.0, ta, tb)
    ref, bound = oracle.gemm_ex(A, B, None, 1.5, 0.0, trans_a=bool(ta), trans_b=bool(tb))
    assert np.all(np.isfinite(got))
    assert_close(got, ref, bound, "beta = 0 over NaN")


def test_alpha_zero_reads_neither_operand():
    A = np.full((64, 48), np.nan, np.float32)
    B = np.full((48, 40), np.nan, np.float32)
    C = inputs.uniform(RNG, (64, 40))
    assert np.array_equal(_ex(A, B, C, 0.0, -2.0, 0, 0), np.float32(-2.0) * C)


def test_k_zero_scales_c():
    t = torch()
    A = t.empty((70, 0), dtype=t.float32, device="cuda")
    B = t.empty((0, 45), dtype=t.float32, device="cuda")
    C = inputs.uniform(RNG, (70, 45))
    dC = dev(C)
    bd.gemm_f32_ex(A, B, dC, 3.0, 0.5)
    assert np.array_equal(host(dC), np.float32(0.5) * C)


@pytest.mark.parametrize("ta,tb,f", [(0, 0, bd.gemm_f32), (1, 0, bd.gemm_f32_tn),
                                     (0, 1, bd.gemm_f32_nt)])
@pytest.mark.parametrize("M,N,K", [(260, 196, 100), (129, 67, 33)])
def test_plain_form_equals_existing_entry_points_bitwise(ta, tb, f, M, N, K):
    A, B = _ops(ta, tb, M, N, K, lambda s: inputs.uniform(RNG, s))
    plain = host(f(dev(A), dev(B)))
    got = _ex(A, B, np.full((M, N), np.nan, np.float32), 1.0, 0.0, ta, tb)
    assert np.array_equal(got, plain)


def test_gradient_accumulation_over_micro_batches():
    # dW = X^T.dY over 512 + 512 rows, accumulated in two calls (beta = 1),
    # against the one product over all 1,024 rows
    X = inputs.normal(RNG, (1024, 768))
    dY = inputs.normal(RNG, (1024, 256))
    dW = dev(np.zeros((768, 256), np.float32))
    bd.gemm_f32_ex(dev(X[:512]), dev(dY[:512]), dW, 1.0, 0.0, trans_a=True)
    bd.gemm_f32_ex(dev(X[512:]), dev(dY[512:]), dW, 1.0, 1.0, trans_a=True)
    ref, bound = oracle.gemm_tn(X, dY)
    assert_close(host(dW), ref, bound, "accumulated dW")


def test_in_place_with_padded_ldc_and_canaries():
    M, N, K = 130, 75, 93
    A = inputs.uniform(RNG, (M, K))
    B = inputs.uniform(RNG, (K, N))
    C0 = inputs.uniform(RNG, (M, N))
    buf, _ = guarded(M, N + 7)
    Cw = buf[64:64 + M * (N + 7)].view(M, N + 7)
    Cw[:, :N].copy_(dev(C0))
    bd.gemm_f32_ex(dev(A), dev(B), Cw[:, :N], -0.5, 2.0)
    ref, bound = oracle.gemm_ex(A, B, C0, -0.5, 2.0)
    assert_close(host(Cw)[:, :N], ref, bound, "in place")
    assert np.all(host(Cw)[:, N:] == np.float32(1.2345e9)), "wrote outside C's columns"
    assert canaries_intact(buf), "wrote outside C"
