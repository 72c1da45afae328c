"""GPU parity of the GEMM on small grids, where a 64 x 64 tile grid would
cover fewer than half the compute units: such products take 32 x 32 tiles
when those fit one per CU, else narrow tiles (64 x 32 or 32 x 64, whichever
pads less) with two waves per k-group.  All four transpose pairs against
the oracle on every element, at the classifier shape (346 x 768 x 768, narrow
tiles), ragged and tiny shapes, a K tail inside a slab, K below one slab,
K-heavy products split over four k-groups, alpha/beta, and padded leading
dimensions with NaN in the padding."""
import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs
from gpu_util import assert_close, dev, host, torch

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(3264)
PAIRS = [(0, 0), (1, 0), (0, 1), (1, 1)]


def _ops(ta, tb, M, N, K, gen):
    return gen((K, M) if ta else (M, K)), gen((N, K) if tb else (K, N))


@pytest.mark.parametrize("ta,tb", PAIRS)
@pytest.mark.parametrize("M,N,K", [(346, 768, 768), (33, 68, 36), (100, 200, 1028),
                                   (256, 256, 256), (64, 96, 4), (132, 36, 100)])
def test_matches_oracle(ta, tb, M, N, K):
    A, B = _ops(ta, tb, M, N, K, lambda s: inputs.uniform(RNG, s))
    C = inputs.uniform(RNG, (M, N))
    ref, bound = oracle.gemm_ex(A, B, C, 1.25, -0.75, trans_a=bool(ta), trans_b=bool(tb))
    dC = dev(C)
    bd.gemm_f32_ex(dev(A), dev(B), dC, 1.25, -0.75, trans_a=bool(ta), trans_b=bool(tb))
    assert_close(host(dC), ref, bound, "small t%d%d %dx%dx%d" % (ta, tb, M, N, K))


@pytest.mark.parametrize("ta,tb", PAIRS)
def test_integer_exact(ta, tb):
    M, N, K = 346, 768, 768
    A, B = _ops(ta, tb, M, N, K, lambda s: inputs.integers(RNG, s))
    ref, _ = oracle.gemm_ex(A, B, None, 1.0, 0.0, trans_a=bool(ta), trans_b=bool(tb))
    got = host(bd.gemm_f32_ex(dev(A), dev(B), None, 1.0, 0.0, trans_a=bool(ta), trans_b=bool(tb)))
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("ta,tb", PAIRS)
def test_padded_leading_dimensions(ta, tb):
    """Leading dimensions padded by 4 and 8 floats (16-byte rows kept, so
    the direct loads apply), NaN in the padding, C padded with a canary."""
    M, N, K = 200, 136, 300
    t = torch()
    A, B = _ops(ta, tb, M, N, K, lambda s: inputs.uniform(RNG, s))

    def padded(X, extra):
        P = np.full((X.shape[0], X.shape[1] + extra), np.nan, np.float32)
        P[:, :X.shape[1]] = X
        return dev(P)[:, :X.shape[1]]
    dA, dB = padded(A, 4), padded(B, 8)
    Cbuf = t.full((M, N + 4), 5.0, dtype=t.float32, device="cuda")
    bd.gemm_f32_ex(dA, dB, Cbuf[:, :N], 1.0, 0.0, trans_a=bool(ta), trans_b=bool(tb))
    got = host(Cbuf)
    assert np.all(got[:, N:] == 5.0)
    ref, bound = oracle.gemm_ex(A, B, None, 1.0, 0.0, trans_a=bool(ta), trans_b=bool(tb))
    assert_close(got[:, :N], ref, bound, "small padded t%d%d" % (ta, tb))


def test_classifier_config_deterministic():
    A, B = inputs.classifier()
    dA, dB = dev(A), dev(B)
    C1, C2 = host(bd.gemm_f32(dA, dB)), host(bd.gemm_f32(dA, dB))
    assert np.array_equal(C1, C2)
    ref, bound = oracle.gemm_nn(A, B)
    assert_close(C1, ref, bound, "346x768x768")
