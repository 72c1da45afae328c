"""GPU parity of the GEMM's smaller direct-load tiles, chosen by how evenly a
grid spreads over the compute units: 32 x 32 tiles on small grids that fit
one per CU, narrow tiles (64 x 32 or 32 x 64, whichever pads M and N less;
on a tie 64 x 32 when A is x-major) on small grids that do not and on
grids whose last round of 64 x 64 tiles would leave most CUs idle.  Small
grids split the k-slabs over up to 8 groups (32 x 32) or 6 (narrow).  All
four transpose pairs are checked against the oracle on every element, with
ragged tile edges, K tails inside a slab, one to eight k-groups, alpha/beta
and padded leading dimensions.  The helper `regime` restates the
launcher's choice so that each case is known to reach the tiles it is
meant for."""
import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs
from gpu_util import assert_close, dev, host, torch

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(3232)
PAIRS = [(0, 0), (1, 0), (0, 1), (1, 1)]


def _cus():
    return torch().cuda.get_device_properties(0).multi_processor_count


def regime(M, N, K, ta, cus):
    """'quarter', 'half', 't48' (64 x 48 tiles of 16 x 16 blocks) or 'full'
    (64 x 64) for an operand layout that takes the direct loads; ta is the
    transpose flag of A (A x-major when not)."""
    cdiv = lambda a, b: -(-a // b)
    t64 = cdiv(M, 64) * cdiv(N, 64)
    t32 = cdiv(M, 32) * cdiv(N, 32)
    tall, wide = cdiv(M, 64) * cdiv(N, 32), cdiv(M, 32) * cdiv(N, 64)
    th = tall if tall < wide or (tall == wide and not ta) else wide
    if 2 * t64 < cus:
        return "quarter" if t32 <= cus else "half"
    share = lambda t: cdiv(t, cus)
    slabs = cdiv(K, 32)
    ks = 4 if t64 <= cus and slabs >= 8 else (2 if slabs >= 4 else 1)
    t48 = cdiv(M, 64) * cdiv(N, 48)
    if ks == 4 and t64 < t48 <= cus:
        return "t48"
    if t64 > cus and 10 * share(t64) >= 6 * share(th):
        return "half"
    return "full"


def _ops(ta, tb, M, N, K, gen):
    return gen((K, M) if ta else (M, K)), gen((N, K) if tb else (K, N))


CASES = [
    # quarter tiles: one to eight k-groups, ragged edges, K tails
    ("quarter", 100, 200, 1028), ("quarter", 33, 68, 36), ("quarter", 132, 36, 100),
    ("quarter", 500, 500, 2000), ("quarter", 256, 256, 256), ("quarter", 4, 4, 4),
    # narrow tiles on a small grid: 64 x 32 (500 rows) and 32 x 64 (348
    # rows) with 1, 2, 4 and 6 k-groups
    ("half", 500, 600, 100), ("half", 348, 772, 772), ("half", 500, 600, 300),
    ("half", 500, 600, 60), ("half", 348, 772, 1540), ("half", 500, 600, 2020),
    ("half", 348, 772, 1249), ("half", 500, 600, 1247),
    # narrow tiles on grids larger than the CUs, K tails in a slab
    ("half", 1000, 1212, 300), ("half", 1024, 1216, 60), ("half", 1280, 2044, 300),
]


@pytest.mark.parametrize("ta,tb", PAIRS)
@pytest.mark.parametrize("want,M,N,K", CASES)
def test_matches_oracle(want, M, N, K, ta, tb):
    assert regime(M, N, K, ta, _cus()) == want
    A, B = _ops(ta, tb, M, N, K, lambda s: inputs.uniform(RNG, s))
    C = inputs.uniform(RNG, (M, N))
    ref, bound = oracle.gemm_ex(A, B, C, 0.75, 1.5, trans_a=bool(ta), trans_b=bool(tb))
    dC = dev(C)
    bd.gemm_f32_ex(dev(A), dev(B), dC, 0.75, 1.5, trans_a=bool(ta), trans_b=bool(tb))
    assert_close(host(dC), ref, bound, "%s t%d%d %dx%dx%d" % (want, ta, tb, M, N, K))


@pytest.mark.parametrize("ta,tb", PAIRS)
@pytest.mark.parametrize("M,N,K", [(1024, 2304, 768), (1280, 2048, 1024)])
def test_transformer_shape_narrow_tiles(ta, tb, M, N, K):
    """1024 x 2304 x 768 (576 tiles of 64 x 64) and 1280 x 2048 x 1024 (640):
    narrow tiles, every element against the oracle, N(0, 1) activations and
    N(0, 0.02) weights."""
    assert regime(M, N, K, ta, _cus()) == "half"
    A = inputs.normal(RNG, (K, M) if ta else (M, K))
    B = (0.02 * inputs.normal(RNG, (N, K) if tb else (K, N))).astype(np.float32)
    ref, bound = oracle.gemm_ex(A, B, None, 1.0, 0.0, trans_a=bool(ta), trans_b=bool(tb))
    got = host(bd.gemm_f32_ex(dev(A), dev(B), None, 1.0, 0.0, trans_a=bool(ta), trans_b=bool(tb)))
    assert_close(got, ref, bound, "%dx%dx%d t%d%d" % (M, N, K, ta, tb))


@pytest.mark.parametrize("ta,tb", PAIRS)
@pytest.mark.parametrize("M,N,K", [(100, 200, 1028), (500, 600, 100), (1280, 2044, 300)])
def test_integer_exact(ta, tb, M, N, K):
    A, B = _ops(ta, tb, M, N, K, lambda s: inputs.integers(RNG, s))
    ref, _ = oracle.gemm_ex(A, B, None, 1.0, 0.0, trans_a=bool(ta), trans_b=bool(tb))
    got = host(bd.gemm_f32_ex(dev(A), dev(B), None, 1.0, 0.0, trans_a=bool(ta), trans_b=bool(tb)))
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("ta,tb", PAIRS)
@pytest.mark.parametrize("M,N,K", [(96, 136, 300), (1280, 2044, 300)])
def test_padded_leading_dimensions(ta, tb, M, N, K):
    """Leading dimensions padded by 4 and 8 floats (16-byte rows kept, so the
    direct loads apply), NaN in the padding, C padded with a canary."""
    t = torch()
    A, B = _ops(ta, tb, M, N, K, lambda s: inputs.uniform(RNG, s))

    def padded(X, extra):
        P = np.full((X.shape[0], X.shape[1] + extra), np.nan, np.float32)
        P[:, :X.shape[1]] = X
        return dev(P)[:, :X.shape[1]]
    dA, dB = padded(A, 8), padded(B, 4)
    Cbuf = t.full((M, N + 4), 5.0, dtype=t.float32, device="cuda")
    bd.gemm_f32_ex(dA, dB, Cbuf[:, :N], 1.0, 0.0, trans_a=bool(ta), trans_b=bool(tb))
    got = host(Cbuf)
    assert np.all(got[:, N:] == 5.0)
    ref, bound = oracle.gemm_ex(A, B, None, 1.0, 0.0, trans_a=bool(ta), trans_b=bool(tb))
    assert_close(got[:, :N], ref, bound, "padded t%d%d %dx%dx%d" % (ta, tb, M, N, K))


@pytest.mark.parametrize("M,N,K", [(500, 500, 2000), (1024, 2304, 768)])
def test_deterministic(M, N, K):
    A = inputs.uniform(RNG, (M, K))
    B = inputs.uniform(RNG, (K, N))
    dA, dB = dev(A), dev(B)
    assert np.array_equal(host(bd.gemm_f32(dA, dB)), host(bd.gemm_f32(dA, dB)))
