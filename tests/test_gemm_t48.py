"""GPU parity of the GEMM's 64 x 48 tiles: 16 x 16 x 4 MFMA blocks, four
waves per k-group stacked along M (16 x 48 each, three accumulators), four
k-groups, taken where 64 x 64 tiles would leave CUs idle and 64 x 48 tiles
still fit one per CU (1,024 x 768 outputs: 256 tiles instead of 192).  A
k-major B tile is staged 64 wide; an x-major one takes six 1 KB loads per
slab over four waves.  All four transpose pairs against the oracle on every
element: the GPT-2 shapes with long K, ragged M and N, K tails inside a slab
(K not a multiple of 4 takes the variant that zeroes a chunk's tail),
alpha/beta, padded leading dimensions, integer exactness and repeat bits."""
import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs
from gpu_util import assert_close, dev, host, torch
from test_gemm_tiles import PAIRS, regime

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(4848)


def _cus():
    return torch().cuda.get_device_properties(0).multi_processor_count


def _ops(ta, tb, M, N, K, gen):
    return gen((K, M) if ta else (M, K)), gen((N, K) if tb else (K, N))


def _check(M, N, K, ta, tb, alpha, beta, gen):
    assert regime(M, N, K, ta, _cus()) == "t48", (M, N, K)
    A, B = _ops(ta, tb, M, N, K, gen)
    C = inputs.uniform(RNG, (M, N)) if beta else None
    ref, bound = oracle.gemm_ex(A, B, C, alpha, beta, trans_a=bool(ta), trans_b=bool(tb))
    dC = dev(C) if beta else None
    got = bd.gemm_f32_ex(dev(A), dev(B), dC, alpha, beta, trans_a=bool(ta), trans_b=bool(tb))
    assert_close(host(got), ref, bound, "t48 t%d%d %dx%dx%d" % (ta, tb, M, N, K))


@pytest.mark.parametrize("ta,tb", PAIRS)
@pytest.mark.parametrize("M,N,K", [(1024, 768, 3072), (1024, 768, 2304), (1024, 768, 256)])
def test_transformer_shapes(ta, tb, M, N, K):
    """N(0, 1) activations against N(0, 0.02) weights, as in a GPT-2 block."""
    _check(M, N, K, ta, tb, 1.0, 0.0,
           lambda s: inputs.normal(RNG, s) if s[0] * s[1] == M * K else
           (0.02 * inputs.normal(RNG, s)).astype(np.float32))


@pytest.mark.parametrize("ta,tb", PAIRS)
@pytest.mark.parametrize("M,N,K", [(1000, 760, 1030), (900, 700, 513), (1024, 720, 260),
                                   (1016, 767, 300)])
def test_ragged_and_k_tails(ta, tb, M, N, K):
    _check(M, N, K, ta, tb, 0.75, 1.5, lambda s: inputs.uniform(RNG, s))


@pytest.mark.parametrize("ta,tb", PAIRS)
def test_integer_exact(ta, tb):
    M, N, K = 1000, 760, 1030
    assert regime(M, N, K, ta, _cus()) == "t48"
    A, B = _ops(ta, tb, M, N, K, lambda s: inputs.integers(RNG, s))
    ref, _ = oracle.gemm_ex(A, B, None, 1.0, 0.0, trans_a=bool(ta), trans_b=bool(tb))
    got = host(bd.gemm_f32_ex(dev(A), dev(B), None, 1.0, 0.0, trans_a=bool(ta), trans_b=bool(tb)))
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("ta,tb", PAIRS)
def test_padded_leading_dimensions(ta, tb):
    """Leading dimensions padded by 8 and 4 floats, NaN in the padding, C
    padded with a canary."""
    t = torch()
    M, N, K = 1000, 760, 600
    assert regime(M, N, K, ta, _cus()) == "t48"
    A, B = _ops(ta, tb, M, N, K, lambda s: inputs.uniform(RNG, s))

    def padded(X, extra):
        P = np.full((X.shape[0], X.shape[1] + extra), np.nan, np.float32)
        P[:, :X.shape[1]] = X
        return dev(P)[:, :X.shape[1]]
    Cbuf = t.full((M, N + 4), 5.0, dtype=t.float32, device="cuda")
    bd.gemm_f32_ex(padded(A, 8), padded(B, 4), Cbuf[:, :N], 1.0, 0.0, trans_a=bool(ta),
                   trans_b=bool(tb))
    got = host(Cbuf)
    assert np.all(got[:, N:] == 5.0)
    ref, bound = oracle.gemm_ex(A, B, None, 1.0, 0.0, trans_a=bool(ta), trans_b=bool(tb))
    assert_close(got[:, :N], ref, bound, "padded t%d%d" % (ta, tb))


def test_repeat_bits():
    M, N, K = 1024, 768, 3072
    A = inputs.uniform(RNG, (M, K))
    B = inputs.uniform(RNG, (K, N))
    dA, dB = dev(A), dev(B)
    assert np.array_equal(host(bd.gemm_f32(dA, dB)), host(bd.gemm_f32(dA, dB)))


def _placed(a, offset, pad):
    """Device copy of 2-D float32 array a, `offset` floats into a NaN-filled
    buffer, with `pad` extra floats per row."""
    t = torch()
    rows, cols = a.shape
    ld = cols + pad
    buf = t.full((offset + rows * ld,), float("nan"), dtype=t.float32, device="cuda")
    view = buf[offset:offset + rows * ld].view(rows, ld)[:, :cols]
    view.copy_(t.from_numpy(np.ascontiguousarray(a)).to("cuda"))
    return view


@pytest.mark.parametrize("seed", range(24))
def test_random_cases(seed):
    """Seeded shapes drawn until the launcher's rule takes 64 x 48 tiles:
    random transpose pairs, K with tails, base offsets of 1 to 4 floats,
    padded leading dimensions and alpha/beta."""
    rng = np.random.default_rng(48000 + seed)
    cus = _cus()
    while True:
        M, N = int(rng.integers(500, 1100)), int(rng.integers(300, 1000))
        K = int(rng.integers(256, 1000))
        ta, tb = (bool(v) for v in rng.integers(0, 2, 2))
        if regime(M, N, K, ta, cus) == "t48":
            break
    alpha, beta = (float(v) for v in rng.choice([1.0, -1.5, 0.5], 2))
    A = inputs.uniform(rng, (K, M) if ta else (M, K))
    B = inputs.uniform(rng, (N, K) if tb else (K, N))
    C = inputs.uniform(rng, (M, N))
    oa, ob, oc = (int(v) for v in rng.choice([0, 4, 1, 3], 3))
    pa, pb, pc = (int(v) for v in rng.choice([0, 4, 8, 5], 3))
    dA, dB, dC = _placed(A, oa, pa), _placed(B, ob, pb), _placed(C, oc, pc)
    bd.gemm_f32_ex(dA, dB, dC, alpha, beta, trans_a=ta, trans_b=tb)
    ref, bound = oracle.gemm_ex(A, B, C, alpha, beta, trans_a=ta, trans_b=tb)
    assert_close(host(dC), ref, bound,
                 "seed %d: %s%s %dx%dx%d offsets %d/%d/%d pads %d/%d/%d"
                 % (seed, "T" if ta else "N", "T" if tb else "N", M, N, K, oa, ob, oc, pa, pb, pc))
