"""GPU parity of the GEMM's direct loads on operands whose rows are not
16-byte aligned: widths, K and leading dimensions that are not multiples of
4 floats, and bases offset by 1 to 3 floats inside NaN-filled buffers.  The
16-byte loads then straddle rows, a chunk can run past K (its part past K is
zeroed in LDS) or past the operand's last element (the buffer's range
check reads zeros there).  Every tile regime (32 x 32, narrow, 64 x 64 with
four or two k-groups), all four transpose pairs, against the oracle on
every element; integer inputs bit for bit; and the vocabulary-sized GPT-2
output projection (N = 50,257) sampled."""
import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs
from gpu_util import assert_close, host, torch

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(4097)
PAIRS = [(0, 0), (1, 0), (0, 1), (1, 1)]


def _placed(X, shift, extra):
    """X inside a NaN-filled device buffer: base offset by `shift` floats,
    leading dimension widened by `extra` floats."""
    t = torch()
    rows, cols = X.shape
    ld = cols + extra
    buf = t.full((shift + rows * ld + 8,), float("nan"), dtype=t.float32, device="cuda")
    view = buf[shift:shift + rows * ld].view(rows, ld)[:, :cols]
    view.copy_(t.from_numpy(np.ascontiguousarray(X)))
    return view


def _ops(ta, tb, M, N, K, gen):
    return gen((K, M) if ta else (M, K)), gen((N, K) if tb else (K, N))


SHAPES = [
    (346, 346, 767),     # 32 x 32 tiles, 8 k-groups
    (33, 47, 1025),      # 32 x 32 tiles, 8 k-groups
    (130, 2, 7),         # K below one slab and below one chunk
    (1, 1, 3),           # one element
    (501, 610, 301),     # narrow tiles on a small grid, 4 k-groups
    (349, 770, 771),     # narrow tiles on a small grid, 4 k-groups
    (349, 770, 1539),    # narrow tiles on a small grid, 6 k-groups
    (1023, 767, 1031),   # 64 x 64 tiles, 4 k-groups
    (2049, 2047, 131),   # 64 x 64 tiles, 2 k-groups
    (1025, 2301, 259),   # narrow tiles past the CU count
]


@pytest.mark.parametrize("ta,tb", PAIRS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_odd_shapes(ta, tb, M, N, K):
    A, B = _ops(ta, tb, M, N, K, lambda s: inputs.uniform(RNG, s))
    C = inputs.uniform(RNG, (M, N))
    ref, bound = oracle.gemm_ex(A, B, C, 1.25, 0.5, trans_a=bool(ta), trans_b=bool(tb))
    dC = _placed(C, 3, 1)
    bd.gemm_f32_ex(_placed(A, 1, 3), _placed(B, 2, 5), dC, 1.25, 0.5,
                   trans_a=bool(ta), trans_b=bool(tb))
    assert_close(host(dC), ref, bound, "t%d%d %dx%dx%d" % (ta, tb, M, N, K))


@pytest.mark.parametrize("ta,tb", PAIRS)
@pytest.mark.parametrize("shift", [1, 2, 3])
def test_integer_exact_offsets(ta, tb, shift):
    M, N, K = 301, 259, 1031
    A, B = _ops(ta, tb, M, N, K, lambda s: inputs.integers(RNG, s))
    ref, _ = oracle.gemm_ex(A, B, None, 1.0, 0.0, trans_a=bool(ta), trans_b=bool(tb))
    got = host(bd.gemm_f32_ex(_placed(A, shift, 0), _placed(B, 4 - shift, 0), None, 1.0, 0.0,
                              trans_a=bool(ta), trans_b=bool(tb)))
    assert np.array_equal(got.astype(np.float64), ref)


def test_same_bits_as_aligned_copy():
    """The same product from 16-byte aligned and from offset operands: the
    loads differ, the arithmetic does not."""
    M, N, K = 700, 900, 1200
    A = inputs.uniform(RNG, (M, K))
    B = inputs.uniform(RNG, (K, N))
    t = torch()
    c1 = host(bd.gemm_f32(t.from_numpy(A).to("cuda"), t.from_numpy(B).to("cuda")))
    c2 = host(bd.gemm_f32(_placed(A, 1, 0), _placed(B, 3, 0)))
    assert np.array_equal(c1, c2)


def test_vocabulary_projection_sampled():
    """1,024 tokens x 768 times 768 x 50,257 (GPT-2's output projection):
    sampled cells, the last columns included."""
    M, K, N = 1024, 768, 50257
    A = inputs.normal(RNG, (M, K))
    B = inputs.normal(RNG, (K, N), 0.02)
    t = torch()
    C = host(bd.gemm_f32(t.from_numpy(A).to("cuda"), t.from_numpy(B).to("cuda")))
    rows = np.concatenate([RNG.integers(0, M, 1500), [0, M - 1, M - 1, 0]])
    cols = np.concatenate([RNG.integers(0, N, 1500), [0, N - 1, N - 2, N - 3]])
    ref, bound = oracle.gemm_cells(A, B, rows, cols)
    assert_close(C[rows, cols], ref, bound, "1024x50257x768")
    assert np.all(np.isfinite(C))
