"""GPU parity of gemm_f32, gemm_f32_tn and gemm_f32_nt against the CPU oracle.

Every call goes through the C ABI (via the ctypes binding).  Acceptance per
element: |gpu - ref| <= 1e-4 * sum_k |a_ik b_kj|; integer-valued inputs must
match bit for bit, since every partial sum is then exact in fp32.
"""
import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs
from golden_io import load
from gpu_util import assert_close, canaries_intact, dev, guarded, host, oracle_product, torch

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(77)

# layout -> (binding function, oracle function, stored A shape, stored B shape)
LAYOUTS = {
    "nn": (bd.gemm_f32, oracle.gemm_nn, lambda M, K: (M, K), lambda K, N: (K, N)),
    "tn": (bd.gemm_f32_tn, oracle.gemm_tn, lambda M, K: (K, M), lambda K, N: (K, N)),
    "nt": (bd.gemm_f32_nt, oracle.gemm_nt, lambda M, K: (M, K), lambda K, N: (N, K)),
}


def _run(layout, A, B, **kw):
    f = LAYOUTS[layout][0]
    return host(f(dev(A), dev(B), **kw))


def _operands(layout, M, N, K, gen):
    _, _, sa, sb = LAYOUTS[layout]
    return gen(sa(M, K)), gen(sb(K, N))


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
def test_tiny_hand_case(layout):
    g = load("gemm_tiny_3x4x2.txt")
    A = np.asarray(g["A"], np.float64).astype(np.float32)
    B = np.asarray(g["B"], np.float64).astype(np.float32)
    C = np.asarray(g["C"], np.float64).astype(np.float32)
    if layout == "tn":
        A = np.ascontiguousarray(A.T)
    if layout == "nt":
        B = np.ascontiguousarray(B.T)
    assert np.array_equal(_run(layout, A, B), C)


INT_SHAPES = [(1, 1, 1), (3, 2, 4), (128, 128, 16), (129, 127, 33), (256, 256, 256),
              (300, 70, 515), (64, 1, 1000), (1, 200, 77), (1024, 768, 3072)]


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
@pytest.mark.parametrize("M,N,K", INT_SHAPES)
def test_integer_inputs_bitwise(layout, M, N, K):
    A, B = _operands(layout, M, N, K, lambda s: inputs.integers(RNG, s))
    C = _run(layout, A, B)
    if M * N * K > 50_000_000:     # sampled cells for the large shape
        rows = RNG.integers(0, M, 4000)
        cols = RNG.integers(0, N, 4000)
        ref, _ = oracle.gemm_cells(A, B, rows, cols, trans_a=layout == "tn",
                                   trans_b=layout == "nt")
        assert np.array_equal(C[rows, cols].astype(np.float64), ref)
    else:
        ref, _ = LAYOUTS[layout][1](A, B)
        assert np.array_equal(C.astype(np.float64), ref)


ODD = [1, 2, 3, 31, 33, 127, 129, 346]


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
@pytest.mark.parametrize("M,N,K", [(m, n, k) for m, n, k in
                                   zip(ODD, ODD[::-1], [5, 129, 2050, 1, 33, 127, 2, 346])] +
                         [(346, 768, 768), (33, 2050, 31), (2050, 3, 129)])
def test_odd_shapes(layout, M, N, K):
    A, B = _operands(layout, M, N, K, lambda s: inputs.uniform(RNG, s))
    C = _run(layout, A, B)
    ref, bound = LAYOUTS[layout][1](A, B)
    assert_close(C, ref, bound, "%s %dx%dx%d" % (layout, M, N, K))


# Operands whose base, leading dimension and contiguous extent are multiples
# of 4 floats take the global -> LDS direct path: K tails of 4..28 columns,
# M and N edges, the 64 x 64 and the 128 x 64 grids (2048 x 2048 gives every
# CU two 128 x 64 tiles).
DIRECT_SHAPES = [(4, 4, 4), (132, 68, 36), (260, 196, 100), (68, 1028, 60), (1028, 132, 292),
                 (8, 2052, 4), (2048, 2048, 100)]


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
@pytest.mark.parametrize("M,N,K", DIRECT_SHAPES)
def test_direct_path_integer_bitwise(layout, M, N, K):
    A, B = _operands(layout, M, N, K, lambda s: inputs.integers(RNG, s))
    C = _run(layout, A, B)
    ref, _ = LAYOUTS[layout][1](A, B)
    assert np.array_equal(C.astype(np.float64), ref), "%s %dx%dx%d" % (layout, M, N, K)


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
def test_direct_path_padded_leading_dims(layout):
    # aligned column slices of wider buffers: ld > row width, 16-byte aligned
    M, N, K = 196, 132, 68
    A, B = _operands(layout, M, N, K, lambda s: inputs.uniform(RNG, s))
    Aw = np.full((A.shape[0], A.shape[1] + 12), np.float32(3e30))
    Aw[:, 4:4 + A.shape[1]] = A
    Bw = np.full((B.shape[0], B.shape[1] + 8), np.float32(-3e30))
    Bw[:, 8:8 + B.shape[1]] = B
    dA, dB = dev(Aw)[:, 4:4 + A.shape[1]], dev(Bw)[:, 8:8 + B.shape[1]]
    buf, _ = guarded(M, N + 4)
    Cw = buf[64:64 + M * (N + 4)].view(M, N + 4)
    C = Cw[:, :N]
    LAYOUTS[layout][0](dA, dB, C=C)
    ref, bound = LAYOUTS[layout][1](A, B)
    assert_close(host(C), ref, bound, layout + " aligned padded")
    assert np.all(host(Cw)[:, N:] == np.float32(1.2345e9)), "wrote outside C's columns"
    assert canaries_intact(buf), "wrote outside C"


def test_small_square_config():
    # 256^3, A then B uniform [-1, 1) from seed 0
    A, B = inputs.small_square(0)
    C = _run("nn", A, B)
    ref, bound = oracle.gemm_nn(A, B)
    assert_close(C, ref, bound, "256^3")


def test_classifier_config():
    A, B = inputs.classifier(33)
    C = _run("nn", A, B)
    ref, bound = oracle.gemm_nn(A, B)
    assert_close(C, ref, bound, "346x768x768")


def _sample_cells(M, N, n=3000):
    rows = np.concatenate([RNG.integers(0, M, n), [0, 0, M - 1, M - 1]])
    cols = np.concatenate([RNG.integers(0, N, n), [0, N - 1, 0, N - 1]])
    return rows, cols


def test_large_square_config_every_cell():
    """The 2048^3 configuration, every cell against the oracle's whole
    product (split over the host's cores)."""
    A, B = inputs.large_square(3)
    C = _run("nn", A, B)
    ref, bound = oracle_product("nn", A, B)
    assert_close(C, ref, bound, "2048^3")
    assert np.all(np.isfinite(C))


def test_large_square_config_sampled_cells():
    """The same product against cells the oracle computes one by one, a check
    of the split above."""
    A, B = inputs.large_square(3)
    C = _run("nn", A, B)
    rows, cols = _sample_cells(2048, 2048)
    ref, bound = oracle.gemm_cells(A, B, rows, cols)
    assert_close(C[rows, cols], ref, bound, "2048^3")


@pytest.mark.parametrize("op", [o[0] for o in inputs.GPT2_OPS])
def test_gpt2_layer_products_every_cell(op):
    t = _gpt2()
    name, layout, M, N, K, (an, bn) = next(o for o in inputs.GPT2_OPS if o[0] == op)
    A, B = t[an], t[bn]
    C = _run(layout, A, B)
    assert C.shape == (M, N)
    ref, bound = oracle_product(layout, A, B)
    assert_close(C, ref, bound, op)


_GPT2 = {}


def _gpt2():
    if not _GPT2:
        _GPT2.update(inputs.gpt2_tensors(2))
    return _GPT2


def test_identity():
    A = inputs.uniform(RNG, (200, 130))
    I = np.eye(130, dtype=np.float32)
    assert np.array_equal(_run("nn", A, I), A)
    assert np.array_equal(_run("nn", np.eye(200, dtype=np.float32), A), A)
    assert np.array_equal(_run("nt", A, I), A)


def test_transpose_identity():
    # (A.B)^T = B^T.A^T through all three entry points
    A = inputs.uniform(RNG, (150, 260))
    B = inputs.uniform(RNG, (260, 90))
    ab = _run("nn", A, B)
    # tn with B as the K x M' operand and A^T as the K x N' one gives B^T.A^T
    bt_at_tn = _run("tn", B, np.ascontiguousarray(A.T))
    bt_at_nt = _run("nt", np.ascontiguousarray(B.T), A)
    ref, bound = oracle.gemm_nn(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    assert_close(bt_at_tn, ref, bound, "tn")
    assert_close(bt_at_nt, ref, bound, "nt")
    assert_close(ab.T, ref, bound, "nn^T")


def test_power_of_two_scaling_bitwise():
    A = inputs.uniform(RNG, (300, 200))
    B = inputs.uniform(RNG, (200, 170))
    c1 = _run("nn", A, B)
    c4 = _run("nn", A * np.float32(4), B)
    assert np.array_equal(c4, c1 * np.float32(4))


def test_linearity():
    A = inputs.uniform(RNG, (160, 300))
    B1 = inputs.uniform(RNG, (300, 140))
    B2 = inputs.uniform(RNG, (300, 140))
    c12 = _run("nn", A, B1 + B2).astype(np.float64)
    c1 = _run("nn", A, B1).astype(np.float64)
    c2 = _run("nn", A, B2).astype(np.float64)
    _, b1 = oracle.gemm_nn(A, B1)
    _, b2 = oracle.gemm_nn(A, B2)
    assert np.all(np.abs(c12 - c1 - c2) <= 3e-4 * (b1 + b2))


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
def test_deterministic(layout):
    A, B = _operands(layout, 700, 500, 900, lambda s: inputs.uniform(RNG, s))
    assert np.array_equal(_run(layout, A, B), _run(layout, A, B))


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
def test_padded_leading_dims_and_canaries(layout):
    t = torch()
    M, N, K = 130, 75, 93
    A, B = _operands(layout, M, N, K, lambda s: inputs.uniform(RNG, s))
    # operands as column slices of wider buffers (ld > row width; the odd
    # offsets also take the scalar-load specialisation)
    Aw = np.zeros((A.shape[0], A.shape[1] + 9), np.float32)
    Aw[:, 3:3 + A.shape[1]] = A
    Bw = np.zeros((B.shape[0], B.shape[1] + 5), np.float32)
    Bw[:, 1:1 + B.shape[1]] = B
    dA, dB = dev(Aw)[:, 3:3 + A.shape[1]], dev(Bw)[:, 1:1 + B.shape[1]]
    buf, _ = guarded(M, N + 7)
    Cw = buf[64:64 + M * (N + 7)].view(M, N + 7)
    C = Cw[:, :N]
    LAYOUTS[layout][0](dA, dB, C=C)
    got = host(C)
    ref, bound = LAYOUTS[layout][1](A, B)
    assert_close(got, ref, bound, layout + " padded")
    pad_cols = host(Cw)[:, N:]
    assert np.all(pad_cols == np.float32(1.2345e9)), "wrote outside C's columns"
    assert canaries_intact(buf), "wrote outside C"


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
def test_k_zero_writes_zeros(layout):
    t = torch()
    M, N = 70, 45
    _, _, sa, sb = LAYOUTS[layout]
    A = t.empty(sa(M, 0), dtype=t.float32, device="cuda")
    B = t.empty(sb(0, N), dtype=t.float32, device="cuda")
    C = t.full((M, N), 7.0, dtype=t.float32, device="cuda")
    LAYOUTS[layout][0](A, B, C=C)
    assert np.all(host(C) == 0.0)


def test_large_magnitudes_stay_finite():
    # |a|, |b| <= 1e17 and K = 3072: |c| <= 3.1e37 < FLT_MAX
    A = (inputs.uniform(RNG, (64, 3072)) * np.float32(1e17)).astype(np.float32)
    B = (inputs.uniform(RNG, (3072, 64)) * np.float32(1e17)).astype(np.float32)
    C = _run("nn", A, B)
    assert np.all(np.isfinite(C))
    ref, bound = oracle.gemm_nn(A, B)
    assert_close(C, ref, bound, "large magnitudes")


def test_status_errors_raise():
    t = torch()
    A = t.zeros((4, 4), dtype=t.float32, device="cuda")
    with pytest.raises(bd.GGError) as e:
        bd.gemm_f32(A, A, C=A)          # output aliases the inputs
    assert e.value.status == bd.GG_ERR_ALIAS
