"""Pins for the CPU oracle: each check ties it to something other than itself.

* hand-worked cases from tests/golden/ (dense product, one-row product, 2-bit
  product with the packing readings written out);
* numpy's float64 matrix product (a library routine) on random and ragged
  shapes, for all three operand layouts;
* exact arithmetic: integer inputs (numpy int64) and dyadic rationals
  (Python ``fractions``) where every correct summation order gives the same
  value;
* identities: A.I = A, (A.B)^T = B^T.A^T across the layouts, linearity;
* the binary16 decoder against numpy on all 65,536 bit patterns;
* the 2-bit path against a packer written independently in this file.

A plausible slip in the oracle (a transposed operand, a dropped term, a
wrong sign or bit order, a wrong scale index) fails at least one of these.
"""
import fractions
import itertools

import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import inputs
from golden_io import load

RNG = np.random.default_rng(1234)


def _f32(a):
    return np.asarray(a, dtype=np.float64).astype(np.float32)


# ------------------------------------------------------ hand-worked cases --

def test_gemm_tiny_golden():
    g = load("gemm_tiny_3x4x2.txt")
    A, B, C = _f32(g["A"]), _f32(g["B"]), np.asarray(g["C"], np.float64)
    c, b = oracle.gemm_nn(A, B)
    assert np.array_equal(c, C)
    # same product through the transposed storage layouts
    c_tn, _ = oracle.gemm_tn(np.ascontiguousarray(A.T), B)
    c_nt, _ = oracle.gemm_nt(A, np.ascontiguousarray(B.T))
    assert np.array_equal(c_tn, C) and np.array_equal(c_nt, C)
    # bound is sum |a*b|: row 0 col 1 = |0|+|2|+|3|+|-4| = 9
    assert b[0, 1] == 9.0 and b[0, 0] == 12.0


def test_generator_tiny_case_matches_golden():
    g = load("gemm_tiny_3x4x2.txt")
    A, B = inputs.tiny_case()
    assert np.array_equal(A, _f32(g["A"])) and np.array_equal(B, _f32(g["B"]))


def test_gemv_tiny_golden():
    g = load("gemv_tiny_3x4.txt")
    W, x = _f32(g["W"]), _f32(g["x"])[0]
    y, b = oracle.gemv(W, x)
    assert np.array_equal(y, np.asarray(g["y"], np.float64)[0])
    assert np.array_equal(b, y)          # all products are >= 0 here


def test_q2_tiny_golden():
    g = load("q2_tiny_2x4.txt")
    Q = np.array(g["Q"], dtype=np.uint8)
    S = np.array(g["S"], dtype=np.uint16)
    x = _f32(g["x"])[0]
    y, b = oracle.gemv_q2(Q, S, x)
    assert np.array_equal(y, np.asarray(g["y"], np.float64)[0])
    W = oracle.q2_unpack(Q, S, 4)
    assert np.array_equal(W, [[-0.75, -0.25, 0.25, 0.75], [3, 3, -3, -3]])
    assert np.array_equal(b, np.abs(W) @ np.abs(x.astype(np.float64)))


def test_q4_tiny_golden():
    g = load("q4_tiny_2x4.txt")
    Q = np.array(g["Q"], dtype=np.uint8)
    S = np.array(g["S"], dtype=np.uint16)
    x = _f32(g["x"])[0]
    y, b = oracle.gemv_q4(Q, S, x)
    assert np.array_equal(y, np.asarray(g["y"], np.float64)[0])
    W = oracle.q4_unpack(Q, S, 4)
    assert np.array_equal(W, [[-3.75, -3.25, -0.25, 3.75], [15, 1, 9, -9]])
    assert np.array_equal(b, np.abs(W) @ np.abs(x.astype(np.float64)))


# ------------------------------------------------------- library routine --

SHAPES = [(1, 1, 1), (1, 7, 3), (5, 1, 9), (3, 4, 2), (17, 33, 31),
          (64, 64, 64), (31, 2, 64), (2, 63, 1), (40, 9, 0)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_matches_numpy(M, N, K):
    A = inputs.uniform(RNG, (M, K))
    B = inputs.uniform(RNG, (K, N))
    ref = A.astype(np.float64) @ B.astype(np.float64)
    ref_abs = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
    for c, b in (oracle.gemm_nn(A, B),
                 oracle.gemm_tn(np.ascontiguousarray(A.T), B),
                 oracle.gemm_nt(A, np.ascontiguousarray(B.T))):
        assert c.shape == (M, N)
        np.testing.assert_allclose(c, ref, rtol=0, atol=1e-12 * max(1, K))
        np.testing.assert_allclose(b, ref_abs, rtol=1e-13, atol=0)
        assert np.all(np.abs(c) <= b * (1 + 1e-12))


def test_gemm_strided_operands():
    # a view with a leading dimension larger than its width
    big_a = inputs.uniform(RNG, (20, 50))
    big_b = inputs.uniform(RNG, (30, 40))
    A, B = big_a[:, 5:35], big_b[:, 3:20]
    c, _ = oracle.gemm_nn(A, B)
    np.testing.assert_allclose(
        c, A.astype(np.float64) @ B.astype(np.float64), rtol=0, atol=1e-12)


@pytest.mark.parametrize("M,K", [(1, 1), (7, 3), (12, 64), (5, 130), (3, 0)])
def test_gemv_matches_numpy(M, K):
    W = inputs.normal(RNG, (M, K))
    x = inputs.normal(RNG, (K,))
    y, b = oracle.gemv(W, x)
    np.testing.assert_allclose(
        y, W.astype(np.float64) @ x.astype(np.float64), rtol=0, atol=1e-12)
    np.testing.assert_allclose(
        b, np.abs(W.astype(np.float64)) @ np.abs(x.astype(np.float64)),
        rtol=1e-13)


# ------------------------------------------------------ exact arithmetic --

def test_gemm_integer_exact():
    # integer entries in [-8, 8]: every partial sum is an integer far below
    # 2^53, so the fp64 result must equal the integer product exactly
    A = inputs.integers(RNG, (37, 300))
    B = inputs.integers(RNG, (300, 29))
    ref = A.astype(np.int64) @ B.astype(np.int64)
    c, _ = oracle.gemm_nn(A, B)
    assert np.array_equal(c, ref.astype(np.float64))
    c, _ = oracle.gemm_tn(np.ascontiguousarray(A.T), B)
    assert np.array_equal(c, ref.astype(np.float64))
    c, _ = oracle.gemm_nt(A, np.ascontiguousarray(B.T))
    assert np.array_equal(c, ref.astype(np.float64))


def test_gemm_brute_force_rationals():
    # dyadic entries j/8: exact in fp32 and fp64; brute-force the definition
    # with exact rationals and compare bit for bit
    M, N, K = 4, 3, 5
    A = (RNG.integers(-16, 17, (M, K)) / 8).astype(np.float32)
    B = (RNG.integers(-16, 17, (K, N)) / 8).astype(np.float32)
    c, b = oracle.gemm_nn(A, B)
    for i, j in itertools.product(range(M), range(N)):
        s = sum(fractions.Fraction(float(A[i, k])) * fractions.Fraction(float(B[k, j]))
                for k in range(K))
        t = sum(abs(fractions.Fraction(float(A[i, k])) * fractions.Fraction(float(B[k, j])))
                for k in range(K))
        assert c[i, j] == float(s) and b[i, j] == float(t)


def test_q2_integer_exact():
    # scale 2.0 and integer x: every weight is an odd integer in [-3, 3], so
    # the product is an exact integer
    M, K = 9, 256
    codes = RNG.integers(0, 4, (M, K))
    Q = _pack_codes(codes)
    S = np.full((M, K // 64), 0x4000, np.uint16)
    x = inputs.integers(RNG, (K,))
    y, _ = oracle.gemv_q2(Q, S, x)
    ref = (2 * codes - 3) @ x.astype(np.int64)
    assert np.array_equal(y, ref.astype(np.float64))


# ------------------------------------------------------------ identities --

def test_identity_matrix():
    A = inputs.uniform(RNG, (23, 41))
    c, _ = oracle.gemm_nn(A, np.eye(41, dtype=np.float32))
    assert np.array_equal(c, A.astype(np.float64))
    c, _ = oracle.gemm_nn(np.eye(23, dtype=np.float32), A)
    assert np.array_equal(c, A.astype(np.float64))


def test_transpose_identity():
    # (A.B)^T = B^T.A^T: the same products in the same k order, so bitwise
    A = inputs.uniform(RNG, (19, 27))
    B = inputs.uniform(RNG, (27, 13))
    ab, _ = oracle.gemm_nn(A, B)
    bt_at, _ = oracle.gemm_nn(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    assert np.array_equal(ab.T, bt_at)
    # B^T.A^T through the transposed layouts, storing B and A untransposed
    c_tn, _ = oracle.gemm_tn(B, np.ascontiguousarray(A.T))
    c_nt, _ = oracle.gemm_nt(np.ascontiguousarray(B.T), A)
    assert np.array_equal(c_tn, bt_at) and np.array_equal(c_nt, bt_at)


def test_linearity():
    A = inputs.uniform(RNG, (11, 20))
    B1 = (RNG.integers(-64, 65, (20, 7)) / 64).astype(np.float32)
    B2 = (RNG.integers(-64, 65, (20, 7)) / 64).astype(np.float32)
    c12, b12 = oracle.gemm_nn(A, B1 + B2)          # B1 + B2 exact in fp32
    c1, b1 = oracle.gemm_nn(A, B1)
    c2, b2 = oracle.gemm_nn(A, B2)
    assert np.all(np.abs(c12 - (c1 + c2)) <= 1e-13 * (b1 + b2 + b12))
    # exact power-of-two scaling
    c4, _ = oracle.gemm_nn(A * np.float32(4), B1)
    assert np.array_equal(c4, 4 * c1)


def test_cells_match_full_product():
    A = inputs.uniform(RNG, (30, 50))
    B = inputs.uniform(RNG, (50, 40))
    full, fb = oracle.gemm_nn(A, B)
    rows = RNG.integers(0, 30, 25)
    cols = RNG.integers(0, 40, 25)
    c, b = oracle.gemm_cells(A, B, rows, cols)
    assert np.array_equal(c, full[rows, cols]) and np.array_equal(b, fb[rows, cols])
    c, _ = oracle.gemm_cells(np.ascontiguousarray(A.T), B, rows, cols, trans_a=True)
    assert np.array_equal(c, full[rows, cols])
    c, _ = oracle.gemm_cells(A, np.ascontiguousarray(B.T), rows, cols, trans_b=True)
    assert np.array_equal(c, full[rows, cols])
    with pytest.raises(ValueError):
        oracle.gemm_cells(A, B, [30], [0])


# --------------------------------------------------------------- binary16 --

def test_half_decoder_exhaustive():
    patterns = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = patterns.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(h)) for h in patterns])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signs of zero survive
    assert np.signbit(oracle.half_to_double(0x8000))


# --------------------------------------------------------------- 2-bit ---

def _pack_codes(codes):
    """Independent packer: codes (M x K, values 0..3) -> bytes with column
    4q+t in bits 2t..2t+1 of byte q; unused bits of a last partial byte are
    left zero."""
    M, K = codes.shape
    nb = (K + 3) // 4
    padded = np.zeros((M, nb * 4), np.uint16)
    padded[:, :K] = codes
    q = padded.reshape(M, nb, 4)
    return (q[..., 0] | (q[..., 1] << 2) | (q[..., 2] << 4) |
            (q[..., 3] << 6)).astype(np.uint8)


def _dequant_numpy(codes, S):
    M, K = codes.shape
    s = S.view(np.float16).astype(np.float64)
    s_full = np.repeat(s, 64, axis=1)[:, :K]
    return (codes.astype(np.float64) - 1.5) * s_full


@pytest.mark.parametrize("M,K", [(1, 64), (5, 1536), (7, 100), (3, 5), (4, 1)])
def test_q2_matches_independent_packer(M, K):
    codes = RNG.integers(0, 4, (M, K))
    Q = _pack_codes(codes)
    S = RNG.uniform(0.01, 0.05, (M, (K + 63) // 64)).astype(np.float16).view(np.uint16)
    x = inputs.normal(RNG, (K,))
    W = _dequant_numpy(codes, S)
    assert np.array_equal(oracle.q2_unpack(Q, S, K), W)
    y, b = oracle.gemv_q2(Q, S, x)
    np.testing.assert_allclose(y, W @ x.astype(np.float64), rtol=0, atol=1e-13)
    np.testing.assert_allclose(b, np.abs(W) @ np.abs(x.astype(np.float64)), rtol=1e-13)


def test_q2_padding_is_ignored():
    # K = 70: the last byte holds 2 live columns and 2 dead ones; the second
    # scale group is partial; the row strides carry extra garbage
    M, K = 6, 70
    codes = RNG.integers(0, 4, (M, K))
    Q = _pack_codes(codes)
    S = RNG.uniform(0.01, 0.05, (M, 2)).astype(np.float16).view(np.uint16)
    x = inputs.normal(RNG, (K,))
    y, _ = oracle.gemv_q2(Q, S, x)
    Qg = RNG.integers(0, 256, (M, Q.shape[1] + 5)).astype(np.uint8)
    Qg[:, :Q.shape[1]] = Q
    Qg[:, Q.shape[1] - 1] |= np.uint8(0b11110000)     # dead columns 70, 71
    Sg = RNG.integers(0, 65536, (M, 4)).astype(np.uint16)
    Sg[:, :2] = S
    y2, _ = oracle.gemv_q2(Qg[:, :Q.shape[1] + 5], Sg, x, K=K)
    assert np.array_equal(y, y2)


def test_q2_scale_doubling():
    M, K = 4, 192
    Q, S = inputs.q2_weight(0, M, K)
    x = inputs.normal(RNG, (K,))
    y, _ = oracle.gemv_q2(Q, S, x)
    S2 = (S.view(np.float16) * np.float16(2)).view(np.uint16)
    y2, _ = oracle.gemv_q2(Q, S2, x)
    assert np.array_equal(y2, 2 * y)


def _pack_nibbles(codes):
    """Independent packer: column 2q+t in bits 4t..4t+3 of byte q."""
    M, K = codes.shape
    nb = (K + 1) // 2
    padded = np.zeros((M, nb * 2), np.uint16)
    padded[:, :K] = codes
    q = padded.reshape(M, nb, 2)
    return (q[..., 0] | (q[..., 1] << 4)).astype(np.uint8)


def _dequant4_numpy(codes, S):
    M, K = codes.shape
    s = S.view(np.float16).astype(np.float64)
    s_full = np.repeat(s, 64, axis=1)[:, :K]
    return (codes.astype(np.float64) - 7.5) * s_full


def test_q4_integer_exact():
    # scale 2.0 and integer x: every weight is an odd integer in [-15, 15]
    M, K = 9, 256
    codes = RNG.integers(0, 16, (M, K))
    Q = _pack_nibbles(codes)
    S = np.full((M, K // 64), 0x4000, np.uint16)
    x = inputs.integers(RNG, (K,))
    y, _ = oracle.gemv_q4(Q, S, x)
    ref = (2 * codes - 15) @ x.astype(np.int64)
    assert np.array_equal(y, ref.astype(np.float64))


@pytest.mark.parametrize("M,K", [(1, 64), (5, 1536), (7, 100), (3, 5), (4, 1)])
def test_q4_matches_independent_packer(M, K):
    codes = RNG.integers(0, 16, (M, K))
    Q = _pack_nibbles(codes)
    S = RNG.uniform(0.01, 0.05, (M, (K + 63) // 64)).astype(np.float16).view(np.uint16)
    x = inputs.normal(RNG, (K,))
    W = _dequant4_numpy(codes, S)
    assert np.array_equal(oracle.q4_unpack(Q, S, K), W)
    y, b = oracle.gemv_q4(Q, S, x)
    np.testing.assert_allclose(y, W @ x.astype(np.float64), rtol=0, atol=1e-13)
    np.testing.assert_allclose(b, np.abs(W) @ np.abs(x.astype(np.float64)), rtol=1e-13)


def test_q4_padding_is_ignored():
    # K = 71: the last byte holds 1 live column and 1 dead one; the second
    # scale group is partial; the row strides carry extra garbage
    M, K = 6, 71
    codes = RNG.integers(0, 16, (M, K))
    Q = _pack_nibbles(codes)
    S = RNG.uniform(0.01, 0.05, (M, 2)).astype(np.float16).view(np.uint16)
    x = inputs.normal(RNG, (K,))
    y, _ = oracle.gemv_q4(Q, S, x)
    Qg = RNG.integers(0, 256, (M, Q.shape[1] + 5)).astype(np.uint8)
    Qg[:, :Q.shape[1]] = Q
    Qg[:, Q.shape[1] - 1] |= np.uint8(0xF0)          # dead column 71
    Sg = RNG.integers(0, 65536, (M, 4)).astype(np.uint16)
    Sg[:, :2] = S
    y2, _ = oracle.gemv_q4(Qg[:, :Q.shape[1] + 5], Sg, x, K=K)
    assert np.array_equal(y, y2)


def test_q4_scale_doubling():
    M, K = 4, 192
    Q, S = inputs.q4_weight(0, M, K)
    x = inputs.normal(RNG, (K,))
    y, _ = oracle.gemv_q4(Q, S, x)
    S2 = (S.view(np.float16) * np.float16(2)).view(np.uint16)
    y2, _ = oracle.gemv_q4(Q, S2, x)
    assert np.array_equal(y2, 2 * y)


def test_q4_agrees_with_q2_on_shared_levels():
    # codes 6..9 of the 4-bit format are the levels -1.5..1.5 of the 2-bit
    # one: (c4 - 7.5) = (c2 - 1.5) with c4 = c2 + 6
    M, K = 5, 130
    c2 = RNG.integers(0, 4, (M, K))
    S = RNG.uniform(0.01, 0.05, (M, 3)).astype(np.float16).view(np.uint16)
    x = inputs.normal(RNG, (K,))
    y2, b2 = oracle.gemv_q2(_pack_codes(c2), S, x)
    y4, b4 = oracle.gemv_q4(_pack_nibbles(c2 + 6), S, x)
    assert np.array_equal(y2, y4) and np.array_equal(b2, b4)


# ------------------------------------------------------- acceptance test --

def test_check_semantics():
    ok, worst, _ = oracle.check([1.0, 2.0], [1.0, 2.0001], [1.0, 2.0])
    assert ok and worst == pytest.approx(5e-5, rel=1e-6)
    ok, worst, idx = oracle.check([1.0, 2.0], [1.0, 2.0003], [1.0, 2.0])
    assert not ok and idx == (1,)
    assert oracle.check([0.0], [0.0], [0.0])[0]
    assert oracle.check([-0.0], [0.0], [0.0])[0]
    assert not oracle.check([1e-30], [0.0], [0.0])[0]
    assert not oracle.check([np.nan], [0.0], [1.0])[0]
    assert not oracle.check([np.inf], [1e38], [1e38])[0]


# ------------------------------------------------------ scaled, accumulating --

def test_gemm_ex_tiny_golden():
    g = load("gemm_ex_tiny_2x3x2.txt")
    A, B, C = _f32(g["A"]), _f32(g["B"]), _f32(g["C"])
    alpha, beta = np.asarray(g["alpha_beta"], np.float64)[0]
    out, bound = oracle.gemm_ex(A, B, C, alpha, beta)
    assert np.array_equal(out, np.asarray(g["out"], np.float64))
    assert np.array_equal(bound, np.asarray(g["bound"], np.float64))


@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (2.5, -0.5), (-1.0, 1.0), (0.75, 3.0)])
def test_gemm_ex_matches_numpy(ta, tb, alpha, beta):
    M, N, K = 13, 9, 21
    A = inputs.uniform(RNG, (K, M) if ta else (M, K))
    B = inputs.uniform(RNG, (N, K) if tb else (K, N))
    C = inputs.uniform(RNG, (M, N))
    a64 = A.astype(np.float64).T if ta else A.astype(np.float64)
    b64 = B.astype(np.float64).T if tb else B.astype(np.float64)
    ref = alpha * (a64 @ b64) + beta * C.astype(np.float64)
    out, bound = oracle.gemm_ex(A, B, C, alpha, beta, trans_a=bool(ta), trans_b=bool(tb))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(bound, abs(alpha) * (np.abs(a64) @ np.abs(b64)) +
                               np.abs(beta * C.astype(np.float64)), rtol=1e-13)


def test_gemm_ex_beta_zero_ignores_c():
    A = inputs.uniform(RNG, (6, 5))
    B = inputs.uniform(RNG, (5, 4))
    C = np.full((6, 4), np.nan, np.float32)
    out, _ = oracle.gemm_ex(A, B, C, 1.5, 0.0)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out, 1.5 * (A.astype(np.float64) @ B.astype(np.float64)),
                               rtol=0, atol=1e-13)


def test_gemm_ex_alpha_zero_scales_c_exactly():
    # alpha = 0: A and B are not read (NaN here), C is scaled exactly
    A = np.full((6, 5), np.nan, np.float32)
    B = inputs.uniform(RNG, (5, 4))
    C = inputs.uniform(RNG, (6, 4))
    out, bound = oracle.gemm_ex(A, B, C, 0.0, -2.0)
    assert np.array_equal(out, -2.0 * C.astype(np.float64))
    assert np.array_equal(bound, np.abs(2.0 * C.astype(np.float64)))


def test_gemm_ex_integer_exact():
    M, N, K = 17, 11, 40
    A = inputs.integers(RNG, (K, M))
    B = inputs.integers(RNG, (N, K))
    C = inputs.integers(RNG, (M, N))
    out, _ = oracle.gemm_ex(A, B, C, 3.0, -2.0, trans_a=True, trans_b=True)
    ref = 3 * (A.T.astype(np.int64) @ B.T.astype(np.int64)) - 2 * C.astype(np.int64)
    assert np.array_equal(out, ref.astype(np.float64))

