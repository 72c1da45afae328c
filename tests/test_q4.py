"""GPU parity of gemv_q4 (4-bit codes + binary16 group scales) against the CPU
oracle's explicit unpack-then-dot, through the C ABI."""
import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs
from golden_io import load
from gpu_util import assert_close, canaries_intact, dev, guarded, host

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(44)


def _run(Q, S, x):
    return host(bd.gemv_q4(dev(Q), dev(S.view(np.int16)), dev(x)))


def _pack(codes):
    """column 2q+t in bits 4t..4t+3 of byte q"""
    M, K = codes.shape
    nb = (K + 1) // 2
    p = np.zeros((M, nb * 2), np.uint16)
    p[:, :K] = codes
    q = p.reshape(M, nb, 2)
    return (q[..., 0] | (q[..., 1] << 4)).astype(np.uint8)


def _pack2(codes):
    M, K = codes.shape
    nb = (K + 3) // 4
    p = np.zeros((M, nb * 4), np.uint16)
    p[:, :K] = codes
    q = p.reshape(M, nb, 4)
    return (q[..., 0] | (q[..., 1] << 2) | (q[..., 2] << 4) | (q[..., 3] << 6)).astype(np.uint8)


def _scales(M, K):
    return RNG.uniform(0.01, 0.05, (M, (K + 63) // 64)).astype(np.float16).view(np.uint16)


def test_tiny_hand_case():
    g = load("q4_tiny_2x4.txt")
    Q = np.array(g["Q"], np.uint8)
    S = np.array(g["S"], np.uint16)
    x = np.asarray(g["x"], np.float64).astype(np.float32)[0]
    assert np.array_equal(_run(Q, S, x), np.asarray(g["y"], np.float64).astype(np.float32)[0])


@pytest.mark.parametrize("M,K", [(1, 16), (7, 64), (48, 1536), (12288, 1536), (13, 100),
                                 (100, 3072), (5, 1), (9, 33)])
def test_integer_exact(M, K):
    # scale 2.0 and integer x: every partial sum is an integer below 2^24
    codes = RNG.integers(0, 16, (M, K))
    Q = _pack(codes)
    S = np.full((M, (K + 63) // 64), 0x4000, np.uint16)
    x = inputs.integers(RNG, (K,))
    ref, _ = oracle.gemv_q4(Q, S, x)
    assert np.array_equal(_run(Q, S, x).astype(np.float64), ref)


@pytest.mark.parametrize("r", [0, 1, 63])
def test_rotation_matrices_full_size(r):
    Q, S = inputs.q4_weight(r)
    x = inputs.q2_x()
    ref, bound = oracle.gemv_q4(Q, S, x)
    assert_close(_run(Q, S, x), ref, bound, "4-bit rotation matrix %d" % r)


@pytest.mark.parametrize("M,K", [(1, 1), (3, 5), (37, 70), (100, 1535), (61, 1537),
                                 (50, 4096), (11, 16 * 97)])
def test_ragged_shapes(M, K):
    codes = RNG.integers(0, 16, (M, K))
    Q = _pack(codes)
    S = _scales(M, K)
    x = inputs.normal(RNG, (K,))
    ref, bound = oracle.gemv_q4(Q, S, x)
    assert_close(_run(Q, S, x), ref, bound, "%dx%d" % (M, K))


def test_worst_case_levels():
    # every code at the middle levels 7 or 8 (|w| = s/2, the smallest), x of
    # one sign and wide range: the case the rounding bound is written for
    M, K = 600, 1536
    codes = RNG.integers(7, 9, (M, K))
    Q = _pack(codes)
    S = _scales(M, K)
    x = np.abs(inputs.normal(RNG, (K,))) * np.float32(2.0) ** RNG.integers(-6, 7, K).astype(np.float32)
    x = x.astype(np.float32)
    ref, bound = oracle.gemv_q4(Q, S, x)
    assert_close(_run(Q, S, x), ref, bound, "middle levels")


def test_matches_gemv_f32_on_dequantised_weights():
    Q, S = inputs.q4_weight(5, 600, 1536)
    x = inputs.q2_x()
    Wd = oracle.q4_unpack(Q, S, 1536)
    W32 = Wd.astype(np.float32)
    assert np.array_equal(W32.astype(np.float64), Wd)   # exact in fp32
    ref, bound = oracle.gemv(W32, x)
    assert_close(_run(Q, S, x), ref, bound, "q4")
    assert_close(host(bd.gemv_f32(dev(W32), dev(x))), ref, bound, "f32")


def test_agrees_with_q2_on_shared_levels():
    # 4-bit codes 6..9 are the 2-bit levels: (c + 6) - 7.5 = c - 1.5
    M, K = 700, 1536
    c2 = RNG.integers(0, 4, (M, K))
    S = _scales(M, K)
    x = inputs.normal(RNG, (K,))
    ref, bound = oracle.gemv_q2(_pack2(c2), S, x)
    y2 = host(bd.gemv_q2(dev(_pack2(c2)), dev(S.view(np.int16)), dev(x)))
    y4 = _run(_pack(c2 + 6), S, x)
    assert_close(y2, ref, bound, "q2")
    assert_close(y4, ref, bound, "q4 on q2 levels")


def test_padding_bits_and_bytes_ignored():
    # K = 71: the last byte has 1 dead column, the second scale group is
    # partial, rows carry garbage bytes/halves beyond their live width
    M, K = 45, 71
    codes = RNG.integers(0, 16, (M, K))
    Q = _pack(codes)
    S = _scales(M, K)
    x = inputs.normal(RNG, (K,))
    y = _run(Q, S, x)
    Qg = RNG.integers(0, 256, (M, Q.shape[1] + 7)).astype(np.uint8)
    Qg[:, :Q.shape[1]] = Q
    Qg[:, Q.shape[1] - 1] |= np.uint8(0xF0)
    Sg = RNG.integers(0, 65536, (M, 5)).astype(np.uint16)
    Sg[:, :2] = S
    y2 = host(bd.gemv_q4(dev(Qg), dev(Sg.view(np.int16)), dev(x)))
    assert np.array_equal(y, y2)


def test_padded_leading_dims_fast_path():
    # ldq, lds larger than needed and multiples of 8: the unit-load path
    M, K = 300, 1536
    Q, S = inputs.q4_weight(9, M, K)
    Qw = np.zeros((M, 800), np.uint8)
    Qw[:, :768] = Q
    Sw = np.zeros((M, 32), np.uint16)
    Sw[:, :24] = S
    x = inputs.q2_x()
    buf, yv = guarded(1, M)
    bd.gemv_q4(dev(Qw)[:, :768], dev(Sw.view(np.int16))[:, :24], dev(x), y=yv[0])
    ref, bound = oracle.gemv_q4(Q, S, x)
    assert_close(host(yv)[0], ref, bound, "padded")
    assert canaries_intact(buf)


def test_scale_doubling_doubles_output_bitwise():
    Q, S = inputs.q4_weight(11, 500, 1536)
    x = inputs.q2_x()
    S2 = (S.view(np.float16) * np.float16(2)).view(np.uint16)
    assert np.array_equal(_run(Q, S2, x), np.float32(2) * _run(Q, S, x))


def test_deterministic():
    Q, S = inputs.q4_weight(2)
    x = inputs.q2_x()
    dQ, dS, dx = dev(Q), dev(S.view(np.int16)), dev(x)
    assert np.array_equal(host(bd.gemv_q4(dQ, dS, dx)), host(bd.gemv_q4(dQ, dS, dx)))


def test_batched_equals_single_calls_and_oracle():
    mats = [inputs.q4_weight(r, 3000, 1536) for r in range(5)]
    x = inputs.q2_x()
    dQ = [dev(Q) for Q, _ in mats]
    dS = [dev(S.view(np.int16)) for _, S in mats]
    dx = dev(x)
    ys = bd.gemv_q4_batched(dQ, dS, [dx] * 5)
    for b, (Q, S) in enumerate(mats):
        assert np.array_equal(host(ys[b]), host(bd.gemv_q4(dQ[b], dS[b], dx))), b
        ref, bound = oracle.gemv_q4(Q, S, x)
        assert_close(host(ys[b]), ref, bound, "batched %d" % b)


def test_batched_more_than_one_launch_and_ragged():
    # 67 products (two launches), K = 200 (partial pass, odd units), own x each
    M, K, n = 70, 200, 67
    rng = np.random.default_rng(5)
    Qs = [rng.integers(0, 256, (M, K // 2), dtype=np.uint8) for _ in range(n)]
    Ss = [rng.uniform(0.01, 0.05, (M, 4)).astype(np.float16).view(np.uint16) for _ in range(n)]
    xs = [inputs.normal(rng, (K,)) for _ in range(n)]
    ys = bd.gemv_q4_batched([dev(q) for q in Qs], [dev(s.view(np.int16)) for s in Ss],
                            [dev(x) for x in xs])
    for b in range(n):
        ref, bound = oracle.gemv_q4(Qs[b], Ss[b], xs[b])
        assert_close(host(ys[b]), ref, bound, "product %d" % b)


# ---- the transposed shape: 1,536 rows of 12,288 columns, split 256 ways

def test_transposed_shape_full_size():
    Q, S = inputs.q4_weight(0, 1536, 12288)
    x = inputs.q2_x(12288)
    ref, bound = oracle.gemv_q4(Q, S, x)
    assert_close(_run(Q, S, x), ref, bound, "4-bit 1536x12288")


@pytest.mark.parametrize("M,K", [(1536, 12288), (100, 6500), (13, 6161)])
def test_transposed_shape_integer_exact(M, K):
    codes = RNG.integers(0, 16, (M, K))
    Q = _pack(codes)
    S = np.full((M, (K + 63) // 64), 0x4000, np.uint16)
    x = inputs.integers(RNG, (K,), -2, 2)
    ref, _ = oracle.gemv_q4(Q, S, x)
    assert np.array_equal(_run(Q, S, x).astype(np.float64), ref)


def test_transposed_shape_batched():
    mats = [inputs.q4_weight(r, 1536, 12288) for r in range(3)]
    x = inputs.q2_x(12288)
    dx = dev(x)
    ys = bd.gemv_q4_batched([dev(Q) for Q, _ in mats], [dev(S.view(np.int16)) for _, S in mats],
                            [dx] * 3)
    for b, (Q, S) in enumerate(mats):
        ref, bound = oracle.gemv_q4(Q, S, x)
        assert_close(host(ys[b]), ref, bound, "4-bit batched transposed %d" % b)
