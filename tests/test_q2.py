"""GPU parity of gemv_q2 (2-bit codes + binary16 group scales) against the CPU
oracle's explicit unpack-then-dot, through the C ABI."""
import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs
from golden_io import load
from gpu_util import assert_close, canaries_intact, dev, guarded, host, torch

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(99)


def _run(Q, S, x):
    t = torch()
    return host(bd.gemv_q2(dev(Q), dev(S.view(np.int16)), dev(x)))


def _pack(codes):
    M, K = codes.shape
    nb = (K + 3) // 4
    p = np.zeros((M, nb * 4), np.uint16)
    p[:, :K] = codes
    q = p.reshape(M, nb, 4)
    return (q[..., 0] | (q[..., 1] << 2) | (q[..., 2] << 4) | (q[..., 3] << 6)).astype(np.uint8)


def _scales(M, K):
    return RNG.uniform(0.01, 0.05, (M, (K + 63) // 64)).astype(np.float16).view(np.uint16)


def test_tiny_hand_case():
    g = load("q2_tiny_2x4.txt")
    Q = np.array(g["Q"], np.uint8)
    S = np.array(g["S"], np.uint16)
    x = np.asarray(g["x"], np.float64).astype(np.float32)[0]
    y = _run(Q, S, x)
    assert np.array_equal(y, np.asarray(g["y"], np.float64).astype(np.float32)[0])


@pytest.mark.parametrize("M,K", [(1, 16), (7, 64), (48, 1536), (12288, 1536), (13, 100),
                                 (100, 3072), (5, 1)])
def test_integer_exact(M, K):
    # scale 2.0 and integer x: every partial sum is an integer below 2^24
    codes = RNG.integers(0, 4, (M, K))
    Q = _pack(codes)
    S = np.full((M, (K + 63) // 64), 0x4000, np.uint16)
    x = inputs.integers(RNG, (K,))
    ref, _ = oracle.gemv_q2(Q, S, x)
    assert np.array_equal(_run(Q, S, x).astype(np.float64), ref)


@pytest.mark.parametrize("r", [0, 1, 63, 127])
def test_rotation_matrices_full_size(r):
    Q, S = inputs.q2_weight(r)
    x = inputs.q2_x()
    ref, bound = oracle.gemv_q2(Q, S, x)
    assert_close(_run(Q, S, x), ref, bound, "rotation matrix %d" % r)


@pytest.mark.parametrize("M,K", [(1, 1), (3, 5), (37, 70), (100, 1535), (61, 1537),
                                 (50, 4096), (11, 16 * 97)])
def test_ragged_shapes(M, K):
    codes = RNG.integers(0, 4, (M, K))
    Q = _pack(codes)
    S = _scales(M, K)
    x = inputs.normal(RNG, (K,))
    ref, bound = oracle.gemv_q2(Q, S, x)
    assert_close(_run(Q, S, x), ref, bound, "%dx%d" % (M, K))


def test_matches_gemv_f32_on_dequantised_weights():
    Q, S = inputs.q2_weight(5, 600, 1536)
    x = inputs.q2_x()
    Wd = oracle.q2_unpack(Q, S, 1536)
    W32 = Wd.astype(np.float32)
    assert np.array_equal(W32.astype(np.float64), Wd)   # exact in fp32
    yq = _run(Q, S, x)
    yf = host(bd.gemv_f32(dev(W32), dev(x)))
    ref, bound = oracle.gemv(W32, x)
    assert_close(yq, ref, bound, "q2")
    assert_close(yf, ref, bound, "f32")


def test_padding_bits_and_bytes_ignored():
    # K = 70: last byte has 2 dead columns, the second scale group is partial,
    # rows carry garbage bytes/halves beyond their live width
    M, K = 45, 70
    codes = RNG.integers(0, 4, (M, K))
    Q = _pack(codes)
    S = _scales(M, K)
    x = inputs.normal(RNG, (K,))
    y = _run(Q, S, x)
    Qg = RNG.integers(0, 256, (M, Q.shape[1] + 7)).astype(np.uint8)
    Qg[:, :Q.shape[1]] = Q
    Qg[:, Q.shape[1] - 1] |= np.uint8(0b11110000)
    Sg = RNG.integers(0, 65536, (M, 5)).astype(np.uint16)
    Sg[:, :2] = S
    y2 = host(bd.gemv_q2(dev(Qg), dev(Sg.view(np.int16)), dev(x)))
    assert np.array_equal(y, y2)


def test_padded_leading_dims_fast_path():
    # ldq, lds larger than needed and multiples of 4: the word-load path
    M, K = 300, 1536
    Q, S = inputs.q2_weight(9, M, K)
    Qw = np.zeros((M, 400), np.uint8)
    Qw[:, :384] = Q
    Sw = np.zeros((M, 32), np.uint16)
    Sw[:, :24] = S
    x = inputs.q2_x()
    buf, yv = guarded(1, M)
    bd.gemv_q2(dev(Qw)[:, :384], dev(Sw.view(np.int16))[:, :24], dev(x), y=yv[0])
    ref, bound = oracle.gemv_q2(Q, S, x)
    assert_close(host(yv)[0], ref, bound, "padded")
    assert canaries_intact(buf)


def test_scale_doubling_doubles_output_bitwise():
    Q, S = inputs.q2_weight(11, 500, 1536)
    x = inputs.q2_x()
    S2 = (S.view(np.float16) * np.float16(2)).view(np.uint16)
    assert np.array_equal(_run(Q, S2, x), np.float32(2) * _run(Q, S, x))


def test_deterministic():
    Q, S = inputs.q2_weight(2)
    x = inputs.q2_x()
    dQ, dS, dx = dev(Q), dev(S.view(np.int16)), dev(x)
    a = host(bd.gemv_q2(dQ, dS, dx))
    b = host(bd.gemv_q2(dQ, dS, dx))
    assert np.array_equal(a, b)


def _rotation(n, M=12288, K=1536, start=0):
    out = []
    for r in range(start, start + n):
        Q, S = inputs.q2_weight(r, M, K)
        out.append((Q, S))
    return out


def test_batched_and_single_calls_agree():
    """A batch and single calls on the same products both meet the tolerance
    (they may run different kernels, so the header promises no more), and a
    repeated batch gives the same bits."""
    mats = _rotation(5, 3000, 1536)
    x = inputs.q2_x()
    dQ = [dev(Q) for Q, _ in mats]
    dS = [dev(S.view(np.int16)) for _, S in mats]
    dx = dev(x)
    ys = bd.gemv_q2_batched(dQ, dS, [dx] * 5)
    again = bd.gemv_q2_batched(dQ, dS, [dx] * 5)
    for b, (Q, S) in enumerate(mats):
        ref, bound = oracle.gemv_q2(Q, S, x)
        assert_close(host(bd.gemv_q2(dQ[b], dS[b], dx)), ref, bound, "single %d" % b)
        assert_close(host(ys[b]), ref, bound, "batched %d" % b)
        assert np.array_equal(host(ys[b]), host(again[b])), b


def test_batched_more_than_one_launch_and_own_x():
    # 70 products: two launches of the kernel (64 + 6); distinct x per product
    M, K = 200, 320
    n = 70
    rng = np.random.default_rng(3)
    Qs = [rng.integers(0, 256, (M, K // 4), dtype=np.uint8) for _ in range(n)]
    Ss = [rng.uniform(0.01, 0.05, (M, K // 64)).astype(np.float16).view(np.uint16) for _ in range(n)]
    xs = [inputs.normal(rng, (K,)) for _ in range(n)]
    ys = bd.gemv_q2_batched([dev(q) for q in Qs], [dev(s.view(np.int16)) for s in Ss],
                            [dev(x) for x in xs])
    for b in range(n):
        ref, bound = oracle.gemv_q2(Qs[b], Ss[b], xs[b])
        assert_close(host(ys[b]), ref, bound, "product %d" % b)


def test_batched_ragged_shape_generic_path():
    M, K = 37, 70
    rng = np.random.default_rng(4)
    mats = []
    for b in range(3):
        codes = rng.integers(0, 4, (M, K))
        mats.append((_pack(codes), _scales(M, K)))
    x = inputs.normal(rng, (K,))
    ys = bd.gemv_q2_batched([dev(Q) for Q, _ in mats], [dev(S.view(np.int16)) for _, S in mats],
                            [dev(x)] * 3)
    for b, (Q, S) in enumerate(mats):
        ref, bound = oracle.gemv_q2(Q, S, x)
        assert_close(host(ys[b]), ref, bound, "ragged %d" % b)


def test_batched_large_full_size():
    # 12 products of the full 12,288 x 1,536 shape in one launch
    n = 12
    mats = _rotation(n)
    x = inputs.q2_x()
    dQ = [dev(Q) for Q, _ in mats]
    dS = [dev(S.view(np.int16)) for _, S in mats]
    dx = dev(x)
    ys = [host(y) for y in bd.gemv_q2_batched(dQ, dS, [dx] * n)]
    again = [host(y) for y in bd.gemv_q2_batched(dQ, dS, [dx] * n)]
    for b in (0, 5, 11):
        ref, bound = oracle.gemv_q2(mats[b][0], mats[b][1], x)
        assert_close(ys[b], ref, bound, "large batch %d" % b)
    for b in range(n):
        assert np.array_equal(ys[b], again[b]), "not reproducible"


@pytest.mark.parametrize("M,K", [(12345, 3072), (20000, 640), (11000, 1600)])
def test_batched_large_ragged(M, K):
    # M not a multiple of any workgroup's rows; K of 48, 10 and 25 scale groups
    n = max(2, -(-131072 // M))
    rng = np.random.default_rng(M + K)
    Qs = [rng.integers(0, 256, (M, K // 4), dtype=np.uint8) for _ in range(n)]
    Ss = [rng.uniform(0.01, 0.05, (M, K // 64)).astype(np.float16).view(np.uint16) for _ in range(n)]
    xs = [inputs.normal(rng, (K,)) for _ in range(n)]
    ys = bd.gemv_q2_batched([dev(q) for q in Qs], [dev(s.view(np.int16)) for s in Ss],
                            [dev(x) for x in xs])
    for b in (0, n - 1):
        ref, bound = oracle.gemv_q2(Qs[b], Ss[b], xs[b])
        assert_close(host(ys[b]), ref, bound, "%dx%d product %d" % (M, K, b))


def test_batched_large_integer_exact():
    # scale 2 and integer x: every partial sum is an exact integer
    M, K, n = 16384, 1536, 8
    rng = np.random.default_rng(8)
    codes = [rng.integers(0, 4, (M, K)) for _ in range(2)]
    Qs = [_pack(c) for c in codes] * (n // 2)
    S = np.full((M, K // 64), 0x4000, np.uint16)
    x = inputs.integers(rng, (K,))
    ys = bd.gemv_q2_batched([dev(q) for q in Qs], [dev(S.view(np.int16))] * n, [dev(x)] * n)
    for b in range(2):
        ref, _ = oracle.gemv_q2(Qs[b], S, x)
        assert np.array_equal(host(ys[b]).astype(np.float64), ref)


# ---- the transposed shape: 1,536 rows of 12,288 columns, split 256 ways

@pytest.mark.parametrize("r", [0, 3])
def test_transposed_shape_full_size(r):
    Q, S = inputs.q2_weight(r, 1536, 12288)
    x = inputs.q2_x(12288)
    ref, bound = oracle.gemv_q2(Q, S, x)
    assert_close(_run(Q, S, x), ref, bound, "1536x12288 #%d" % r)


@pytest.mark.parametrize("M,K", [(1536, 12288), (100, 6500), (7, 24576), (13, 6160)])
def test_transposed_shape_integer_exact(M, K):
    codes = RNG.integers(0, 4, (M, K))
    Q = _pack(codes)
    S = np.full((M, (K + 63) // 64), 0x4000, np.uint16)
    x = inputs.integers(RNG, (K,), -4, 4)
    ref, _ = oracle.gemv_q2(Q, S, x)
    assert np.array_equal(_run(Q, S, x).astype(np.float64), ref)


def test_transposed_shape_batched():
    mats = [inputs.q2_weight(r, 1536, 12288) for r in range(3)]
    x = inputs.q2_x(12288)
    dx = dev(x)
    ys = bd.gemv_q2_batched([dev(Q) for Q, _ in mats], [dev(S.view(np.int16)) for _, S in mats],
                            [dx] * 3)
    for b, (Q, S) in enumerate(mats):
        ref, bound = oracle.gemv_q2(Q, S, x)
        assert_close(host(ys[b]), ref, bound, "batched transposed %d" % b)
