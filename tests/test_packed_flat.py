"""GPU parity of the packed-weight GEMVs on the shapes that take the flat
split: K a multiple of 64 whose rows hold 8 to 48 chunks of 16 bytes that
divide a 192-lane workgroup (2-bit K in {512, 768, 1024, 1536, 2048, 3072},
4-bit K in {256, 384, 512, 768, 1024, 1536}), with 16-byte aligned code rows
and x.  Row counts fall on both sides of a workgroup's rows (24 rows per
workgroup for one product at 24 chunks, 64 in a batch),
leading dimensions are padded with garbage, and results are checked against
the oracle element by element, bit for bit where every partial sum is an
integer."""
import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs
from gpu_util import assert_close, dev, host, torch

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(192)

K2 = [512, 768, 1024, 1536, 2048, 3072]
K4 = [256, 384, 512, 768, 1024, 1536]


def _pack(codes, bits):
    """column c of a row in bits bits*(c % (8/bits)).. of byte c // (8/bits)"""
    M, K = codes.shape
    per = 8 // bits
    q = codes.reshape(M, K // per, per).astype(np.uint16)
    out = np.zeros((M, K // per), np.uint16)
    for t in range(per):
        out |= q[..., t] << (bits * t)
    return out.astype(np.uint8)


def _padded(a, extra, fill_rng):
    """a copy of the M x n array inside an M x (n + extra) one whose padding
    holds random bytes; returns the full array (the caller slices it)."""
    M, n = a.shape
    full = fill_rng.integers(0, 256 if a.dtype == np.uint8 else 65536,
                             (M, n + extra)).astype(a.dtype)
    full[:, :n] = a
    return full


def _operands(M, K, bits, integer=False, rng=RNG):
    codes = rng.integers(0, 1 << bits, (M, K))
    Q = _pack(codes, bits)
    if integer:
        S = np.full((M, K // 64), 0x4000, np.uint16)
        x = inputs.integers(rng, (K,))
    else:
        S = rng.uniform(0.01, 0.05, (M, K // 64)).astype(np.float16).view(np.uint16)
        x = inputs.normal(rng, (K,))
    return Q, S, x


def _oracle(bits, Q, S, x):
    return (oracle.gemv_q2 if bits == 2 else oracle.gemv_q4)(Q, S, x)


def _single(bits, dQ, dS, dx):
    f = bd.gemv_q2 if bits == 2 else bd.gemv_q4
    return host(f(dQ, dS, dx))


def _batched(bits, dQs, dSs, dxs):
    f = bd.gemv_q2_batched if bits == 2 else bd.gemv_q4_batched
    ys = f(dQs, dSs, dxs)
    torch().cuda.synchronize()
    return [host(y) for y in ys]


def _cases():
    for bits, ks in ((2, K2), (4, K4)):
        for K in ks:
            for M in (1, 7, 129, 1000):
                yield bits, M, K


@pytest.mark.parametrize("bits,M,K", list(_cases()))
def test_single_and_batched(bits, M, K):
    Q, S, x = _operands(M, K, bits)
    ref, bound = _oracle(bits, Q, S, x)
    y = _single(bits, dev(Q), dev(S.view(np.int16)), dev(x))
    assert_close(y, ref, bound, "%d-bit single %dx%d" % (bits, M, K))
    # a batch of three: this product between two others of the same shape
    Q1, S1, x1 = _operands(M, K, bits)
    Q2, S2, x2 = _operands(M, K, bits)
    ys = _batched(bits, [dev(Q1), dev(Q), dev(Q2)],
                  [dev(S1.view(np.int16)), dev(S.view(np.int16)), dev(S2.view(np.int16))],
                  [dev(x1), dev(x), dev(x2)])
    assert_close(ys[1], ref, bound, "%d-bit batched %dx%d" % (bits, M, K))
    for (Qb, Sb, xb), yb in (((Q1, S1, x1), ys[0]), ((Q2, S2, x2), ys[2])):
        rb, bb = _oracle(bits, Qb, Sb, xb)
        assert_close(yb, rb, bb, "%d-bit batched neighbour %dx%d" % (bits, M, K))
    # 4-bit batches run the single call's arithmetic per row; 2-bit batches
    # of these shapes may take the integer-dot kernel, so they are held to
    # the tolerance above and to repeating their own bits
    if bits == 4:
        assert np.array_equal(y, ys[1])
    else:
        again = _batched(bits, [dev(Q1), dev(Q), dev(Q2)],
                         [dev(S1.view(np.int16)), dev(S.view(np.int16)), dev(S2.view(np.int16))],
                         [dev(x1), dev(x), dev(x2)])
        assert np.array_equal(again[1], ys[1])


@pytest.mark.parametrize("bits,K", [(2, 1536), (2, 512), (2, 3072), (4, 1536), (4, 256)])
@pytest.mark.parametrize("M", [8, 300, 2049])
def test_integer_exact(bits, M, K):
    # scale 2.0 and integers in [-8, 8]: every partial sum is an integer below
    # 2^24, so the result is exact whatever the order
    Q, S, x = _operands(M, K, bits, integer=True)
    ref, _ = _oracle(bits, Q, S, x)
    y = _single(bits, dev(Q), dev(S.view(np.int16)), dev(x))
    assert np.array_equal(y.astype(np.float64), ref)
    ys = _batched(bits, [dev(Q)] * 2, [dev(S.view(np.int16))] * 2, [dev(x)] * 2)
    assert np.array_equal(ys[0].astype(np.float64), ref)
    assert np.array_equal(ys[1].astype(np.float64), ref)


@pytest.mark.parametrize("bits,K", [(2, 1536), (4, 768), (2, 512)])
def test_padded_leading_dimensions(bits, K):
    """ldq padded by 16 and by 48 bytes and lds by 5 halves, padding full of
    random bits: only the K columns of each row may count."""
    M = 333
    Q, S, x = _operands(M, K, bits)
    ref, bound = _oracle(bits, Q, S, x)
    for extra in (16, 48):
        Qp = _padded(Q, extra, RNG)
        Sp = _padded(S, 5, RNG)
        dQ = dev(Qp)[:, :Q.shape[1]]
        dS = dev(Sp.view(np.int16))[:, :S.shape[1]]
        assert dQ.stride(0) == Q.shape[1] + extra
        y = _single(bits, dQ, dS, dev(x))
        assert_close(y, ref, bound, "%d-bit ldq+%d" % (bits, extra))
        ys = _batched(bits, [dQ, dQ], [dS, dS], [dev(x), dev(x)])
        assert_close(ys[1], ref, bound, "%d-bit batched ldq+%d" % (bits, extra))


@pytest.mark.parametrize("bits", [2, 4])
def test_guarded_output_and_deterministic(bits):
    """The output is written exactly: canaries around y stay intact, and two
    calls give the same bits."""
    M, K = 1001, 1536
    Q, S, x = _operands(M, K, bits)
    ref, bound = _oracle(bits, Q, S, x)
    t = torch()
    pad = 64
    buf = t.full((M + 2 * pad,), 7.5e8, dtype=t.float32, device="cuda")
    y = buf[pad:pad + M]
    f = bd.gemv_q2 if bits == 2 else bd.gemv_q4
    dQ, dS, dx = dev(Q), dev(S.view(np.int16)), dev(x)
    f(dQ, dS, dx, y=y)
    h = host(buf)
    assert np.all(h[:pad] == np.float32(7.5e8)) and np.all(h[-pad:] == np.float32(7.5e8))
    assert_close(h[pad:pad + M], ref, bound, "%d-bit guarded" % bits)
    y2 = host(f(dQ, dS, dx))
    assert np.array_equal(h[pad:pad + M], y2)


@pytest.mark.parametrize("bits", [2, 4])
def test_full_size_batch_of_forty(bits):
    """A token's 40 products at 12,288 x 1,536 over the seeded rotation
    matrices, each checked against the oracle."""
    gen = inputs.q2_weight if bits == 2 else inputs.q4_weight
    x = inputs.q2_x()
    dx = dev(x)
    mats = [gen(r) for r in range(40)]
    ys = _batched(bits, [dev(Q) for Q, _ in mats], [dev(S.view(np.int16)) for _, S in mats],
                  [dx] * 40)
    for r in (0, 13, 39):
        ref, bound = _oracle(bits, *mats[r], x)
        assert_close(ys[r], ref, bound, "%d-bit batch product %d" % (bits, r))


@pytest.mark.parametrize("bits,M,count", [(2, 5000, 64), (2, 12288, 50), (2, 777, 40),
                                          (4, 3001, 33), (4, 12288, 7)])
def test_large_batches(bits, M, count):
    """Batches of 7 to 64 products, with a partial last workgroup at 5,000,
    777 and 3,001 rows: sampled products against the oracle, and the same
    bits as single calls (4-bit) or as a second launch of the batch (2-bit,
    whose batches may take the integer-dot kernel)."""
    K = 1536
    rng = np.random.default_rng(7 * M + count)
    x = inputs.normal(rng, (K,))
    dx = dev(x)
    mats = [_operands(M, K, bits, rng=rng)[:2] for _ in range(count)]
    dQ = [dev(Q) for Q, _ in mats]
    dS = [dev(S.view(np.int16)) for _, S in mats]
    ys = _batched(bits, dQ, dS, [dx] * count)
    again = _batched(bits, dQ, dS, [dx] * count) if bits == 2 else None
    for r in (0, count // 2, count - 1):
        ref, bound = _oracle(bits, *mats[r], x)
        assert_close(ys[r], ref, bound, "%d-bit batch product %d of %d, M=%d" % (bits, r, count, M))
        other = _single(bits, dQ[r], dS[r], dx) if bits == 4 else again[r]
        assert np.array_equal(ys[r], other)


@pytest.mark.parametrize("bits,K", [(2, 12288), (4, 6144)])
@pytest.mark.parametrize("M", [1, 7, 1001, 1536])
def test_long_rows(bits, M, K):
    """Rows of 192 chunks of 16 bytes (the transposed 12,288-input shape for
    2-bit codes), which the row-split kernel serves with a row over a whole
    workgroup: single and batched calls against the oracle and bit for bit
    against each other, and integer inputs exactly."""
    Q, S, x = _operands(M, K, bits)
    ref, bound = _oracle(bits, Q, S, x)
    y = _single(bits, dev(Q), dev(S.view(np.int16)), dev(x))
    assert_close(y, ref, bound, "%d-bit long %dx%d" % (bits, M, K))
    Q1, S1, x1 = _operands(M, K, bits)
    ys = _batched(bits, [dev(Q1), dev(Q)], [dev(S1.view(np.int16)), dev(S.view(np.int16))],
                  [dev(x1), dev(x)])
    assert np.array_equal(y, ys[1])
    r1, b1 = _oracle(bits, Q1, S1, x1)
    assert_close(ys[0], r1, b1, "%d-bit long batched %dx%d" % (bits, M, K))
    Qi, Si, xi = _operands(M, K, bits, integer=True)
    refi, _ = _oracle(bits, Qi, Si, xi)
    assert np.array_equal(_single(bits, dev(Qi), dev(Si.view(np.int16)), dev(xi)).astype(np.float64), refi)


@pytest.mark.parametrize("bits,K", [(2, 12288), (4, 6144)])
def test_long_rows_padded(bits, K):
    """The same long rows with ldq padded by 32 bytes and lds by 3 halves,
    padding full of random bits."""
    M = 301
    Q, S, x = _operands(M, K, bits)
    ref, bound = _oracle(bits, Q, S, x)
    dQ = dev(_padded(Q, 32, RNG))[:, :Q.shape[1]]
    dS = dev(_padded(S, 3, RNG).view(np.int16))[:, :S.shape[1]]
    assert_close(_single(bits, dQ, dS, dev(x)), ref, bound, "%d-bit long padded" % bits)
    ys = _batched(bits, [dQ] * 3, [dS] * 3, [dev(x)] * 3)
    assert_close(ys[2], ref, bound, "%d-bit long padded batched" % bits)
