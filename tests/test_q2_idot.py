"""The integer-dot 2-bit kernel that serves batches (K a multiple of 512, up
to 3,072 columns, 16-byte aligned operands), element by element against the
oracle.

The kernel rounds x to integers per 64-column chunk, with 6 base-16 digits in
general and 5 when the chunk's sum of |x| is at least 8 times its largest
power of two (the wave of 8 chunks takes 6 if any of its chunks needs them).
These tests cover both digit counts and the waves that mix them, x scaled far
from 1, the worst case for rounding x (one large value per chunk among tiny
ones), exact integer sums, non-finite x and scales, the launches that must
fall back to the multiply-add kernel (misaligned scales, x or scale rows), and
ragged row counts on both sides of a workgroup's 128 rows.
"""
import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs

from gpu_util import assert_close, dev, host

pytestmark = pytest.mark.gpu

K_IDOT = (512, 1024, 1536, 2048, 3072)


def _mats(n, M, K, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        Q = rng.integers(0, 256, (M, K // 4), dtype=np.uint8)
        S = rng.uniform(0.01, 0.05, (M, K // 64)).astype(np.float16).view(np.uint16)
        out.append((Q, S))
    return out


def _batch(mats, xs):
    ys = bd.gemv_q2_batched([dev(Q) for Q, _ in mats], [dev(S.view(np.int16)) for _, S in mats],
                            [dev(x) for x in xs])
    return [host(y) for y in ys]


def _check_all(mats, xs, ys, what):
    for b, ((Q, S), x, y) in enumerate(zip(mats, xs, ys)):
        ref, bound = oracle.gemv_q2(Q, S, x)
        assert_close(y, ref, bound, "%s, product %d" % (what, b))


@pytest.mark.parametrize("K", K_IDOT)
@pytest.mark.parametrize("M", [1, 7, 127, 128, 129, 3000])
def test_shapes(M, K):
    mats = _mats(3, M, K, 11 * M + K)
    rng = np.random.default_rng(M + K)
    xs = [inputs.normal(rng, (K,)) for _ in range(3)]
    _check_all(mats, xs, _batch(mats, xs), "%dx%d" % (M, K))


@pytest.mark.parametrize("scale", [2.0 ** 110, 2.0 ** 60, 2.0 ** -60, 2.0 ** -100, 2.0 ** -120])
def test_x_far_from_one(scale):
    """x scaled by powers of two from 2^-120 to 2^110: the quantisation
    follows each chunk's exponent, so the relative error does not move."""
    M, K = 700, 1536
    mats = _mats(2, M, K, 5)
    rng = np.random.default_rng(6)
    xs = [(inputs.normal(rng, (K,)).astype(np.float64) * scale).astype(np.float32)
          for _ in range(2)]
    ys = _batch(mats, xs)
    assert all(np.all(np.isfinite(y)) for y in ys)
    _check_all(mats, xs, ys, "x scaled by 2^%d" % int(np.log2(scale)))


def test_chunks_of_different_magnitudes():
    """Each 64-column chunk at its own scale, 2^-90 .. 2^90."""
    M, K = 500, 3072
    mats = _mats(2, M, K, 8)
    rng = np.random.default_rng(9)
    xs = []
    for _ in range(2):
        x = inputs.normal(rng, (K,)).astype(np.float64)
        for c in range(K // 64):
            x[64 * c:64 * c + 64] *= 2.0 ** int(rng.integers(-90, 91))
        xs.append(x.astype(np.float32))
    _check_all(mats, xs, _batch(mats, xs), "mixed chunk scales")


def test_one_large_value_per_chunk():
    """The worst case for rounding x: in each chunk one value near 1 and 63
    values about 2^-24 of it, so nearly all of the chunk's bound comes from one
    column and the small ones are rounded the most.  These chunks need six
    digits."""
    M, K = 1000, 2048
    mats = _mats(2, M, K, 12)
    rng = np.random.default_rng(13)
    xs = []
    for _ in range(2):
        x = rng.uniform(-1.0, 1.0, K) * 2.0 ** -24
        x[rng.integers(0, 64) :: 64] = rng.uniform(0.5, 1.0) * rng.choice([-1.0, 1.0])
        xs.append(x.astype(np.float32))
    _check_all(mats, xs, _batch(mats, xs), "one large value per chunk")


def test_waves_with_five_and_six_digits():
    """Typical x (five digits) in some 512-column waves and concentrated x
    (six digits) in others, within one row."""
    M, K = 900, 3072
    mats = _mats(3, M, K, 14)
    rng = np.random.default_rng(15)
    xs = []
    for b in range(3):
        x = inputs.normal(rng, (K,)).astype(np.float64)
        for w in range(K // 512):
            if (w + b) % 2:
                blk = x[512 * w:512 * w + 512]
                blk *= 1e-6
                blk[::64] = 3.5
        xs.append(x.astype(np.float32))
    _check_all(mats, xs, _batch(mats, xs), "five- and six-digit waves")


@pytest.mark.parametrize("K", [512, 1536, 3072])
def test_integer_sums_are_exact(K):
    """Scales 2.0 and integer x in [-8, 8]: every partial sum is an integer
    below 2^24, so the result equals the oracle bit for bit."""
    M = 1001
    rng = np.random.default_rng(K)
    mats = []
    for _ in range(2):
        Q = rng.integers(0, 256, (M, K // 4), dtype=np.uint8)
        mats.append((Q, np.full((M, K // 64), 0x4000, np.uint16)))
    xs = [rng.integers(-8, 9, K).astype(np.float32) for _ in range(2)]
    for (Q, S), x, y in zip(mats, xs, _batch(mats, xs)):
        ref, _ = oracle.gemv_q2(Q, S, x)
        assert np.array_equal(y.astype(np.float64), ref)


def test_scale_doubling_and_repeat_bits():
    M, K = 1234, 1536
    mats = _mats(3, M, K, 21)
    rng = np.random.default_rng(22)
    xs = [inputs.normal(rng, (K,)) for _ in range(3)]
    ys = _batch(mats, xs)
    again = _batch(mats, xs)
    doubled = [(Q, (S.view(np.float16) * np.float16(2)).view(np.uint16)) for Q, S in mats]
    ys2 = _batch(doubled, xs)
    for y, a, y2 in zip(ys, again, ys2):
        assert np.array_equal(y, a)
        assert np.array_equal(y2, np.float32(2) * y)


def test_padded_rows_are_ignored():
    """Code rows and scale rows padded with garbage (ldq > K/4, lds > K/64, both
    keeping 16-byte alignment): the padding is never read into a sum."""
    M, K = 333, 1024
    rng = np.random.default_rng(23)
    Qp = rng.integers(0, 256, (M, K // 4 + 32), dtype=np.uint8)
    Sp = rng.uniform(0.01, 0.05, (M, K // 64 + 8)).astype(np.float16)
    Sp[:, K // 64:] = np.float16(np.nan)
    x = inputs.normal(rng, (K,))
    dQ, dS = dev(Qp)[:, :K // 4], dev(Sp.view(np.int16))[:, :K // 64]
    ys = bd.gemv_q2_batched([dQ, dQ], [dS, dS], [dev(x), dev(x)])
    ref, bound = oracle.gemv_q2(np.ascontiguousarray(Qp[:, :K // 4]),
                                np.ascontiguousarray(Sp[:, :K // 64]).view(np.uint16), x)
    for y in ys:
        assert_close(host(y), ref, bound, "padded rows")


@pytest.mark.parametrize("what", ["lds", "S", "x"])
def test_misaligned_operands_fall_back(what):
    """Scale rows whose stride is not a multiple of 8 halves, a scale base off
    16 bytes, or an x off 16 bytes: the batch takes the multiply-add kernel and
    still matches the oracle."""
    M, K = 777, 1536
    rng = np.random.default_rng(24)
    Q = rng.integers(0, 256, (M, K // 4), dtype=np.uint8)
    lds = K // 64 + (1 if what == "lds" else 0)
    Sp = rng.uniform(0.01, 0.05, (M + 1, lds)).astype(np.float16)
    x = inputs.normal(rng, (K + 1,))
    t = dev(Sp.view(np.int16))
    if what == "S":
        dS = t.view(-1)[2:2 + M * lds].view(M, lds)[:, :K // 64]
        S = Sp.reshape(-1)[2:2 + M * lds].reshape(M, lds)[:, :K // 64]
    else:
        dS, S = t[:M, :K // 64], Sp[:M, :K // 64]
    dx = dev(x)[1:] if what == "x" else dev(x)[:K]
    xv = x[1:] if what == "x" else x[:K]
    ys = bd.gemv_q2_batched([dev(Q)] * 2, [dS] * 2, [dx] * 2)
    ref, bound = oracle.gemv_q2(Q, np.ascontiguousarray(S).view(np.uint16),
                                np.ascontiguousarray(xv))
    for y in ys:
        assert_close(host(y), ref, bound, "misaligned %s" % what)


def test_non_finite_x_makes_every_output_nan():
    M, K = 300, 1536
    mats = _mats(2, M, K, 25)
    rng = np.random.default_rng(26)
    for bad in (np.inf, -np.inf, np.nan):
        xs = [inputs.normal(rng, (K,)) for _ in range(2)]
        xs[1][1000] = bad
        ys = _batch(mats, xs)
        assert np.all(np.isnan(ys[1])), bad
        ref, bound = oracle.gemv_q2(mats[0][0], mats[0][1], xs[0])
        assert_close(ys[0], ref, bound, "finite neighbour of a non-finite x")


def test_nan_scale_makes_its_row_nan():
    M, K = 300, 1024
    (Q, S), = _mats(1, M, K, 27)
    S = S.copy()
    S[17, 5] = np.float16(np.nan).view(np.uint16)
    x = inputs.normal(np.random.default_rng(28), (K,))
    y = _batch([(Q, S)] * 2, [x, x])[0]
    assert np.isnan(y[17])
    rows = np.arange(M) != 17
    ref, bound = oracle.gemv_q2(Q, S, x)
    assert_close(y[rows], ref[rows], bound[rows], "rows beside a NaN scale")
