"""GPU parity where operands reach past 2 GiB: the launchers pick their load
paths by byte offsets.  The GEMM's direct loads address each operand with
32-bit offsets and take operands whose extent stays below 2^31 bytes, so
an operand just below that limit runs the direct path at its largest
offsets and one just above it the staged path with 64-bit row offsets; the
packed GEMV's flat split needs offsets below 2^31 and the row split's fast
path offsets below 2^32; the fp32 GEMV forms 64-bit row offsets.  Each
operand sits in a device buffer of its full leading dimension, padding
filled with NaN or garbage bytes, and results are checked against the
oracle on every element."""
import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs
from gpu_util import assert_close, host, torch

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(2 ** 31 - 1)
LIMIT = 1 << 31


def _padded_f32(X, ld):
    """X (rows x cols) in a device buffer of rows x ld floats, NaN padding."""
    t = torch()
    rows, cols = X.shape
    buf = t.full((rows, ld), float("nan"), dtype=t.float32, device="cuda")
    buf[:, :cols].copy_(t.from_numpy(np.ascontiguousarray(X)))
    return buf[:, :cols]


def _padded_u8(Q, ld):
    t = torch()
    rows, cols = Q.shape
    buf = t.full((rows, ld), 0xA5, dtype=t.uint8, device="cuda")
    buf[:, :cols].copy_(t.from_numpy(np.ascontiguousarray(Q)))
    return buf[:, :cols]


def _release():
    t = torch()
    t.cuda.synchronize()
    t.cuda.empty_cache()


def _extent(rows, cols, ld):
    return ((rows - 1) * ld + cols) * 4


# (layout, M, N, K, padded operand, its leading dimension): each operand's
# byte extent just below or just above 2^31
GEMM_CASES = [
    ("nn", 2048, 256, 256, "A", 262140),    # direct, 64 x 64 tiles
    ("nn", 2048, 256, 256, "A", 262400),    # staged
    ("tn", 256, 256, 2048, "A", 262140),    # direct, k-major A, small grid
    ("tn", 256, 256, 2048, "A", 262400),    # staged
    ("nt", 256, 2048, 256, "B", 262140),    # direct, x-major B
    ("nn", 256, 256, 2048, "B", 262140),    # direct, k-major B
    ("nn", 256, 256, 2048, "B", 262400),    # staged
    ("nn", 2048, 256, 256, "A", 262401),    # staged, rows not 16-byte aligned
    ("nn", 256, 256, 2048, "B", 262401),    # staged, rows not 16-byte aligned
]


@pytest.mark.parametrize("layout,M,N,K,which,ld", GEMM_CASES)
def test_gemm_operand_near_2gib(layout, M, N, K, which, ld):
    ta, tb = layout == "tn", layout == "nt"
    A = inputs.uniform(RNG, (K, M) if ta else (M, K))
    B = inputs.uniform(RNG, (N, K) if tb else (K, N))
    big = A if which == "A" else B
    ext = _extent(big.shape[0], big.shape[1], ld)
    assert (ext < LIMIT) == (ld == 262140)   # the intended side of 2^31
    if which == "A":
        dA, dB = _padded_f32(A, ld), torch().from_numpy(B).to("cuda")
    else:
        dA, dB = torch().from_numpy(A).to("cuda"), _padded_f32(B, ld)
    got = host(bd.gemm_f32_ex(dA, dB, None, 1.0, 0.0, trans_a=ta, trans_b=tb))
    ref, bound = oracle.gemm_ex(A, B, None, 1.0, 0.0, trans_a=ta, trans_b=tb)
    assert_close(got, ref, bound, "%s %dx%dx%d %s ld=%d extent=%d" % (layout, M, N, K, which, ld, ext))
    del dA, dB
    _release()


def _codes(M, K, bits, rng):
    per = 8 // bits
    codes = rng.integers(0, 1 << bits, (M, K)).astype(np.uint16).reshape(M, K // per, per)
    Q = np.zeros((M, K // per), np.uint16)
    for t in range(per):
        Q |= codes[..., t] << (bits * t)
    S = rng.uniform(0.01, 0.05, (M, K // 64)).astype(np.float16).view(np.uint16)
    return Q.astype(np.uint8), S


# (bits, rows, ldq): M * ldq past 2^31 (row split, 32-bit offsets) and past
# 2^32 (row split, 64-bit offsets)
PACKED_CASES = [(2, 2049, (1 << 20) + 16), (2, 2049, (1 << 21) + 16), (4, 2049, (1 << 20) + 32),
                (2, 2052, (1 << 20) + 16)]


@pytest.mark.parametrize("bits,M,ldq", PACKED_CASES)
def test_packed_rows_past_2gib(bits, M, ldq):
    K = 1536
    assert M * ldq >= LIMIT
    Q, S = _codes(M, K, bits, RNG)
    x = inputs.normal(RNG, (K,))
    ref, bound = (oracle.gemv_q2 if bits == 2 else oracle.gemv_q4)(Q, S, x)
    t = torch()
    dQ = _padded_u8(Q, ldq)
    dS = t.from_numpy(S.view(np.int16)).to("cuda")
    dx = t.from_numpy(x).to("cuda")
    f = bd.gemv_q2 if bits == 2 else bd.gemv_q4
    y = host(f(dQ, dS, dx))
    assert_close(y, ref, bound, "%d-bit M=%d ldq=%d" % (bits, M, ldq))
    fb = bd.gemv_q2_batched if bits == 2 else bd.gemv_q4_batched
    ys = fb([dQ, dQ], [dS, dS], [dx, dx])
    t.cuda.synchronize()
    assert np.array_equal(host(ys[1]), y)
    del dQ
    _release()


def test_gemv_f32_rows_past_2gib():
    M, K, ldw = 600, 1536, 1 << 20
    assert (M - 1) * ldw * 4 >= LIMIT
    W = inputs.normal(RNG, (M, K), 0.02)
    x = inputs.normal(RNG, (K,))
    ref, bound = oracle.gemv(W, x)
    dW = _padded_f32(W, ldw)
    y = host(bd.gemv_f32(dW, torch().from_numpy(x).to("cuda")))
    assert_close(y, ref, bound, "gemv_f32 ldw=%d" % ldw)
    del dW
    _release()
