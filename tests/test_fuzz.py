"""Seeded random cases through the C ABI against the CPU oracle: shapes on
both sides of the tile, slab and tile-count boundaries, transpose pairs,
alignment offsets, leading-dimension padding and alpha/beta for the matrix
product; widths, shapes, padding, offsets and batch sizes for
the packed matrix-vector products.  Each case is named by its seed.

GG_FUZZ_SCALE=n (default 1) multiplies every test's number of seeds by n for
longer runs; the first seeds stay the same."""
import os

import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs
from gpu_util import assert_close, dev, host, torch

pytestmark = pytest.mark.gpu

SCALE = max(1, int(os.environ.get("GG_FUZZ_SCALE", "1")))


def _placed(a, offset, pad):
    """Device copy of 2-D float32 array a, starting `offset` floats into a
    buffer, with `pad` extra floats per row (leading dimension cols + pad)."""
    t = torch()
    rows, cols = a.shape
    ld = cols + pad
    buf = t.full((offset + max(rows * ld, 1),), float("nan"), dtype=t.float32, device="cuda")
    view = buf[offset:offset + rows * ld].view(rows, ld)[:, :cols]
    view.copy_(t.from_numpy(np.ascontiguousarray(a)).to("cuda"))
    return view


@pytest.mark.parametrize("seed", range(120 * SCALE))
def test_gemm_random_cases(seed):
    rng = np.random.default_rng(1000 + seed)
    hi = 1100 if seed % 4 == 3 else 300          # one case in four past the CU count
    M, N = (int(v) for v in rng.integers(1, hi, 2))
    K = int(rng.integers(0, 400 if hi > 300 else 1200))
    if rng.random() < 0.5:                       # rows of whole 16-byte chunks
        M, N, K = (v + (-v) % 4 for v in (M, N, K))
    ta, tb = (bool(v) for v in rng.integers(0, 2, 2))
    alpha, beta = (float(v) for v in rng.choice([0.0, 1.0, -1.5, 0.5], 2))
    A = inputs.uniform(rng, (K, M) if ta else (M, K))
    B = inputs.uniform(rng, (N, K) if tb else (K, N))
    C = inputs.uniform(rng, (M, N))
    oa, ob, oc = (int(v) for v in rng.choice([0, 0, 4, 1, 3], 3))
    pa, pb, pc = (int(v) for v in rng.choice([0, 0, 4, 8, 5], 3))
    dA, dB, dC = _placed(A, oa, pa), _placed(B, ob, pb), _placed(C, oc, pc)
    bd.gemm_f32_ex(dA, dB, dC, alpha, beta, trans_a=ta, trans_b=tb)
    ref, bound = oracle.gemm_ex(A, B, C, alpha, beta, trans_a=ta, trans_b=tb)
    assert_close(host(dC), ref, bound,
                 "seed %d: %s%s %dx%dx%d a=%g b=%g offsets %d/%d/%d pads %d/%d/%d"
                 % (seed, "T" if ta else "N", "T" if tb else "N", M, N, K, alpha, beta,
                    oa, ob, oc, pa, pb, pc))


def _packed_case(rng, bits, M, K, pad_q, pad_s):
    per_byte = 8 // bits
    nb = (K + per_byte - 1) // per_byte
    Q = rng.integers(0, 256, (M, nb + pad_q), dtype=np.uint8)
    S = rng.uniform(0.01, 0.05, (M, (K + 63) // 64 + pad_s)).astype(np.float16).view(np.uint16)
    return Q, S


@pytest.mark.parametrize("seed", range(36 * SCALE))
def test_packed_random_cases(seed):
    rng = np.random.default_rng(2000 + seed)
    bits = int(rng.choice([2, 4]))
    if rng.random() < 0.3:                        # long rows, few of them: the 256-way split
        M, K = int(rng.integers(1, 300)), int(rng.integers(6144, 9000))
    else:
        M, K = int(rng.integers(1, 800)), int(rng.integers(1, 3200))
    count = int(rng.choice([1, 1, 2, 3]))
    t = torch()
    # one shape and leading dimension for every product of a batch
    pad_q, pad_s = int(rng.choice([0, 0, 8, 3])), int(rng.choice([0, 0, 8, 1]))
    mats = [_packed_case(rng, bits, M, K, pad_q, pad_s) for _ in range(count)]
    xs = [inputs.normal(rng, (K,)) for _ in range(count)]
    off = int(rng.choice([0, 0, 1]))              # a misaligned code base takes the byte path
    dQ, dS = [], []
    for Q, S in mats:
        buf = t.zeros(off + Q.size, dtype=t.uint8, device="cuda")
        q = buf[off:].view(Q.shape)
        q.copy_(t.from_numpy(Q).to("cuda"))
        dQ.append(q)
        dS.append(dev(S.view(np.int16)))
    live = (K + 8 // bits - 1) // (8 // bits)
    dQ = [q[:, :live] for q in dQ]
    dS = [s[:, :(K + 63) // 64] for s in dS]
    f1 = bd.gemv_q2 if bits == 2 else bd.gemv_q4
    fb = bd.gemv_q2_batched if bits == 2 else bd.gemv_q4_batched
    ref_fn = oracle.gemv_q2 if bits == 2 else oracle.gemv_q4
    if count == 1:
        ys = [f1(dQ[0], dS[0], dev(xs[0]))]
    else:
        ys = fb(dQ, dS, [dev(x) for x in xs])
    for b in range(count):
        Q, S = mats[b]
        ref, bound = ref_fn(Q, S, xs[b], K=K)
        assert_close(host(ys[b]), ref, bound, "seed %d: %d-bit %dx%d, %d products, offset %d"
                     % (seed, bits, M, K, count, off))


K_FLAT = {2: [512, 768, 1024, 1536, 2048, 3072], 4: [256, 384, 512, 768, 1024, 1536]}


@pytest.mark.parametrize("seed", range(40 * SCALE))
def test_packed_flat_random_cases(seed):
    """Shapes the flat split takes: K with 8 to 48 chunks per row, rows on
    both sides of a workgroup's block, batches of 1 to 65 products (two
    launches past 64) with one shared x or one x each, padded leading
    dimensions and code bases offset by whole chunks; sampled products
    against the oracle, and the last one bit for bit against a single call
    (4-bit) or a second launch of the batch (2-bit)."""
    rng = np.random.default_rng(3000 + seed)
    bits = int(rng.choice([2, 4]))
    K = int(rng.choice(K_FLAT[bits]))
    M = int(rng.integers(1, 3000)) if rng.random() < 0.7 else int(rng.integers(1, 64))
    count = int(rng.choice([1, 2, 5, 40, 65]))
    shared = bool(rng.random() < 0.5)
    pad_q, pad_s = int(rng.choice([0, 16, 48, 5])), int(rng.choice([0, 3]))
    off = int(rng.choice([0, 16, 32]))
    t = torch()
    nb = K * bits // 8
    mats, dQ, dS = [], [], []
    for _ in range(count):
        Q = rng.integers(0, 256, (M, nb + pad_q), dtype=np.uint8)
        S = rng.uniform(0.01, 0.05, (M, K // 64 + pad_s)).astype(np.float16).view(np.uint16)
        mats.append((Q, S))
        buf = t.zeros(off + Q.size, dtype=t.uint8, device="cuda")
        q = buf[off:].view(Q.shape)
        q.copy_(t.from_numpy(Q).to("cuda"))
        dQ.append(q[:, :nb])
        dS.append(dev(S.view(np.int16))[:, :K // 64])
    xs = [inputs.normal(rng, (K,))] * count if shared else [inputs.normal(rng, (K,))
                                                             for _ in range(count)]
    dxs = [dev(xs[0])] * count if shared else [dev(x) for x in xs]
    f1 = bd.gemv_q2 if bits == 2 else bd.gemv_q4
    fb = bd.gemv_q2_batched if bits == 2 else bd.gemv_q4_batched
    ref_fn = oracle.gemv_q2 if bits == 2 else oracle.gemv_q4
    ys = [f1(dQ[0], dS[0], dxs[0])] if count == 1 else fb(dQ, dS, dxs)
    t.cuda.synchronize()
    for b in sorted({0, count // 2, count - 1}):
        Q, S = mats[b]
        ref, bound = ref_fn(Q, S, xs[b], K=K)
        assert_close(host(ys[b]), ref, bound, "seed %d: %d-bit %dx%d, product %d of %d"
                     % (seed, bits, M, K, b, count))
    if count > 1:
        # 4-bit: the single call's bits; 2-bit batches may take the
        # integer-dot kernel, so a second launch's bits
        b = count - 1
        other = f1(dQ[b], dS[b], dxs[b]) if bits == 4 else fb(dQ, dS, dxs)[b]
        assert np.array_equal(host(other), host(ys[b]))
