"""The packed GEMVs with x far from 1, element by element against the oracle.

The header guarantees the tolerance for finite x whose largest entry lies in
[2^-100, 2^100] in magnitude (entries far below the largest may underflow in
partial products, which moves the sum by far less than the bound).  Every
kernel that serves 12,288 x 1,536 and the other shapes is checked at 2^96,
2^60, 2^-60 and 2^-100 times N(0, 1) inputs: single products and batches,
2-bit and 4-bit, on the flat shapes (K = 768 and 1536), a ragged shape that
takes the row-split kernel (K = 1000) and the transposed shape (K = 12,288).
"""
import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import binding as bd
from gemv_gemm_f32_amd import inputs
from gpu_util import assert_close, dev, host

pytestmark = pytest.mark.gpu

SCALES = (2.0 ** 96, 2.0 ** 60, 2.0 ** -60, 2.0 ** -100)


def _case(bits, M, K, scale, seed):
    rng = np.random.default_rng(seed)
    nb = (K * bits + 7) // 8
    Q = rng.integers(0, 256, (M, nb), dtype=np.uint8)
    S = rng.uniform(0.01, 0.05, (M, (K + 63) // 64)).astype(np.float16).view(np.uint16)
    x = (inputs.normal(rng, (K,)).astype(np.float64) * scale).astype(np.float32)
    return Q, S, x


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("bits,M,K", [(2, 12288, 1536), (2, 1000, 768), (2, 777, 1000),
                                      (2, 1536, 12288), (4, 12288, 1536), (4, 999, 1000)])
def test_single_and_batched(bits, M, K, scale):
    seed = int(np.log2(scale)) + 1000 * bits + M + K
    Q, S, x = _case(bits, M, K, scale, seed)
    Q2, S2, x2 = _case(bits, M, K, scale, seed + 1)
    f1 = bd.gemv_q2 if bits == 2 else bd.gemv_q4
    fb = bd.gemv_q2_batched if bits == 2 else bd.gemv_q4_batched
    ref_fn = oracle.gemv_q2 if bits == 2 else oracle.gemv_q4
    ref, bound = ref_fn(Q, S, x)
    what = "%d-bit %dx%d, x scaled by 2^%d" % (bits, M, K, int(np.log2(scale)))
    y = host(f1(dev(Q), dev(S.view(np.int16)), dev(x)))
    assert np.all(np.isfinite(y)), what
    assert_close(y, ref, bound, what + ", single")
    ys = fb([dev(Q2), dev(Q)], [dev(S2.view(np.int16)), dev(S.view(np.int16))], [dev(x2), dev(x)])
    assert_close(host(ys[1]), ref, bound, what + ", batched")
    ref2, bound2 = ref_fn(Q2, S2, x2)
    assert_close(host(ys[0]), ref2, bound2, what + ", batched neighbour")
