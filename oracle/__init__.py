"""CPU oracle for the dense fp32 product, the fp32 GEMV and the 2-bit and
4-bit GEMVs.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``gemv_gemm_f32_amd``) never imports it, and this package imports nothing from
the product path: the two share only the seeded input generators.

The arithmetic lives in ``oracle.c`` (plain C, IEEE binary64 sums in the order
k = 0..K-1); this module only builds it with gcc, loads it with ctypes and
marshals numpy arrays.  Each function returns ``(value, bound)`` where
``bound = sum_k |a_ik * b_kj|`` is the scale of the acceptance test
``|gpu - value| <= 1e-4 * bound``.

Definitions followed (the pages):
  * "More Stumbling, This Time in the Browser", section "Four answers per
    worker": an output cell walks the inner dimension, multiplying each
    activation by its weight and adding the products.
  * "I built a GPT-2 in the browser, then made it 2.6x-12.1x faster",
    section "The architecture in 60 seconds": backward passes derived by hand,
    so dX = dY.W^T (``gemm_nt``) and dW = X^T.dY (``gemm_tn``).
  * "Kernel 0112", sections "What is being measured" and "The kernel": a
    12,288 x 1,536 matrix of 2-bit weights times a vector of 1,536 inputs, the
    2-bit fields unpacked to floating point; bit order, code map and scale
    layout are readings (see ``oracle.c``).
  * The 4-bit matrices of the same page's patch set (kernels 0099 and 0105)
    and the packed NF4 path of "More Stumbling, This Time in the Browser":
    4-bit weights with no format given; the reading (nibbles least
    significant first, w = (code - 7.5) * s, one binary16 scale per 64
    columns) is in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into oracle/liboracle.so (no fast-math, so the
    fp64 sums keep their written order)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                               "-fno-fast-math", "-ffp-contract=off",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized(path: str) -> str:
    """Compile oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer
    (any finding aborts) into `path`, for the sanitizer test; load it by
    setting ORACLE_LIB=path in a process that preloads the gcc sanitizer
    runtimes."""
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared",
                           "-fno-fast-math", "-ffp-contract=off",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", _SRC, "-o", path, "-lm"])
    return path


def _load():
    global _lib
    if _lib is not None:
        return _lib
    alt = os.environ.get("ORACLE_LIB")
    if alt:
        # another build of oracle.c (the sanitizer test's), used as is
        _lib = bind(ctypes.CDLL(alt))
        return _lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build(force=True)
    _lib = bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def bind(lib):
    """Declare the C signatures on a loaded copy of oracle.c."""
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    for name in ("oracle_gemm_nn", "oracle_gemm_tn", "oracle_gemm_nt"):
        f = getattr(lib, name)
        f.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, vp, i64]
        f.restype = None
    lib.oracle_gemm_cells.argtypes = [i32, i32, i64, vp, i64, vp, i64, i64,
                                      vp, vp, vp, vp]
    lib.oracle_gemm_cells.restype = None
    lib.oracle_gemv.argtypes = [i64, i64, vp, i64, vp, vp, vp]
    lib.oracle_gemv.restype = None
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_q2_unpack_row.argtypes = [i64, i64, vp, i64, vp, i64, vp]
    lib.oracle_q2_unpack_row.restype = None
    lib.oracle_gemv_q2.argtypes = [i64, i64, vp, i64, vp, i64, vp, vp, vp, vp]
    lib.oracle_gemv_q2.restype = None
    dbl = ctypes.c_double
    lib.oracle_gemm_ex.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, dbl, vp, i64,
                                   vp, i64, dbl, vp, i64, vp, vp]
    lib.oracle_gemm_ex.restype = None
    lib.oracle_q4_unpack_row.argtypes = [i64, i64, vp, i64, vp, i64, vp]
    lib.oracle_q4_unpack_row.restype = None
    lib.oracle_gemv_q4.argtypes = [i64, i64, vp, i64, vp, i64, vp, vp, vp, vp]
    lib.oracle_gemv_q4.restype = None
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _as2d(a, dtype):
    """Row-major 2-D view with unit inner stride; returns (array, ld)."""
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (dtype, a.dtype))
    if a.ndim != 2:
        raise ValueError("expected a 2-D array")
    if a.strides[1] != a.itemsize or a.strides[0] % a.itemsize:
        a = np.ascontiguousarray(a)
    return a, a.strides[0] // a.itemsize


def _gemm(fname, A, B, M, N, K):
    lib = _load()
    A, lda = _as2d(A, np.float32)
    B, ldb = _as2d(B, np.float32)
    C = np.zeros((M, N), np.float64)
    bound = np.zeros((M, N), np.float64)
    getattr(lib, fname)(M, N, K, _ptr(A), lda, _ptr(B), ldb,
                        _ptr(C), _ptr(bound), N)
    return C, bound


def gemm_nn(A, B):
    """C = A.B, A (M x K), B (K x N) fp32 row-major. Returns (C, bound) fp64."""
    M, K = np.shape(A)
    K2, N = np.shape(B)
    if K2 != K:
        raise ValueError("inner dimensions differ")
    return _gemm("oracle_gemm_nn", A, B, M, N, K)


def gemm_tn(A, B):
    """C = A^T.B with A stored K x M and B stored K x N."""
    K, M = np.shape(A)
    K2, N = np.shape(B)
    if K2 != K:
        raise ValueError("inner dimensions differ")
    return _gemm("oracle_gemm_tn", A, B, M, N, K)


def gemm_nt(A, B):
    """C = A.B^T with A stored M x K and B stored N x K."""
    M, K = np.shape(A)
    N, K2 = np.shape(B)
    if K2 != K:
        raise ValueError("inner dimensions differ")
    return _gemm("oracle_gemm_nt", A, B, M, N, K)


def gemm_cells(A, B, rows, cols, trans_a=False, trans_b=False):
    """Selected cells (rows[q], cols[q]) of op(A).op(B), each one plain dot
    product over k.  Returns (values, bounds) as fp64 vectors."""
    lib = _load()
    A, lda = _as2d(A, np.float32)
    B, ldb = _as2d(B, np.float32)
    K = A.shape[0] if trans_a else A.shape[1]
    Kb = B.shape[1] if trans_b else B.shape[0]
    if K != Kb:
        raise ValueError("inner dimensions differ")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    Mdim = A.shape[1] if trans_a else A.shape[0]
    Ndim = B.shape[0] if trans_b else B.shape[1]
    if rows.shape != cols.shape or (rows.size and (
            rows.min() < 0 or rows.max() >= Mdim or
            cols.min() < 0 or cols.max() >= Ndim)):
        raise ValueError("cell index out of range")
    c = np.zeros(rows.size, np.float64)
    b = np.zeros(rows.size, np.float64)
    lib.oracle_gemm_cells(int(trans_a), int(trans_b), K, _ptr(A), lda,
                          _ptr(B), ldb, rows.size, _ptr(rows), _ptr(cols),
                          _ptr(c), _ptr(b))
    return c, b


def gemm_ex(A, B, C=None, alpha=1.0, beta=0.0, trans_a=False, trans_b=False):
    """alpha * op(A).op(B) + beta * C (C is not read when beta == 0), with
    op(A) = A^T if trans_a and op(B) = B^T if trans_b; alpha and beta are
    taken as fp32 values.  Returns (values, bounds) as M x N fp64 arrays."""
    lib = _load()
    A, lda = _as2d(A, np.float32)
    B, ldb = _as2d(B, np.float32)
    M = A.shape[1] if trans_a else A.shape[0]
    K = A.shape[0] if trans_a else A.shape[1]
    Kb = B.shape[1] if trans_b else B.shape[0]
    N = B.shape[0] if trans_b else B.shape[1]
    if K != Kb:
        raise ValueError("inner dimensions differ")
    alpha = float(np.float32(alpha))
    beta = float(np.float32(beta))
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs C")
        C = np.full((M, N), np.nan, np.float32)     # never read when beta == 0
    C, ldc = _as2d(C, np.float32)
    if C.shape != (M, N):
        raise ValueError("C must be M x N")
    out = np.zeros((M, N), np.float64)
    bnd = np.zeros((M, N), np.float64)
    lib.oracle_gemm_ex(int(trans_a), int(trans_b), M, N, K, alpha, _ptr(A), lda,
                       _ptr(B), ldb, beta, _ptr(C), ldc, _ptr(out), _ptr(bnd))
    return out, bnd


def gemv(W, x):
    """y = W.x, W (M x K) fp32 row-major, x (K,) fp32. Returns (y, bound)."""
    lib = _load()
    W, ldw = _as2d(W, np.float32)
    M, K = W.shape
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.shape != (K,):
        raise ValueError("x must have K entries")
    y = np.zeros(M, np.float64)
    b = np.zeros(M, np.float64)
    lib.oracle_gemv(M, K, _ptr(W), ldw, _ptr(x), _ptr(y), _ptr(b))
    return y, b


def half_to_double(h: int) -> float:
    """IEEE binary16 bit pattern -> float, decoded from the format definition."""
    return _load().oracle_half_to_double(int(h) & 0xFFFF)


def _q2_args(Q, S, K):
    Q, ldq = _as2d(Q, np.uint8)
    S, lds = _as2d(S, np.uint16)
    M = Q.shape[0]
    if S.shape[0] != M:
        raise ValueError("Q and S must have the same number of rows")
    if ldq < (K + 3) // 4 or Q.shape[1] < (K + 3) // 4:
        raise ValueError("Q rows hold fewer than ceil(K/4) bytes")
    if lds < (K + 63) // 64 or S.shape[1] < (K + 63) // 64:
        raise ValueError("S rows hold fewer than ceil(K/64) scales")
    return Q, ldq, S, lds, M


def q2_unpack(Q, S, K):
    """The dequantised matrix (M x K, fp64): w = (code - 1.5) * s."""
    lib = _load()
    Q, ldq, S, lds, M = _q2_args(Q, S, K)
    W = np.zeros((M, K), np.float64)
    for i in range(M):
        lib.oracle_q2_unpack_row(i, K, _ptr(Q), ldq, _ptr(S), lds,
                                 _ptr(W[i]))
    return W


def gemv_q2(Q, S, x, K=None):
    """y = W.x for the 2-bit matrix (Q codes uint8 M x ceil(K/4),
    S binary16 bit patterns uint16 M x ceil(K/64), x fp32 (K,))."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    if K is None:
        K = x.shape[0]
    if x.shape != (K,):
        raise ValueError("x must have K entries")
    Q, ldq, S, lds, M = _q2_args(Q, S, K)
    y = np.zeros(M, np.float64)
    b = np.zeros(M, np.float64)
    w = np.zeros(max(K, 1), np.float64)
    lib.oracle_gemv_q2(M, K, _ptr(Q), ldq, _ptr(S), lds, _ptr(x),
                       _ptr(y), _ptr(b), _ptr(w))
    return y, b


def _q4_args(Q, S, K):
    Q, ldq = _as2d(Q, np.uint8)
    S, lds = _as2d(S, np.uint16)
    M = Q.shape[0]
    if S.shape[0] != M:
        raise ValueError("Q and S must have the same number of rows")
    if ldq < (K + 1) // 2 or Q.shape[1] < (K + 1) // 2:
        raise ValueError("Q rows hold fewer than ceil(K/2) bytes")
    if lds < (K + 63) // 64 or S.shape[1] < (K + 63) // 64:
        raise ValueError("S rows hold fewer than ceil(K/64) scales")
    return Q, ldq, S, lds, M


def q4_unpack(Q, S, K):
    """The dequantised 4-bit matrix (M x K, fp64): w = (code - 7.5) * s."""
    lib = _load()
    Q, ldq, S, lds, M = _q4_args(Q, S, K)
    W = np.zeros((M, K), np.float64)
    for i in range(M):
        lib.oracle_q4_unpack_row(i, K, _ptr(Q), ldq, _ptr(S), lds,
                                 _ptr(W[i]))
    return W


def gemv_q4(Q, S, x, K=None):
    """y = W.x for the 4-bit matrix (Q codes uint8 M x ceil(K/2),
    S binary16 bit patterns uint16 M x ceil(K/64), x fp32 (K,))."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    if K is None:
        K = x.shape[0]
    if x.shape != (K,):
        raise ValueError("x must have K entries")
    Q, ldq, S, lds, M = _q4_args(Q, S, K)
    y = np.zeros(M, np.float64)
    b = np.zeros(M, np.float64)
    w = np.zeros(max(K, 1), np.float64)
    lib.oracle_gemv_q4(M, K, _ptr(Q), ldq, _ptr(S), lds, _ptr(x),
                       _ptr(y), _ptr(b), _ptr(w))
    return y, b


def check(value_gpu, value_ref, bound, rel=1e-4):
    """Acceptance test, per element: |gpu - ref| <= rel * bound, finite gpu,
    and gpu == +-0 where bound == 0.  Returns (ok, worst_ratio, worst_index)
    with ratio = |gpu - ref| / bound (inf where bound == 0 and gpu != 0)."""
    g = np.asarray(value_gpu, np.float64)
    r = np.asarray(value_ref, np.float64)
    b = np.asarray(bound, np.float64)
    if g.shape != r.shape or r.shape != b.shape:
        raise ValueError("shape mismatch %s %s %s" % (g.shape, r.shape, b.shape))
    if g.size == 0:
        return True, 0.0, None
    err = np.abs(g - r)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(b > 0, err / np.where(b > 0, b, 1.0),
                         np.where(err == 0, 0.0, np.inf))
    ratio = np.where(np.isfinite(g), ratio, np.inf)
    idx = int(np.argmax(ratio))
    worst = float(ratio.flat[idx])
    return bool(worst <= rel), worst, np.unravel_index(idx, g.shape)
