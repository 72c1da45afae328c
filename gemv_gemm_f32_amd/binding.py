"""ctypes binding of libgemvgemm.so: the C entry points on torch tensors.

Argument marshalling only: every step of every product runs in the HIP
kernels behind the C ABI (include/gemvgemm.h).  torch supplies device memory
and the current stream.  If the library has not been built this module
raises; there is no fallback of any kind.

Each tensor function has the name of its C entry point and takes row-major
2-D tensors whose last dimension is contiguous; the row stride is passed as
the leading dimension.  The output is written in place (allocated when not
given) and returned.  A non-zero status raises ``GGError``.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgemvgemm.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "gemvgemm.h")

GG_OK = 0
GG_ERR_INVALID_ARG = -1
GG_ERR_ALIAS = -2
GG_ERR_NO_DEVICE = -3
GG_ERR_LAUNCH = -4
GG_ERR_SCRATCH = -5

ENTRY_POINTS = ("gemm_f32", "gemm_f32_tn", "gemm_f32_nt", "gemm_f32_ex", "gemv_f32",
                "gemv_f32_batched", "gemv_q2", "gemv_q2_batched", "gemv_q2_batched_ws",
                "gemv_q2_batched_ws_size", "gemv_q2_batched_noalloc", "gemv_q4",
                "gemv_q4_batched", "gg_strerror")

_lib = None


class GGError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, strerror(status), status))


def load(path: str = LIB_PATH):
    """Open the library (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    # torch ships its own HIP runtime (soname libamdhip64.so.7).  Importing it
    # first makes this library's libamdhip64.so.7 dependency resolve to that
    # already-loaded copy, so torch's streams and allocations and these
    # kernels live in one runtime.  (Loaded first on its own, the library
    # would pull in a second runtime, and torch's stream handles would be
    # meaningless to it.)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise RuntimeError(
            "libgemvgemm.so is not built (%s); run `python -m gemv_gemm_f32_amd.build`"
            % path)
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    for name in ("gemm_f32", "gemm_f32_tn", "gemm_f32_nt"):
        f = getattr(lib, name)
        f.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp]
        f.restype = ctypes.c_int
    f32 = ctypes.c_float
    lib.gemm_f32_ex.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, f32, vp, i64,
                                vp, i64, f32, vp, i64, vp]
    lib.gemm_f32_ex.restype = ctypes.c_int
    lib.gemv_f32.argtypes = [i64, i64, vp, i64, vp, vp, vp]
    lib.gemv_f32.restype = ctypes.c_int
    pp = ctypes.POINTER(ctypes.c_void_p)
    lib.gemv_f32_batched.argtypes = [i64, i64, i64, pp, i64, pp, pp, vp]
    lib.gemv_f32_batched.restype = ctypes.c_int
    for name in ("gemv_q2", "gemv_q4"):
        f = getattr(lib, name)
        f.argtypes = [i64, i64, vp, i64, vp, i64, vp, vp, vp]
        f.restype = ctypes.c_int
        f = getattr(lib, name + "_batched")
        f.argtypes = [i64, i64, i64, pp, i64, pp, i64, pp, pp, vp]
        f.restype = ctypes.c_int
    lib.gemv_q2_batched_ws.argtypes = [i64, i64, i64, pp, i64, pp, i64, pp, pp, vp, i64, vp]
    lib.gemv_q2_batched_ws.restype = ctypes.c_int
    lib.gemv_q2_batched_noalloc.argtypes = [i64, i64, i64, pp, i64, pp, i64, pp, pp, vp]
    lib.gemv_q2_batched_noalloc.restype = ctypes.c_int
    lib.gemv_q2_batched_ws_size.argtypes = [i64, i64, i64]
    lib.gemv_q2_batched_ws_size.restype = i64
    lib.gg_strerror.argtypes = [ctypes.c_int]
    lib.gg_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().gg_strerror(int(status)).decode()


def header_functions(path: str = HEADER):
    """Names of the functions declared in the public header."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


# ------------------------------------------------------------ tensor side --

def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _mat(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device" % name)
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("%s must have a contiguous last dimension" % name)
    ld = t.stride(0) if t.shape[0] > 1 else max(t.shape[1], 1)
    return t.data_ptr(), ld


def _vec(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.device.type != "cuda":
        raise TypeError("%s must be a %s GPU tensor" % (name, dtype))
    if t.dim() != 1 or (t.numel() > 1 and t.stride(0) != 1):
        raise ValueError("%s must be a contiguous vector" % name)
    return t.data_ptr()


def _check(status, where):
    if status != GG_OK:
        raise GGError(status, where)


def _gemm(name, A, B, C, M, N, K, stream):
    torch = _torch()
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    if tuple(C.shape) != (M, N):
        raise ValueError("C must be %d x %d" % (M, N))
    pa, lda = _mat(A, torch.float32, "A")
    pb, ldb = _mat(B, torch.float32, "B")
    pc, ldc = _mat(C, torch.float32, "C")
    _check(getattr(load(), name)(M, N, K, pa, lda, pb, ldb, pc, ldc, _stream(stream)), name)
    return C


def gemm_f32(A, B, C=None, stream=None):
    """C = A.B with A (M x K) and B (K x N)."""
    M, K = A.shape
    if B.shape[0] != K:
        raise ValueError("inner dimensions differ")
    return _gemm("gemm_f32", A, B, C, M, B.shape[1], K, stream)


def gemm_f32_tn(A, B, C=None, stream=None):
    """C = A^T.B with A stored K x M and B (K x N)."""
    K, M = A.shape
    if B.shape[0] != K:
        raise ValueError("inner dimensions differ")
    return _gemm("gemm_f32_tn", A, B, C, M, B.shape[1], K, stream)


def gemm_f32_nt(A, B, C=None, stream=None):
    """C = A.B^T with A (M x K) and B stored N x K."""
    M, K = A.shape
    if B.shape[1] != K:
        raise ValueError("inner dimensions differ")
    return _gemm("gemm_f32_nt", A, B, C, M, B.shape[0], K, stream)


def gemm_f32_ex(A, B, C=None, alpha=1.0, beta=0.0, trans_a=False, trans_b=False,
                stream=None):
    """C = alpha * op(A).op(B) + beta * C in place (C is not read when beta
    == 0; a new C is allocated when None, which needs beta == 0).  op(A) =
    A^T when trans_a (A stored K x M), op(B) = B^T when trans_b."""
    torch = _torch()
    M = A.shape[1] if trans_a else A.shape[0]
    K = A.shape[0] if trans_a else A.shape[1]
    Kb = B.shape[1] if trans_b else B.shape[0]
    N = B.shape[0] if trans_b else B.shape[1]
    if K != Kb:
        raise ValueError("inner dimensions differ")
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs C")
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    if tuple(C.shape) != (M, N):
        raise ValueError("C must be M x N")
    pa, lda = _mat(A, torch.float32, "A")
    pb, ldb = _mat(B, torch.float32, "B")
    pc, ldc = _mat(C, torch.float32, "C")
    _check(load().gemm_f32_ex(int(bool(trans_a)), int(bool(trans_b)), M, N, K, float(alpha),
                              pa, lda, pb, ldb, float(beta), pc, ldc, _stream(stream)),
           "gemm_f32_ex")
    return C


def gemv_f32(W, x, y=None, stream=None):
    """y = W.x with W (M x K) fp32 and x (K,) fp32."""
    torch = _torch()
    M, K = W.shape
    if x.shape != (K,):
        raise ValueError("x must have K entries")
    if y is None:
        y = torch.empty(M, dtype=torch.float32, device=W.device)
    if y.shape != (M,):
        raise ValueError("y must have M entries")
    pw, ldw = _mat(W, torch.float32, "W")
    _check(load().gemv_f32(M, K, pw, ldw, _vec(x, torch.float32, "x"),
                           _vec(y, torch.float32, "y"), _stream(stream)), "gemv_f32")
    return y


def gemv_f32_batched(Ws, xs, ys=None, stream=None):
    """y_b = W_b.x_b for every b: lists of W (fp32 M x K, one shape and
    leading dimension for all) and x (K,) fp32.  Returns the list of
    outputs."""
    torch = _torch()
    n = len(Ws)
    if len(xs) != n:
        raise ValueError("Ws and xs must have the same length")
    if n == 0:
        return []
    M, K = Ws[0].shape
    if ys is None:
        ys = [torch.empty(M, dtype=torch.float32, device=Ws[0].device) for _ in range(n)]
    wp, xp, yp, ldw = [], [], [], None
    for W, x, y in zip(Ws, xs, ys):
        if tuple(W.shape) != (M, K) or x.shape != (K,) or y.shape != (M,):
            raise ValueError("every product must have the same M and K")
        pw, lw = _mat(W, torch.float32, "W")
        if ldw is None:
            ldw = lw
        elif lw != ldw:
            raise ValueError("every W must have the same leading dimension")
        wp.append(pw)
        xp.append(_vec(x, torch.float32, "x"))
        yp.append(_vec(y, torch.float32, "y"))
    _check(load().gemv_f32_batched(n, M, K, _ptr_array(wp), ldw, _ptr_array(xp),
                                   _ptr_array(yp), _stream(stream)), "gemv_f32_batched")
    return ys


def _packed(name, Q, S, x, y, stream):
    torch = _torch()
    M = Q.shape[0]
    K = x.shape[0]
    if S.shape[0] != M:
        raise ValueError("Q and S must have the same number of rows")
    if S.dtype in (torch.float16, torch.int16):
        S = S.view(torch.float16)
    else:
        raise TypeError("S must hold binary16 bit patterns (float16 or int16)")
    if y is None:
        y = torch.empty(M, dtype=torch.float32, device=Q.device)
    if y.shape != (M,):
        raise ValueError("y must have M entries")
    pq, ldq = _mat(Q, torch.uint8, "Q")
    ps, lds = _mat(S, torch.float16, "S")
    _check(getattr(load(), name)(M, K, pq, ldq, ps, lds, _vec(x, torch.float32, "x"),
                                 _vec(y, torch.float32, "y"), _stream(stream)), name)
    return y


def gemv_q2(Q, S, x, y=None, stream=None):
    """y = W.x with W as 2-bit codes Q (uint8, M x >= ceil(K/4)) and binary16
    scales S (float16 or int16 bit patterns, M x >= ceil(K/64)); x (K,) fp32."""
    return _packed("gemv_q2", Q, S, x, y, stream)


def gemv_q4(Q, S, x, y=None, stream=None):
    """y = W.x with W as 4-bit codes Q (uint8, M x >= ceil(K/2)) and binary16
    scales S (float16 or int16 bit patterns, M x >= ceil(K/64)); x (K,) fp32."""
    return _packed("gemv_q4", Q, S, x, y, stream)


def _ptr_array(ptrs):
    arr = (ctypes.c_void_p * max(len(ptrs), 1))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return arr


def _packed_batched(name, Qs, Ss, xs, ys, stream, ws=None):
    torch = _torch()
    n = len(Qs)
    if len(Ss) != n or len(xs) != n:
        raise ValueError("Qs, Ss and xs must have the same length")
    if n == 0:
        return []
    M, K = Qs[0].shape[0], xs[0].shape[0]
    if ys is None:
        ys = [torch.empty(M, dtype=torch.float32, device=Qs[0].device) for _ in range(n)]
    qp, sp, xp, yp, ldq, lds = [], [], [], [], None, None
    for Q, S, x, y in zip(Qs, Ss, xs, ys):
        if Q.shape[0] != M or S.shape[0] != M or x.shape != (K,) or y.shape != (M,):
            raise ValueError("every product must have the same M and K")
        if S.dtype not in (torch.float16, torch.int16):
            raise TypeError("S must hold binary16 bit patterns (float16 or int16)")
        pq, lq = _mat(Q, torch.uint8, "Q")
        ps, ls = _mat(S.view(torch.float16), torch.float16, "S")
        if ldq is None:
            ldq, lds = lq, ls
        elif (lq, ls) != (ldq, lds):
            raise ValueError("every Q (and every S) must have the same leading dimension")
        qp.append(pq)
        sp.append(ps)
        xp.append(_vec(x, torch.float32, "x"))
        yp.append(_vec(y, torch.float32, "y"))
    args = [n, M, K, _ptr_array(qp), ldq, _ptr_array(sp), lds, _ptr_array(xp), _ptr_array(yp)]
    if ws is not None:
        if ws.numel() and (ws.device.type != "cuda" or not ws.is_contiguous()):
            raise ValueError("the workspace must be a contiguous GPU tensor")
        args += [ws.data_ptr() if ws.numel() else None, ws.numel() * ws.element_size()]
    _check(getattr(load(), name)(*args, _stream(stream)), name)
    return ys


def gemv_q2_batched(Qs, Ss, xs, ys=None, stream=None):
    """y_b = W_b.x_b for every b: lists of Q (uint8 M x >= ceil(K/4)), S
    (float16/int16 M x >= ceil(K/64)), x (K,) fp32; all Q share one shape and
    leading dimension, as do all S.  Returns the list of outputs."""
    return _packed_batched("gemv_q2_batched", Qs, Ss, xs, ys, stream)


def gemv_q2_batched_ws_size(count, M, K):
    """Bytes of workspace gemv_q2_batched_ws needs for count products of M x K."""
    n = load().gemv_q2_batched_ws_size(count, M, K)
    if n < 0:
        raise GGError(n, "gemv_q2_batched_ws_size")
    return n


def gemv_q2_batched_ws(Qs, Ss, xs, ys=None, workspace=None, stream=None):
    """gemv_q2_batched with a workspace (a contiguous GPU tensor of at least
    gemv_q2_batched_ws_size bytes; allocated here as uint8 when None)."""
    torch = _torch()
    if workspace is None:
        n = gemv_q2_batched_ws_size(len(Qs), Qs[0].shape[0] if Qs else 0,
                                    xs[0].shape[0] if xs else 0)
        workspace = torch.empty(n, dtype=torch.uint8, device=Qs[0].device if Qs else "cuda")
    return _packed_batched("gemv_q2_batched_ws", Qs, Ss, xs, ys, stream, ws=workspace)


def gemv_q2_batched_noalloc(Qs, Ss, xs, ys=None, stream=None):
    """gemv_q2_batched_ws on the library's fixed per-GPU scratch buffer
    instead of a workspace (outputs are allocated here when ys is None)."""
    return _packed_batched("gemv_q2_batched_noalloc", Qs, Ss, xs, ys, stream)


def gemv_q4_batched(Qs, Ss, xs, ys=None, stream=None):
    """As gemv_q2_batched for 4-bit codes (Q uint8 M x >= ceil(K/2))."""
    return _packed_batched("gemv_q4_batched", Qs, Ss, xs, ys, stream)
