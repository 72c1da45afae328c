"""MI355X (gfx950) fp32 GEMM, fp32 GEMV and 2-bit GEMV through a C ABI.

The kernels and the C entry points live in ``csrc/`` and build into
``libgemvgemm.so``; ``gemv_gemm_f32_amd.binding`` loads that library with
ctypes and exposes the same entry points on torch tensors.  Importing this
package loads nothing: the library is opened on first use, and a missing
library is an error, never a fallback.
"""

__all__ = ["binding", "inputs"]


def __getattr__(name):
    if name in ("gemm_f32", "gemm_f32_tn", "gemm_f32_nt", "gemv_f32",
                "gemv_q2", "GGError"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
