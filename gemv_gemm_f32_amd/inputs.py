"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module draws random numbers and nothing else: it holds none of the
products' arithmetic, so that both the HIP path and the CPU oracle can take
their inputs from it without sharing any of the method.  Every generator uses
numpy's ``default_rng(seed)`` (PCG64).

Workloads (shapes and value distributions stand in for the pages' own):
  * square products 256^3 and 2048^3 with entries uniform in [-1, 1), the
    sizes of the kernel sweep in "I built a GPT-2 in the browser, then made it
    2.6x-12.1x faster", section "The kernel sweep";
  * the layer products of a GPT-2-small block (d = 768, 1024 tokens = batch 4
    x sequence 256), forward and both backward transposes, weights N(0, 0.02),
    activations and output gradients N(0, 1) (same page, sections "The
    architecture in 60 seconds" and "The kernel sweep");
  * the 346-token classifier prompt times a 768 x 768 dense layer, entries
    uniform in [-1, 1) ("More Stumbling, This Time in the Browser", sections
    "This time, in a browser" and "Four answers per worker");
  * 12,288 x 1,536 matrix-vector products, fp32 and 2-bit, with many distinct
    weight matrices rotated per call so that the weight set is far larger than
    the on-chip caches, and unpatterned random code bytes ("Kernel 0112",
    sections "What is being measured" and "How it is measured").
"""
from __future__ import annotations

import hashlib

import numpy as np

# --------------------------------------------------------------- shapes --

GEMV_M = 12288
GEMV_K = 1536
GEMV_CALLS_PER_TOKEN = 40
GEMV_F32_ROTATION = 48
GEMV_Q2_ROTATION = 128
Q2_GROUP = 64                       # columns per fp16 scale

# GPT-2-small block products: (name, op, M, N, K, operand names).
# op "nn": C = A.B;  "nt": C = A.B^T (B stored N x K);  "tn": C = A^T.B
# (A stored K x M).  Forward Y = X.W, backward dX = dY.W^T, dW = X^T.dY.
GPT2_OPS = (
    ("F1", "nn", 1024, 2304, 768, ("X1", "W1")),
    ("F2", "nn", 1024, 3072, 768, ("X2", "W2")),
    ("F3", "nn", 1024, 768, 3072, ("X3", "W3")),
    ("B1x", "nt", 1024, 768, 2304, ("dY1", "W1")),
    ("B1w", "tn", 768, 2304, 1024, ("X1", "dY1")),
    ("B2x", "nt", 1024, 768, 3072, ("dY2", "W2")),
    ("B2w", "tn", 768, 3072, 1024, ("X2", "dY2")),
    ("B3x", "nt", 1024, 3072, 768, ("dY3", "W3")),
    ("B3w", "tn", 3072, 768, 1024, ("X3", "dY3")),
)


def sha256(*arrays) -> str:
    """Hash of the raw bytes of the given arrays, logged beside results so a
    swapped input cannot pass unnoticed."""
    h = hashlib.sha256()
    for a in arrays:
        a = np.ascontiguousarray(a)
        h.update(str(a.dtype).encode())
        h.update(str(a.shape).encode())
        h.update(a.tobytes())
    return h.hexdigest()


def uniform(rng, shape) -> np.ndarray:
    """fp32 entries uniform in [-1, 1)."""
    return (rng.random(shape, dtype=np.float32) * np.float32(2.0)
            - np.float32(1.0))


def normal(rng, shape, std=1.0) -> np.ndarray:
    """fp32 entries N(0, std^2)."""
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def integers(rng, shape, lo=-8, hi=8) -> np.ndarray:
    """fp32 matrix of integers in [lo, hi]."""
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


# -------------------------------------------------------------- configs --

def tiny_case():
    """The 3 x 4 by 4 x 2 integer-valued product that is checked by hand."""
    A = np.array([[1, 2, 3, 4], [5, 6, 7, 8], [9, 10, 11, 12]], np.float32)
    B = np.array([[1, 0], [0, 1], [1, 1], [2, -1]], np.float32)
    return A, B


def square_pair(n: int, seed: int):
    """A, B (n x n), uniform [-1, 1), drawn A then B from one generator."""
    rng = np.random.default_rng(seed)
    A = uniform(rng, (n, n))
    B = uniform(rng, (n, n))
    return A, B


def small_square(seed: int = 0):
    return square_pair(256, seed)


def large_square(seed: int = 3):
    return square_pair(2048, seed)


def classifier(seed: int = 33):
    """346 x 768 prompt activations times a 768 x 768 dense layer."""
    rng = np.random.default_rng(seed)
    A = uniform(rng, (346, 768))
    B = uniform(rng, (768, 768))
    return A, B


def gpt2_tensors(seed: int = 2):
    """The nine operands of a GPT-2-small block's products, in a fixed draw
    order.  X, dY ~ N(0, 1); W ~ N(0, 0.02)."""
    rng = np.random.default_rng(seed)
    t = {}
    t["X1"] = normal(rng, (1024, 768))
    t["W1"] = normal(rng, (768, 2304), 0.02)
    t["dY1"] = normal(rng, (1024, 2304))
    t["X2"] = normal(rng, (1024, 768))
    t["W2"] = normal(rng, (768, 3072), 0.02)
    t["dY2"] = normal(rng, (1024, 3072))
    t["X3"] = normal(rng, (1024, 3072))
    t["W3"] = normal(rng, (3072, 768), 0.02)
    t["dY3"] = normal(rng, (1024, 768))
    return t


def gemv_f32_weight(r: int, M: int = GEMV_M, K: int = GEMV_K) -> np.ndarray:
    """Rotation matrix r of the fp32 GEMV set: 0.02 * N(0, 1)."""
    rng = np.random.default_rng(4000 + r)
    return normal(rng, (M, K), 0.02)


def gemv_f32_x(K: int = GEMV_K) -> np.ndarray:
    return normal(np.random.default_rng(4999), (K,))


def q2_weight(r: int, M: int = GEMV_M, K: int = GEMV_K):
    """Rotation matrix r of the 2-bit set: (Q, S).

    Q: uint8 M x ceil(K/4), i.i.d. uniform random bytes (every 2-bit code
       equally likely, no pattern).
    S: uint16 M x ceil(K/64), the binary16 bit patterns of scales drawn
       uniform in [0.01, 0.05) and rounded to binary16 (nearest even); the
       stored half is the scale for both sides.
    """
    rng = np.random.default_rng(5000 + r)
    Q = rng.integers(0, 256, size=(M, (K + 3) // 4), dtype=np.uint8)
    S = rng.uniform(0.01, 0.05, size=(M, (K + Q2_GROUP - 1) // Q2_GROUP))
    S = S.astype(np.float16).view(np.uint16)
    return Q, S


def q4_weight(r: int, M: int = GEMV_M, K: int = GEMV_K):
    """Rotation matrix r of the 4-bit set: (Q, S), drawn like the 2-bit set.

    Q: uint8 M x ceil(K/2), i.i.d. uniform random bytes (every 4-bit code
       equally likely).
    S: uint16 M x ceil(K/64), binary16 bit patterns of scales drawn uniform
       in [0.01, 0.05) and rounded to binary16.
    """
    rng = np.random.default_rng(6000 + r)
    Q = rng.integers(0, 256, size=(M, (K + 1) // 2), dtype=np.uint8)
    S = rng.uniform(0.01, 0.05, size=(M, (K + Q2_GROUP - 1) // Q2_GROUP))
    S = S.astype(np.float16).view(np.uint16)
    return Q, S


def q2_x(K: int = GEMV_K) -> np.ndarray:
    return normal(np.random.default_rng(5999), (K,))
