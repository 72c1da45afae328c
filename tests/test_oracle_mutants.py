"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle/oracle.c, plants one plausible slip (a transposed
index, a dropped term, a wrong sign, bit order or scale index, a wrong
binary16 bias), builds the copy with gcc into a temporary directory, swaps it
in for the real oracle and runs a compact battery of the pins of
test_oracle.py.  The battery must pass on the real oracle and fail on every
mutant.  Everything here runs on the CPU.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from gemv_gemm_f32_amd import inputs
from golden_io import load

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "nn_reads_A_transposed": ("double a = (double)A[i * lda + k];\n            const float *brow = B + k * ldb;",
                              "double a = (double)A[k * lda + i];\n            const float *brow = B + k * ldb;"),
    "tn_reads_A_untransposed": ("double a = (double)A[k * lda + i];\n            const float *brow",
                                "double a = (double)A[i * lda + k];\n            const float *brow"),
    "nt_reads_B_untransposed": ("(double)A[i * lda + k] * (double)B[j * ldb + k]",
                                "(double)A[i * lda + k] * (double)B[k * ldb + j]"),
    "nn_drops_last_term": ("for (int64_t k = 0; k < K; ++k) {\n            double a = (double)A[i * lda + k];",
                           "for (int64_t k = 0; k + 1 < K; ++k) {\n            double a = (double)A[i * lda + k];"),
    "bound_signed": ("c[j] += p;\n                b[j] += fabs(p);",
                     "c[j] += p;\n                b[j] += p;"),
    "gemv_wrong_x_index": ("(double)W[i * ldw + k] * (double)x[k]",
                           "(double)W[i * ldw + k] * (double)x[K - 1 - k]"),
    "q2_sign_flipped": ("w[k] = ((double)code - 1.5) * s;", "w[k] = (1.5 - (double)code) * s;"),
    "q2_offset_wrong": ("w[k] = ((double)code - 1.5) * s;", "w[k] = ((double)code - 2.0) * s;"),
    "q2_bit_order_msb_first": ("(byte >> (2 * (k % 4))) & 3u", "(byte >> (6 - 2 * (k % 4))) & 3u"),
    "q2_scale_index": ("S[i * lds + k / 64]", "S[i * lds + k / 32]"),
    "q2_byte_index": ("Q[i * ldq + k / 4]", "Q[i * ldq + k / 8]"),
    "half_bias": ("e - 25", "e - 24"),
    "half_subnormal": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "q2_dot_drops_first": ("for (int64_t k = 0; k < K; ++k) {\n            double p = w[k]",
                           "for (int64_t k = 1; k < K; ++k) {\n            double p = w[k]"),
    "q4_sign_flipped": ("w[k] = ((double)code - 7.5) * s;", "w[k] = (7.5 - (double)code) * s;"),
    "q4_offset_wrong": ("w[k] = ((double)code - 7.5) * s;", "w[k] = ((double)code - 8.0) * s;"),
    "q4_nibble_order_msb_first": ("(byte >> (4 * (k % 2))) & 15u", "(byte >> (4 - 4 * (k % 2))) & 15u"),
    "q4_mask_three_bits": ("(byte >> (4 * (k % 2))) & 15u", "(byte >> (4 * (k % 2))) & 7u"),
    "q4_byte_index": ("Q[i * ldq + k / 2]", "Q[i * ldq + k / 4]"),
    "q4_scale_index": ("& 15u;\n        double s = oracle_half_to_double(S[i * lds + k / 64]);",
                       "& 15u;\n        double s = oracle_half_to_double(S[i * lds + k / 32]);"),
    "q4_dot_drops_last": ("oracle_q4_unpack_row(i, K, Q, ldq, S, lds, w);\n        double s = 0.0, t = 0.0;\n        for (int64_t k = 0; k < K; ++k)",
                          "oracle_q4_unpack_row(i, K, Q, ldq, S, lds, w);\n        double s = 0.0, t = 0.0;\n        for (int64_t k = 0; k + 1 < K; ++k)"),
    "ex_bound_drops_beta": ("u += fabs(cin);", "u += 0.0;"),
    "ex_beta_scales_product": ("double c = alpha != 0.0 ? alpha * s : 0.0, u = fabs(alpha) * t;",
                               "double c = alpha != 0.0 ? beta * s : 0.0, u = fabs(alpha) * t;"),
    "ex_reads_c_when_beta_zero": ("if (beta != 0.0) {\n                double cin", "if (1) {\n                double cin"),
    "ex_trans_a_ignored": ("double a = trans_a ? (double)A[k * lda + i] : (double)A[i * lda + k];\n                double b = trans_b ? (double)B[j * ldb + k] : (double)B[k * ldb + j];\n                s += a * b;",
                           "double a = (double)A[i * lda + k];\n                double b = trans_b ? (double)B[j * ldb + k] : (double)B[k * ldb + j];\n                s += a * b;"),
    "cells_trans_b_ignored": ("double b = trans_b ? (double)B[j * ldb + k] : (double)B[k * ldb + j];",
                              "double b = (double)B[k * ldb + j];"),
}


def _pack(codes):
    M, K = codes.shape
    nb = (K + 3) // 4
    p = np.zeros((M, nb * 4), np.uint16)
    p[:, :K] = codes
    q = p.reshape(M, nb, 4)
    return (q[..., 0] | (q[..., 1] << 2) | (q[..., 2] << 4) | (q[..., 3] << 6)).astype(np.uint8)


def _battery():
    """Compact pins; returns the list of names that failed."""
    rng = np.random.default_rng(99)
    failed = []

    def expect(name, cond):
        if not cond:
            failed.append(name)

    g = load("gemm_tiny_3x4x2.txt")
    A = np.asarray(g["A"], np.float64).astype(np.float32)
    B = np.asarray(g["B"], np.float64).astype(np.float32)
    C = np.asarray(g["C"], np.float64)
    expect("tiny_nn", np.array_equal(oracle.gemm_nn(A, B)[0], C))
    expect("tiny_tn", np.array_equal(oracle.gemm_tn(np.ascontiguousarray(A.T), B)[0], C))
    expect("tiny_nt", np.array_equal(oracle.gemm_nt(A, np.ascontiguousarray(B.T))[0], C))

    A = inputs.uniform(rng, (17, 31))
    B = inputs.uniform(rng, (31, 13))
    ref = A.astype(np.float64) @ B.astype(np.float64)
    ref_abs = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
    for name, (c, b) in (("np_nn", oracle.gemm_nn(A, B)),
                         ("np_tn", oracle.gemm_tn(np.ascontiguousarray(A.T), B)),
                         ("np_nt", oracle.gemm_nt(A, np.ascontiguousarray(B.T)))):
        expect(name, np.allclose(c, ref, rtol=0, atol=1e-11) and
               np.allclose(b, ref_abs, rtol=1e-12, atol=0))
    rows, cols = rng.integers(0, 17, 9), rng.integers(0, 13, 9)
    for ta, tb in ((0, 0), (1, 0), (0, 1)):
        Aa = np.ascontiguousarray(A.T) if ta else A
        Bb = np.ascontiguousarray(B.T) if tb else B
        c, _ = oracle.gemm_cells(Aa, Bb, rows, cols, trans_a=ta, trans_b=tb)
        expect("cells_%d%d" % (ta, tb), np.allclose(c, ref[rows, cols], rtol=0, atol=1e-11))

    W = inputs.normal(rng, (7, 130))
    x = inputs.normal(rng, (130,))
    y, _ = oracle.gemv(W, x)
    expect("gemv_np", np.allclose(y, W.astype(np.float64) @ x.astype(np.float64), rtol=0, atol=1e-12))

    g = load("q2_tiny_2x4.txt")
    y, _ = oracle.gemv_q2(np.array(g["Q"], np.uint8), np.array(g["S"], np.uint16),
                          np.asarray(g["x"], np.float64).astype(np.float32)[0])
    expect("q2_tiny", np.array_equal(y, np.asarray(g["y"], np.float64)[0]))

    M, K = 5, 200
    codes = rng.integers(0, 4, (M, K))
    S = rng.uniform(0.01, 0.05, (M, 4)).astype(np.float16).view(np.uint16)
    x = inputs.normal(rng, (K,))
    Wd = (codes - 1.5) * np.repeat(S.view(np.float16).astype(np.float64), 64, 1)[:, :K]
    y, _ = oracle.gemv_q2(_pack(codes), S, x)
    expect("q2_np", np.allclose(y, Wd @ x.astype(np.float64), rtol=0, atol=1e-12))

    g = load("gemm_ex_tiny_2x3x2.txt")
    ab = np.asarray(g["alpha_beta"], np.float64)[0]
    out, bnd = oracle.gemm_ex(np.asarray(g["A"], np.float64).astype(np.float32),
                              np.asarray(g["B"], np.float64).astype(np.float32),
                              np.asarray(g["C"], np.float64).astype(np.float32), ab[0], ab[1])
    expect("ex_tiny", np.array_equal(out, np.asarray(g["out"], np.float64)) and
           np.array_equal(bnd, np.asarray(g["bound"], np.float64)))
    At = inputs.uniform(rng, (9, 7))
    Bt = inputs.uniform(rng, (9, 5))
    Cn = np.full((7, 5), np.nan, np.float32)
    out, _ = oracle.gemm_ex(At, Bt, Cn, 1.0, 0.0, trans_a=True)
    expect("ex_ta_beta0", np.allclose(out, At.T.astype(np.float64) @ Bt.astype(np.float64),
                                      rtol=0, atol=1e-12))

    g = load("q4_tiny_2x4.txt")
    y, _ = oracle.gemv_q4(np.array(g["Q"], np.uint8), np.array(g["S"], np.uint16),
                          np.asarray(g["x"], np.float64).astype(np.float32)[0])
    expect("q4_tiny", np.array_equal(y, np.asarray(g["y"], np.float64)[0]))

    M, K = 5, 200
    codes = rng.integers(0, 16, (M, K))
    S = rng.uniform(0.01, 0.05, (M, 4)).astype(np.float16).view(np.uint16)
    x = inputs.normal(rng, (K,))
    Wd = (codes - 7.5) * np.repeat(S.view(np.float16).astype(np.float64), 64, 1)[:, :K]
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    y, _ = oracle.gemv_q4(packed, S, x)
    expect("q4_np", np.allclose(y, Wd @ x.astype(np.float64), rtol=0, atol=1e-12))

    pats = np.arange(0, 65536, 97, dtype=np.uint32).astype(np.uint16)
    got = np.array([oracle.half_to_double(int(h)) for h in pats])
    ref = pats.view(np.float16).astype(np.float64)
    ok = np.array_equal(np.isnan(got), np.isnan(ref)) and np.array_equal(
        got[~np.isnan(ref)], ref[~np.isnan(ref)])
    expect("half", ok)
    return failed


def _with_lib(path):
    saved = oracle._lib
    oracle._lib = oracle.bind(ctypes.CDLL(path))
    try:
        return _battery()
    finally:
        oracle._lib = saved


def test_battery_passes_on_real_oracle():
    assert _battery() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site not found: " + name
    mutated = src.replace(old, new, 1)
    cfile = tmp_path / "oracle_mut.c"
    cfile.write_text(mutated)
    so = tmp_path / ("liboracle_%s.so" % name)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                           str(cfile), "-o", str(so), "-lm"])
    failed = _with_lib(str(so))
    assert failed, "planted mistake %r passed every pin" % name
