"""The public header from plain C, on the CPU: gemvgemm.h compiles as strict
C99 with every warning an error, and a C program linked against
libgemvgemm.so (no Python, no torch) calls the entry points through it.  The
program only makes calls that the library rejects, or returns from, before
its first HIP call -- negative and oversized sizes, null and misaligned
pointers, short leading dimensions, an empty output -- so it runs the same
with or without a GPU, and it checks each returned status and message."""
import os
import shutil
import subprocess

import pytest

from gemv_gemm_f32_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <stdint.h>
#include <string.h>
#include "gemvgemm.h"

static int failures = 0;

static void expect(int got, int want, const char *what) {
    if (got != want) {
        printf("FAIL %s: got %d (%s), want %d\n", what, got, gg_strerror(got), want);
        ++failures;
    }
}

int main(void) {
    /* made-up device addresses, never dereferenced: every call below is
       rejected, or returns, before the library's first HIP call */
    const float *A = (const float *)(uintptr_t)0x10000000u;
    const float *B = (const float *)(uintptr_t)0x20000000u;
    float *C = (float *)(uintptr_t)0x30000000u;
    const uint8_t *Q = (const uint8_t *)(uintptr_t)0x40000000u;
    const uint16_t *S = (const uint16_t *)(uintptr_t)0x50000000u;
    const float *x = (const float *)(uintptr_t)0x60000000u;
    float *y = (float *)(uintptr_t)0x70000000u;
    gg_stream_t s = NULL;

    expect(gemm_f32(-1, 4, 4, A, 4, B, 4, C, 4, s), GG_ERR_INVALID_ARG, "negative M");
    expect(gemm_f32(4, (int64_t)1 << 31, 4, A, 4, B, (int64_t)1 << 31, C, (int64_t)1 << 31, s),
           GG_ERR_INVALID_ARG, "N = 2^31");
    expect(gemm_f32(0, 4, 4, NULL, 4, NULL, 4, NULL, 4, s), GG_OK, "empty output");
    expect(gemm_f32(4, 4, 4, NULL, 4, B, 4, C, 4, s), GG_ERR_INVALID_ARG, "null A");
    expect(gemm_f32(4, 4, 4, A, 3, B, 4, C, 4, s), GG_ERR_INVALID_ARG, "lda < K");
    expect(gemm_f32_tn(4, 4, 4, A, 4, B, 4, (float *)((char *)C + 2), 4, s),
           GG_ERR_INVALID_ARG, "misaligned C");
    expect(gemm_f32_nt(4, 4, 4, A, 4, B, 3, C, 4, s), GG_ERR_INVALID_ARG, "ldb < K");
    expect(gemm_f32_ex(2, 0, 4, 4, 4, 1.0f, A, 4, B, 4, 0.0f, C, 4, s),
           GG_ERR_INVALID_ARG, "trans_a = 2");
    expect(gemm_f32(4, 4, 4, A, 4, B, 4, (float *)A, 4, s), GG_ERR_ALIAS, "C on A");
    expect(gemv_f32(8, 8, A, 7, x, y, s), GG_ERR_INVALID_ARG, "ldw < K");
    expect(gemv_f32(0, 8, NULL, 8, NULL, NULL, s), GG_OK, "empty y");
    expect(gemv_q2(8, 64, Q, 15, S, 1, x, y, s), GG_ERR_INVALID_ARG, "ldq < K/4");
    expect(gemv_q4(8, 64, Q, 32, S, 0, x, y, s), GG_ERR_INVALID_ARG, "lds < K/64");
    {
        const uint8_t *qs[1] = {Q};
        const uint16_t *ss[1] = {S};
        const float *xs[1] = {x};
        float *ys[1] = {NULL};
        expect(gemv_q2_batched(1, 8, 64, qs, 16, ss, 1, xs, ys, s), GG_ERR_INVALID_ARG,
               "null y in a batch");
        expect(gemv_q4_batched(-1, 8, 64, qs, 32, ss, 1, xs, ys, s), GG_ERR_INVALID_ARG,
               "negative count");
    }
    {
        const float *ws[2] = {A, B};
        const float *xs[2] = {x, x};
        float *ys[2] = {y, (float *)A};
        expect(gemv_f32_batched(2, 8, 8, ws, 7, xs, ys, s), GG_ERR_INVALID_ARG,
               "ldw < K in an fp32 batch");
        expect(gemv_f32_batched(2, 8, 8, ws, 8, xs, ys, s), GG_ERR_ALIAS,
               "an fp32 batch output on another product's W");
        expect(gemv_f32_batched(2, 8, 8, NULL, 8, xs, ys, s), GG_ERR_INVALID_ARG,
               "null W array");
        expect(gemv_f32_batched(0, 8, 8, NULL, 8, NULL, NULL, s), GG_OK, "empty fp32 batch");
    }
    {
        const uint8_t *qs[16];
        const uint16_t *ss[16];
        const float *xs[16];
        float *ys[16];
        const int64_t need = gemv_q2_batched_ws_size(16, 16, 6144);
        for (int b = 0; b < 16; ++b) {
            qs[b] = Q;
            ss[b] = S;
            xs[b] = x;
            ys[b] = y + 1024 * b;
        }
        if (need != 16 * 4 * 16 * 4) {
            printf("FAIL workspace size %lld\n", (long long)need);
            ++failures;
        }
        expect((int)gemv_q2_batched_ws_size(-1, 16, 6144), GG_ERR_INVALID_ARG, "negative count size");
        expect(gemv_q2_batched_ws(16, 16, 6144, qs, 1536, ss, 96, xs, ys, NULL, need, s),
               GG_ERR_INVALID_ARG, "null workspace");
        expect(gemv_q2_batched_ws(16, 16, 6144, qs, 1536, ss, 96, xs, ys, (void *)C, need - 1, s),
               GG_ERR_INVALID_ARG, "short workspace");
    }
    {
        const int codes[] = {GG_OK, GG_ERR_INVALID_ARG, GG_ERR_ALIAS, GG_ERR_NO_DEVICE,
                             GG_ERR_LAUNCH, GG_ERR_SCRATCH, 12345};
        for (unsigned i = 0; i < sizeof codes / sizeof codes[0]; ++i) {
            const char *m = gg_strerror(codes[i]);
            if (m == NULL || strlen(m) == 0) {
                printf("FAIL gg_strerror(%d)\n", codes[i]);
                ++failures;
            }
        }
    }
    printf("%s\n", failures ? "FAILED" : "ALL OK");
    return failures != 0;
}
"""


@pytest.fixture(scope="module")
def program(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not installed")
    lib = bd.LIB_PATH
    assert os.path.exists(lib), "libgemvgemm.so is not built"
    d = tmp_path_factory.mktemp("c_header")
    src, exe = d / "use_header.c", d / "use_header"
    src.write_text(PROGRAM)
    libdir = os.path.dirname(lib)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Wpedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    "-L", libdir, "-l:libgemvgemm.so", "-Wl,-rpath," + libdir],
                   check=True, capture_output=True, text=True, timeout=120)
    return str(exe)


def test_header_compiles_as_c99():
    """Every declaration, with no program around it."""
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not installed")
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Wpedantic", "-Werror",
                        "-fsyntax-only", "-x", "c", os.path.join(ROOT, "include", "gemvgemm.h")],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr


def test_c_program_calls_the_library(program):
    r = subprocess.run([program], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ALL OK" in r.stdout
