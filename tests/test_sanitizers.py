"""AddressSanitizer and UndefinedBehaviorSanitizer builds (gcc, any finding
aborts), on the CPU:

  * the oracle (oracle.c), run under the oracle's own pin tests in a Python
    process that preloads the sanitizer runtimes;
  * the library's argument checks (the C entry points of api.hip compiled as
    host C++, linked with launchers that launch nothing), driven by the C
    program of test_c_header.py plus calls that pass every check -- among
    them a batch of 200 products, whose alias sweep sorts 800 byte ranges --
    and stop at the device check (no GPU) or at a stub launcher.

Neither build runs a kernel, so both run the same with or without a GPU."""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gemv_gemm_f32_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout
    p = p.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.fixture(scope="module")
def tools():
    if not (shutil.which("gcc") and shutil.which("g++")):
        pytest.skip("gcc/g++ are not installed")
    rt = [_runtime("libasan.so"), _runtime("libubsan.so")]
    if None in rt:
        pytest.skip("the gcc sanitizer runtimes are not installed")
    return rt


EXTRA_CALLS = r"""
    /* calls that pass every argument check: GG_ERR_NO_DEVICE without a
       GPU, GG_ERR_LAUNCH from the stub launchers with one */
    {
        int st;
        enum { NB = 200 };
        static const uint8_t *qs[NB];
        static const uint16_t *ss[NB];
        static const float *xs[NB];
        static float *ys[NB];
        static const float *ws[NB];
        for (int b = 0; b < NB; ++b) {
            ws[b] = A + (size_t)b * 256;
            qs[b] = Q + (size_t)b * 4096;
            ss[b] = (const uint16_t *)((const char *)S + (size_t)b * 4096);
            xs[b] = x;
            ys[b] = (float *)((char *)y + (size_t)b * 4096);
        }
        st = gemm_f32(64, 64, 64, A, 64, B, 64, C, 64, s);
        if (st != GG_ERR_NO_DEVICE && st != GG_ERR_LAUNCH) { printf("FAIL valid gemm %d\n", st); ++failures; }
        st = gemm_f32_ex(1, 1, 64, 32, 16, 2.0f, A, 64, B, 16, 1.0f, C, 32, s);
        if (st != GG_ERR_NO_DEVICE && st != GG_ERR_LAUNCH) { printf("FAIL valid gemm_ex %d\n", st); ++failures; }
        st = gemv_f32(100, 37, A, 40, x, y, s);
        if (st != GG_ERR_NO_DEVICE && st != GG_ERR_LAUNCH) { printf("FAIL valid gemv %d\n", st); ++failures; }
        st = gemv_q2(100, 100, Q, 25, S, 2, x, y, s);
        if (st != GG_ERR_NO_DEVICE && st != GG_ERR_LAUNCH) { printf("FAIL valid q2 %d\n", st); ++failures; }
        st = gemv_q2_batched(NB, 16, 1536, qs, 384, ss, 24, xs, ys, s);
        if (st != GG_ERR_NO_DEVICE && st != GG_ERR_LAUNCH) { printf("FAIL valid batch %d\n", st); ++failures; }
        st = gemv_f32_batched(NB, 16, 16, ws, 16, xs, ys, s);
        if (st != GG_ERR_NO_DEVICE && st != GG_ERR_LAUNCH) { printf("FAIL valid f32 batch %d\n", st); ++failures; }
        {
            static uint8_t wsb[16 * 4 * 16 * 4 + 16];
            void *ws = (void *)(((uintptr_t)wsb + 15) & ~(uintptr_t)15);
            st = gemv_q2_batched_ws(16, 16, 6144, qs, 1536, ss, 96, xs, ys, ws,
                                    gemv_q2_batched_ws_size(16, 16, 6144), s);
            if (st != GG_ERR_NO_DEVICE && st != GG_ERR_LAUNCH) { printf("FAIL valid ws batch %d\n", st); ++failures; }
        }
        ys[NB - 1] = ys[3];
        expect(gemv_f32_batched(NB, 16, 16, ws, 16, xs, ys, s), GG_ERR_ALIAS,
               "two outputs of an fp32 batch overlap");
        expect(gemv_q4_batched(NB, 16, 1536, qs, 768, ss, 24, xs, ys, s), GG_ERR_ALIAS,
               "two outputs of a batch overlap");
    }
"""


@pytest.fixture(scope="module")
def checks_program(tools, tmp_path_factory):
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "c_header_under_test", os.path.join(ROOT, "tests", "test_c_header.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    d = tmp_path_factory.mktemp("sanitize")
    api = d / "api_checks.cpp"                 # api.hip, compiled as host C++
    shutil.copyfile(os.path.join(CSRC, "api.hip"), api)
    text = api.read_text().replace('"../../include/gemvgemm.h"',
                                   '"%s"' % os.path.join(ROOT, "include", "gemvgemm.h"))
    api.write_text(text)
    lib = d / "libgemvgemm_checks.so"
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
                    "-I/opt/rocm/include", "-I", CSRC] + SAN +
                   [str(api), os.path.join(ROOT, "tests", "sanitize_stubs.cpp"), "-o", str(lib),
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"],
                   check=True, capture_output=True, text=True, timeout=300)
    prog = mod.PROGRAM.replace('    printf("%s\\n", failures ? "FAILED" : "ALL OK");',
                               EXTRA_CALLS + '    printf("%s\\n", failures ? "FAILED" : "ALL OK");')
    assert EXTRA_CALLS in prog
    src, exe = d / "use_header.c", d / "use_header"
    src.write_text(prog)
    subprocess.run(["gcc", "-std=c99", "-g", "-I", os.path.join(ROOT, "include")] + SAN +
                   [str(src), "-o", str(exe), "-L", str(d), "-l:libgemvgemm_checks.so",
                    "-Wl,-rpath," + str(d)],
                   check=True, capture_output=True, text=True, timeout=120)
    return str(exe)


def test_argument_checks_under_sanitizers(checks_program):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([checks_program], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ALL OK" in r.stdout


def test_oracle_pins_under_sanitizers(tools, tmp_path):
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ, LD_PRELOAD=":".join(tools), ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # the sanitized build is the one the tests load
    probe = subprocess.run([sys.executable, "-c",
                            "import oracle; oracle._load(); "
                            "print(any('liboracle_san' in l for l in open('/proc/self/maps')))"],
                           cwd=ROOT, capture_output=True, text=True, timeout=120, env=env)
    assert probe.returncode == 0 and probe.stdout.strip() == "True", probe.stdout + probe.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"),
                        "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, capture_output=True, text=True, timeout=900, env=env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
