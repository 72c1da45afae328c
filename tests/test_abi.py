"""The C ABI on a CPU-only machine: the library loads, exports every function
the public header declares, and rejects bad arguments before any HIP call.

Argument checks run before the library touches the HIP runtime, so they can
be exercised here with made-up (never dereferenced) device addresses.  With no
GPU present, well-formed calls must report GG_ERR_NO_DEVICE rather than crash.
A call that passes every argument check would launch a kernel on those
made-up addresses if a GPU were visible, so such calls are made only through
``passes_checks``, which skips the test when a device is present.
"""
import ctypes

import pytest

from gemv_gemm_f32_amd import binding as bd

lib = bd.load()

# made-up, 256-byte aligned addresses far apart; never dereferenced here
PA, PB, PC, PX = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def _gpu_present():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def passes_checks(status_of):
    """Run `status_of()` (a call whose arguments are all valid, on made-up
    addresses) only without a GPU, where it must stop at the device check."""
    if _gpu_present():
        pytest.skip("a valid call on made-up addresses would launch on the GPU")
    st = status_of()
    assert st not in (bd.GG_ERR_ALIAS, bd.GG_ERR_INVALID_ARG), st
    assert st == bd.GG_ERR_NO_DEVICE, st


def test_exports_every_header_function():
    declared = bd.header_functions()
    assert sorted(declared) == sorted(bd.ENTRY_POINTS)
    for name in declared:
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_strerror_covers_every_status():
    for st in (bd.GG_OK, bd.GG_ERR_INVALID_ARG, bd.GG_ERR_ALIAS,
               bd.GG_ERR_NO_DEVICE, bd.GG_ERR_LAUNCH, bd.GG_ERR_SCRATCH):
        msg = bd.strerror(st)
        assert msg and msg != "unknown status"
    assert bd.strerror(12345) == "unknown status"


GEMMS = ("gemm_f32", "gemm_f32_tn", "gemm_f32_nt")


@pytest.mark.parametrize("name", GEMMS)
def test_gemm_rejects_bad_sizes(name):
    f = getattr(lib, name)
    assert f(-1, 4, 4, PA, 4, PB, 4, PC, 4, None) == bd.GG_ERR_INVALID_ARG
    assert f(4, -1, 4, PA, 4, PB, 4, PC, 4, None) == bd.GG_ERR_INVALID_ARG
    assert f(4, 4, -1, PA, 4, PB, 4, PC, 4, None) == bd.GG_ERR_INVALID_ARG
    assert f(1 << 31, 4, 4, PA, 1 << 31, PB, 4, PC, 4, None) == bd.GG_ERR_INVALID_ARG


@pytest.mark.parametrize("name", GEMMS)
def test_gemm_rejects_ranges_past_the_address_space(name):
    """Sizes below 2^31 whose byte range would wrap: invalid, not an alias."""
    f = getattr(lib, name)
    big = (1 << 31) - 1
    high = (1 << 64) - (1 << 20)          # 1 MiB below the top of the address space
    assert f(big, big, 1, PA, big, PB, big, high, big, None) == bd.GG_ERR_INVALID_ARG
    assert f(4, 4, big, high, big, PB, big, PC, 4, None) == bd.GG_ERR_INVALID_ARG


def test_packed_and_gemv_reject_ranges_past_the_address_space():
    big = (1 << 31) - 1
    high = (1 << 64) - (1 << 20)
    assert lib.gemv_f32(big, big, high, big, PB, PC, None) == bd.GG_ERR_INVALID_ARG
    assert lib.gemv_q2(big, 64, high, 16, PB, 1, PA, PC, None) == bd.GG_ERR_INVALID_ARG


@pytest.mark.parametrize("name", GEMMS)
def test_gemm_empty_output_is_ok_without_pointers(name):
    f = getattr(lib, name)
    assert f(0, 5, 7, None, 0, None, 0, None, 0, None) == bd.GG_OK
    assert f(5, 0, 7, None, 0, None, 0, None, 0, None) == bd.GG_OK


@pytest.mark.parametrize("name", GEMMS)
def test_gemm_rejects_null_and_misaligned(name):
    f = getattr(lib, name)
    assert f(4, 4, 4, None, 4, PB, 4, PC, 4, None) == bd.GG_ERR_INVALID_ARG
    assert f(4, 4, 4, PA, 4, None, 4, PC, 4, None) == bd.GG_ERR_INVALID_ARG
    assert f(4, 4, 4, PA, 4, PB, 4, None, 4, None) == bd.GG_ERR_INVALID_ARG
    assert f(4, 4, 4, PA + 2, 4, PB, 4, PC, 4, None) == bd.GG_ERR_INVALID_ARG
    assert f(4, 4, 4, PA, 4, PB, 4, PC + 1, 4, None) == bd.GG_ERR_INVALID_ARG


def test_gemm_leading_dimensions():
    # NN: lda >= K, ldb >= N, ldc >= N
    assert lib.gemm_f32(8, 6, 5, PA, 4, PB, 6, PC, 6, None) == bd.GG_ERR_INVALID_ARG
    assert lib.gemm_f32(8, 6, 5, PA, 5, PB, 5, PC, 6, None) == bd.GG_ERR_INVALID_ARG
    assert lib.gemm_f32(8, 6, 5, PA, 5, PB, 6, PC, 5, None) == bd.GG_ERR_INVALID_ARG
    # TN: A stored K x M, so lda >= M
    assert lib.gemm_f32_tn(8, 6, 5, PA, 7, PB, 6, PC, 6, None) == bd.GG_ERR_INVALID_ARG
    # NT: B stored N x K, so ldb >= K
    assert lib.gemm_f32_nt(8, 6, 5, PA, 5, PB, 4, PC, 6, None) == bd.GG_ERR_INVALID_ARG


def test_gemm_alias():
    # C placed inside A's span
    assert lib.gemm_f32(8, 8, 8, PA, 8, PB, 8, PA + 4 * 8, 8, None) == bd.GG_ERR_ALIAS
    # C inside B for the transposed layouts
    assert lib.gemm_f32_tn(8, 8, 8, PA, 8, PB, 8, PB, 8, None) == bd.GG_ERR_ALIAS
    assert lib.gemm_f32_nt(8, 8, 8, PA, 8, PB, 8, PB + 4 * 63, 8, None) == bd.GG_ERR_ALIAS


def test_gemm_adjacent_output_passes_checks():
    # adjacent but disjoint is fine (rejected later only for lack of a GPU)
    passes_checks(lambda: lib.gemm_f32(8, 8, 8, PA, 8, PB, 8, PA + 4 * 64, 8, None))


def test_gemv_validation():
    f = lib.gemv_f32
    assert f(-1, 4, PA, 4, PX, PC, None) == bd.GG_ERR_INVALID_ARG
    assert f(0, 4, None, 0, None, None, None) == bd.GG_OK
    assert f(4, 4, PA, 3, PX, PC, None) == bd.GG_ERR_INVALID_ARG
    assert f(4, 4, None, 4, PX, PC, None) == bd.GG_ERR_INVALID_ARG
    assert f(4, 4, PA, 4, PX, None, None) == bd.GG_ERR_INVALID_ARG
    assert f(4, 4, PA, 4, PX, PA + 8, None) == bd.GG_ERR_ALIAS
    assert f(4, 4, PA, 4, PX, PX, None) == bd.GG_ERR_ALIAS


def test_gemv_q2_validation():
    f = lib.gemv_q2
    # K = 100: rows need ceil(100/4) = 25 bytes and ceil(100/64) = 2 scales
    assert f(4, 100, PA, 24, PB, 2, PX, PC, None) == bd.GG_ERR_INVALID_ARG
    assert f(4, 100, PA, 25, PB, 1, PX, PC, None) == bd.GG_ERR_INVALID_ARG
    assert f(4, 100, PA, 25, PB + 1, 2, PX, PC, None) == bd.GG_ERR_INVALID_ARG
    assert f(4, 100, PA, 25, PB, 2, PX + 2, PC, None) == bd.GG_ERR_INVALID_ARG
    assert f(4, 100, None, 25, PB, 2, PX, PC, None) == bd.GG_ERR_INVALID_ARG
    assert f(0, 100, None, 0, None, 0, None, None, None) == bd.GG_OK
    assert f(4, 100, PA, 25, PB, 2, PX, PA + 16, None) == bd.GG_ERR_ALIAS
    assert f(4, 100, PA, 25, PB, 2, PX, PB + 4, None) == bd.GG_ERR_ALIAS


def test_gemm_ex_validation():
    f = lib.gemm_f32_ex
    # trans flags must be 0 or 1
    assert f(2, 0, 4, 4, 4, 1.0, PA, 4, PB, 4, 0.0, PC, 4, None) == bd.GG_ERR_INVALID_ARG
    assert f(0, -1, 4, 4, 4, 1.0, PA, 4, PB, 4, 0.0, PC, 4, None) == bd.GG_ERR_INVALID_ARG
    # transposed A is K x M: lda >= M
    assert f(1, 0, 8, 4, 4, 1.0, PA, 7, PB, 4, 0.0, PC, 4, None) == bd.GG_ERR_INVALID_ARG
    # transposed B is N x K: ldb >= K
    assert f(0, 1, 4, 8, 6, 1.0, PA, 6, PB, 5, 0.0, PC, 8, None) == bd.GG_ERR_INVALID_ARG
    assert f(1, 1, 4, 4, 4, 1.0, PA, 4, PB, 4, 0.0, PA + 4, 4, None) == bd.GG_ERR_ALIAS
    assert f(0, 0, 4, 4, 4, 1.0, None, 4, PB, 4, 2.0, PC, 4, None) == bd.GG_ERR_INVALID_ARG
    assert f(0, 0, 0, 4, 4, 1.0, None, 0, None, 0, 2.0, None, 0, None) == bd.GG_OK


def test_gemm_ex_alpha_zero_accepts_null_operands():
    # alpha == 0: A and B are not read, so NULL operands are accepted
    passes_checks(lambda: lib.gemm_f32_ex(0, 0, 4, 4, 4, 0.0, None, 0, None, 0, 2.0, PC, 4,
                                          None))


def test_gemv_q4_validation():
    f = lib.gemv_q4
    # K = 101: rows need ceil(101/2) = 51 bytes and ceil(101/64) = 2 scales
    assert f(4, 101, PA, 50, PB, 2, PX, PC, None) == bd.GG_ERR_INVALID_ARG
    assert f(4, 101, PA, 51, PB, 1, PX, PC, None) == bd.GG_ERR_INVALID_ARG
    assert f(4, 101, PA, 51, PB + 1, 2, PX, PC, None) == bd.GG_ERR_INVALID_ARG
    assert f(4, 101, PA, 51, PB, 2, PX + 2, PC, None) == bd.GG_ERR_INVALID_ARG
    assert f(-1, 101, PA, 51, PB, 2, PX, PC, None) == bd.GG_ERR_INVALID_ARG
    assert f(0, 101, None, 0, None, 0, None, None, None) == bd.GG_OK
    # the codes of 4 rows of 51 bytes end at PA + 204: y starting there is fine,
    # y starting at PA + 200 overlaps
    assert f(4, 101, PA, 51, PB, 2, PX, PA + 200, None) == bd.GG_ERR_ALIAS
    assert f(4, 101, PA, 51, PB, 2, PX, PB + 4, None) == bd.GG_ERR_ALIAS


def test_gemv_q4_adjacent_output_passes_checks():
    passes_checks(lambda: lib.gemv_q4(4, 101, PA, 51, PB, 2, PX, PA + 204, None))


def test_gemv_q4_batched_validation():
    f = lib.gemv_q4_batched
    Q = _parr(PA, PA + 0x100000)
    S = _parr(PB, PB + 0x100000)
    x = _parr(PX, PX)
    y = _parr(PC, PC + 0x100000)
    assert f(2, 4, 64, Q, 31, S, 1, x, y, None) == bd.GG_ERR_INVALID_ARG   # needs 32 bytes
    assert f(2, 4, 64, Q, 32, S, 1, x, _parr(PC, PA + 96), None) == bd.GG_ERR_ALIAS
    passes_checks(lambda: f(2, 4, 64, Q, 32, S, 1, x, y, None))


@pytest.mark.skipif(_gpu_present(), reason="checks the no-device path")
def test_no_device_is_reported():
    assert lib.gemm_f32(4, 4, 4, PA, 4, PB, 4, PC, 4, None) == bd.GG_ERR_NO_DEVICE
    assert lib.gemv_f32(4, 4, PA, 4, PX, PC, None) == bd.GG_ERR_NO_DEVICE
    assert lib.gemv_q2(4, 64, PA, 16, PB, 1, PX, PC, None) == bd.GG_ERR_NO_DEVICE
    assert lib.gemv_q4(4, 64, PA, 32, PB, 1, PX, PC, None) == bd.GG_ERR_NO_DEVICE


def test_single_hip_runtime_in_process():
    # The library must share torch's HIP runtime rather than load a second one
    # (torch's stream handles and allocations are only valid in its own).
    import re
    maps = open("/proc/self/maps").read()
    hip = set(re.findall(r"\S*libamdhip64\S*", maps))
    assert len(hip) == 1, hip


def _parr(*ps):
    arr = (ctypes.c_void_p * len(ps))()
    for i, p in enumerate(ps):
        arr[i] = p
    return arr


def test_gemv_q2_batched_validation():
    f = lib.gemv_q2_batched
    Q = _parr(PA, PA + 0x100000)
    S = _parr(PB, PB + 0x100000)
    x = _parr(PX, PX)                    # a shared x is allowed
    y = _parr(PC, PC + 0x100000)
    assert f(-1, 4, 64, Q, 16, S, 1, x, y, None) == bd.GG_ERR_INVALID_ARG
    assert f(0, 4, 64, None, 16, None, 1, None, None, None) == bd.GG_OK
    assert f(2, 0, 64, Q, 16, S, 1, x, y, None) == bd.GG_OK
    assert f(2, 4, 64, None, 16, S, 1, x, y, None) == bd.GG_ERR_INVALID_ARG
    assert f(2, 4, 64, Q, 15, S, 1, x, y, None) == bd.GG_ERR_INVALID_ARG
    assert f(2, 4, 64, Q, 16, S, 1, x, _parr(PC, PC + 2), None) == bd.GG_ERR_INVALID_ARG
    # y[1] overlaps y[0]
    assert f(2, 4, 64, Q, 16, S, 1, x, _parr(PC, PC + 8), None) == bd.GG_ERR_ALIAS
    # y[1] overlaps the codes of product 0
    assert f(2, 4, 64, Q, 16, S, 1, x, _parr(PC, PA + 16), None) == bd.GG_ERR_ALIAS
    # y[0] overlaps the shared x
    assert f(2, 4, 64, Q, 16, S, 1, x, _parr(PX + 4, PC), None) == bd.GG_ERR_ALIAS
    passes_checks(lambda: f(2, 4, 64, Q, 16, S, 1, x, y, None))


def test_gemv_f32_batched_validation():
    f = lib.gemv_f32_batched
    W = _parr(PA, PA + 0x100000)
    x = _parr(PX, PX)                    # a shared x is allowed
    y = _parr(PC, PC + 0x100000)
    assert f(-1, 4, 64, W, 64, x, y, None) == bd.GG_ERR_INVALID_ARG
    assert f(0, 4, 64, None, 64, None, None, None) == bd.GG_OK
    assert f(2, 0, 64, W, 64, x, y, None) == bd.GG_OK
    assert f(2, 4, 64, None, 64, x, y, None) == bd.GG_ERR_INVALID_ARG
    assert f(2, 4, 64, W, 63, x, y, None) == bd.GG_ERR_INVALID_ARG
    assert f(2, 4, 64, _parr(PA, PA + 2), 64, x, y, None) == bd.GG_ERR_INVALID_ARG
    assert f(2, 4, 64, W, 64, x, _parr(PC, PC + 2), None) == bd.GG_ERR_INVALID_ARG
    # y[1] overlaps y[0]
    assert f(2, 4, 64, W, 64, x, _parr(PC, PC + 8), None) == bd.GG_ERR_ALIAS
    # y[1] overlaps W of product 0
    assert f(2, 4, 64, W, 64, x, _parr(PC, PA + 64), None) == bd.GG_ERR_ALIAS
    # y[0] overlaps the shared x
    assert f(2, 4, 64, W, 64, x, _parr(PX + 4, PC), None) == bd.GG_ERR_ALIAS
    passes_checks(lambda: f(2, 4, 64, W, 64, x, y, None))
    # K = 0 reads no input: null W and x pass, only the outputs are checked
    passes_checks(lambda: f(2, 4, 0, _parr(0, 0), 0, _parr(0, 0), y, None))


def test_gemv_q2_batched_ws_validation():
    f, size = lib.gemv_q2_batched_ws, lib.gemv_q2_batched_ws_size
    assert size(-1, 4, 6144) == bd.GG_ERR_INVALID_ARG
    assert size(16, 1 << 31, 6144) == bd.GG_ERR_INVALID_ARG
    assert size(16, 4, 6144) == 16 * 4 * 4 * 4
    assert size(7, 4, 6144) == 0 and size(16, 4, 3072) == 0
    n, M, K = 16, 4, 6144
    need = size(n, M, K)
    Q = _parr(*[PA + 0x10000 * b for b in range(n)])
    S = _parr(*[PB + 0x10000 * b for b in range(n)])
    x = _parr(*[PX] * n)
    y = _parr(*[PC + 0x1000 * b for b in range(n)])
    W = 0x50000000
    # workspace missing, too small, misaligned
    assert f(n, M, K, Q, 1536, S, 96, x, y, None, need, None) == bd.GG_ERR_INVALID_ARG
    assert f(n, M, K, Q, 1536, S, 96, x, y, W, need - 4, None) == bd.GG_ERR_INVALID_ARG
    assert f(n, M, K, Q, 1536, S, 96, x, y, W + 4, need, None) == bd.GG_ERR_INVALID_ARG
    # workspace over an output, over an input
    assert f(n, M, K, Q, 1536, S, 96, x, y, PC + 0x1000 * 3 - 16, need, None) == bd.GG_ERR_ALIAS
    assert f(n, M, K, Q, 1536, S, 96, x, y, PX, need, None) == bd.GG_ERR_ALIAS
    # the usual batch checks still apply
    assert f(n, M, K, Q, 1535, S, 96, x, y, W, need, None) == bd.GG_ERR_INVALID_ARG
    passes_checks(lambda: f(n, M, K, Q, 1536, S, 96, x, y, W, need, None))
    # a batch that does not cut its rows ignores the workspace (NULL is fine)
    passes_checks(lambda: f(7, M, K, Q, 1536, S, 96, x, y, None, 0, None))


def test_gemv_q2_batched_noalloc_validation():
    f = lib.gemv_q2_batched_noalloc
    n, K = 64, 12288
    Q = _parr(*[PA] * n)                       # inputs may be shared
    S = _parr(*[PB] * n)
    x = _parr(*[PX] * n)
    y = _parr(*[PC + 0x10000 * b for b in range(n)])
    assert f(-1, 16, K, Q, 3072, S, 192, x, y, None) == bd.GG_ERR_INVALID_ARG
    assert f(n, 16, K, Q, 3071, S, 192, x, y, None) == bd.GG_ERR_INVALID_ARG
    # partial sums beyond the fixed 4 MiB buffer: 64 x 8 slices x 2,049 rows
    assert f(n, 2049, K, Q, 3072, S, 192, x, y, None) == bd.GG_ERR_SCRATCH
    assert f(n, 16, K, Q, 3072, S, 192, x, _parr(*([PC] * n)), None) == bd.GG_ERR_ALIAS
    passes_checks(lambda: f(n, 2048, K, Q, 3072, S, 192, x, y, None))   # exactly 4 MiB
    passes_checks(lambda: f(7, 2049, K, Q, 3072, S, 192, x, y, None))   # rows not cut
