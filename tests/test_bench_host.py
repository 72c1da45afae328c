"""Host logic of bench.py, on the CPU: the kernel-trace summary and the
calibrated traffic computed from synthetic rocprofv3 databases (the tables and
columns rocprofv3 writes), the source-hash gate on stored traffic, and the
one-GPU guard."""
import importlib.util
import json
import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


GEMM = "void gg::(anonymous namespace)::gemm_f32_direct<64, 64, true, false, 2, 4>(int, int, int)"
COPY = "__amd_rocclr_copyBuffer"


def _trace_db(path, rows):
    db = sqlite3.connect(path)
    db.execute("create table kernels (name text, duration integer)")
    db.executemany("insert into kernels values (?, ?)", rows)
    db.commit()
    db.close()


def _counter_db(path, counter, rows):
    """rows: (kernel name, dispatch id, value in KiB), one row per instance."""
    db = sqlite3.connect(path)
    db.execute("create table counters_collection (kernel_name text, dispatch_id integer, "
               "counter_name text, value real)")
    db.executemany("insert into counters_collection values (?, ?, ?, ?)",
                   [(k, d, counter, v) for k, d, v in rows])
    db.commit()
    db.close()


def test_summarize_trace(bench, tmp_path):
    p = str(tmp_path / "t.db")
    _trace_db(p, [(GEMM, 130000), (GEMM, 134000), (COPY, 5000)])
    lines = bench.summarize_trace(p).splitlines()
    assert lines[0].startswith("| kernel | calls |")
    row = [l for l in lines if "gemm_f32_direct<64, 64, true, false, 2, 4>" in l][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[0] == "gemm_f32_direct<64, 64, true, false, 2, 4>"   # namespace and arguments cut
    assert cells[1] == "2"
    assert float(cells[2]) == pytest.approx(264.0)       # total us
    assert float(cells[3]) == pytest.approx(132.0)       # average us
    assert float(cells[4]) == pytest.approx(130.0) and float(cells[5]) == pytest.approx(134.0)
    assert float(cells[6]) == pytest.approx(132.0)       # median us
    assert lines[2].find("gemm") > 0                     # sorted by total time


def test_traffic_uses_the_calibration_copy(bench, tmp_path, monkeypatch):
    """The calibration copy is the copy dispatch whose WRITE_SIZE is closest to
    its size: neither the input uploads nor the larger context copies."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    cal = bench.CALIBRATION_BYTES // 1024                 # KiB
    fetch_rows = [(COPY, 5, 100.0), (COPY, 36, cal / 2.0), (COPY, 90, 4.0 * cal / 2.0),
                  (COPY, 91, 4.0 * cal / 2.0)]
    write_rows = [(COPY, 5, 200.0), (COPY, 36, float(cal)), (COPY, 90, 4.0 * cal),
                  (COPY, 91, 4.0 * cal)]
    # the GEMM: two instances per dispatch (summed), three dispatches (median)
    for d, f in ((40, 40000.0), (41, 41000.0), (42, 45000.0)):
        fetch_rows += [(GEMM, d, f / 2), (GEMM, d, f / 2)]
        write_rows += [(GEMM, d, 8192.0), (GEMM, d, 8192.0)]
    fdb, wdb = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    _counter_db(fdb, "FETCH_SIZE", fetch_rows)
    _counter_db(wdb, "WRITE_SIZE", write_rows)
    assert bench.write_traffic(fdb, wdb) == 0
    with open(tmp_path / "traffic_gemm_f32_2048.json") as f:
        d = json.load(f)
    assert d["fetch_scale"] == pytest.approx(2.0)
    assert d["write_scale"] == pytest.approx(1.0)
    assert d["fetch_kib_raw"] == pytest.approx(41000.0)
    assert d["write_kib_raw"] == pytest.approx(16384.0)
    expect = 41000.0 * 1024 * 2.0 + 16384.0 * 1024
    assert d["hbm_bytes_per_launch"] == pytest.approx(expect)
    assert d["traffic_over_algorithmic"] == pytest.approx(expect / (3 * 4 * 2048 * 2048))


def _trace_db_shapes(path, rows):
    """rows: (name, duration, grid work-items, workgroup size)"""
    db = sqlite3.connect(path)
    db.execute("create table kernels (name text, duration integer, grid_x integer, "
               "grid_y integer, grid_z integer, workgroup_x integer, workgroup_y integer, "
               "workgroup_z integer)")
    db.executemany("insert into kernels values (?, ?, ?, 1, 1, ?, 1, 1)", rows)
    db.commit()
    db.close()


def _counter_db_shapes(path, counter, rows):
    """rows: (kernel name, dispatch id, value in KiB, grid work-items, workgroup size)"""
    db = sqlite3.connect(path)
    db.execute("create table counters_collection (kernel_name text, dispatch_id integer, "
               "counter_name text, value real, grid_size integer, workgroup_size integer)")
    db.executemany("insert into counters_collection values (?, ?, ?, ?, ?, ?)",
                   [(k, d, counter, v, g, w) for k, d, v, g, w in rows])
    db.commit()
    db.close()


def test_one_kernel_at_two_shapes(bench, tmp_path, monkeypatch):
    """The same GEMM kernel launched at 1,024 workgroups (2048^3) and at 768
    (a smaller product) gives a trace row per shape, and the traffic of the
    2048^3 launches alone."""
    p = str(tmp_path / "t.db")
    _trace_db_shapes(p, [(GEMM, 130000, 524288, 512), (GEMM, 134000, 524288, 512),
                         (GEMM, 40000, 393216, 512)])
    lines = bench.summarize_trace(p).splitlines()
    big = [l for l in lines if "@1024wg" in l][0]
    small = [l for l in lines if "@768wg" in l][0]
    assert float(big.strip("|").split("|")[3]) == pytest.approx(132.0)
    assert float(small.strip("|").split("|")[3]) == pytest.approx(40.0)
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    cal = bench.CALIBRATION_BYTES // 1024
    # copies at two shapes: the upload (small) and the calibration copy
    fetch_rows = [(COPY, 5, 100.0, 512, 512), (COPY, 36, cal / 2.0, 65536, 512)]
    write_rows = [(COPY, 5, 200.0, 512, 512), (COPY, 36, float(cal), 65536, 512)]
    for d in (40, 41, 42):
        fetch_rows.append((GEMM, d, 40000.0, 524288, 512))
        write_rows.append((GEMM, d, 16384.0, 524288, 512))
    for d in (50, 51):
        fetch_rows.append((GEMM, d, 9000.0, 393216, 512))
        write_rows.append((GEMM, d, 3000.0, 393216, 512))
    fdb, wdb = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    _counter_db_shapes(fdb, "FETCH_SIZE", fetch_rows)
    _counter_db_shapes(wdb, "WRITE_SIZE", write_rows)
    assert bench.write_traffic(fdb, wdb) == 0
    with open(tmp_path / "traffic_gemm_f32_2048.json") as f:
        d = json.load(f)
    assert d["kernel"].endswith("@1024wg")
    assert d["fetch_kib_raw"] == pytest.approx(40000.0)
    assert d["write_kib_raw"] == pytest.approx(16384.0)
    assert d["fetch_scale"] == pytest.approx(2.0)


def test_traffic_gated_by_source_hash(bench, tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    with open(tmp_path / "x.json", "w") as f:
        json.dump({"kernel_src_sha": "abc", "hbm_bytes_per_launch": 123.0}, f)
    assert bench.traffic_from_profile("x.json", "abc") == 123.0
    assert bench.traffic_from_profile("x.json", "def") is None
    assert bench.traffic_from_profile("missing.json", "abc") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_summarize_counters(bench, tmp_path):
    """Medians per dispatch and the derived figures of a 40-product 2-bit
    batch: VALU instructions per lane per weight, issue share, L2 hit rate."""
    p = str(tmp_path / "c.db")
    name = ("void gg::(anonymous namespace)::gemv_q2_idot<3, 16, 64, false>(int, long, long, "
            "gg::(anonymous namespace)::PackedPtrs<64>)")
    vals = {"SQ_INSTS_VALU": 14.5e6, "SQ_ACTIVE_INST_VALU": 14.5e6, "GRBM_GUI_ACTIVE": 8.0e5,
            "SQ_INSTS_LDS": 7.0e5, "SQ_LDS_BANK_CONFLICT": 1.4e6, "TCC_HIT_sum": 1.0e5,
            "TCC_MISS_sum": 9.0e5}
    rows = []
    for disp, f in ((1, 1.0), (2, 1.1), (3, 0.9)):
        rows += [(name, disp, c, v * f, 3840 * 192, 192) for c, v in vals.items()]
    _counter_db_shapes(p, "unused", [])
    db = sqlite3.connect(p)
    db.executemany("insert into counters_collection values (?, ?, ?, ?, ?, ?)", rows)
    db.commit()
    db.close()
    out = bench.summarize_counters([p])
    derived = [l for l in out.splitlines() if l.startswith("| gemv_q2_idot") and
               l.count("|") == 7][0]
    cells = [c.strip() for c in derived.strip("|").split("|")]
    weights = 40 * 12288 * 1536
    assert float(cells[1]) == pytest.approx(14.5e6 * 64 / weights, abs=1e-3)
    assert float(cells[2]) == pytest.approx(4 * 14.5e6 / (1024 * 8.0e5 / 8), abs=0.01)
    assert float(cells[4]) == pytest.approx(2.0, abs=0.01)
    assert float(cells[5]) == pytest.approx(0.1, abs=1e-3)


def test_probe_library_exports_and_checks(bench):
    """The probe kernels' library (built by the build entry point) exports
    both probes, and each rejects out-of-range sizes before any HIP call."""
    import ctypes
    if not os.path.exists(bench.PROBE_LIB):
        sys.path.insert(0, ROOT)
        from gemv_gemm_f32_amd import build as b
        b.build_probes(os.path.join(ROOT, "bench_probes.hip"), bench.PROBE_LIB)
    lib = ctypes.CDLL(bench.PROBE_LIB)
    lib.probe_empty.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.probe_chase.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int,
                                ctypes.c_void_p, ctypes.c_void_p]
    invalid = 1   # hipErrorInvalidValue
    for grid, block in ((0, 64), (1, 0), (1, 1025)):
        assert lib.probe_empty(grid, block, None) == invalid
    dummy = ctypes.c_void_p(0x10000000)
    assert lib.probe_chase(dummy, 100, 100, 10, dummy, None) == invalid     # start >= n
    assert lib.probe_chase(dummy, 100, 0, -1, dummy, None) == invalid       # links < 0
    assert lib.probe_chase(dummy, 1 << 33, 0, 10, dummy, None) == invalid   # n beyond 32 bits


def test_probe_mfma_checks(bench):
    import ctypes
    lib = ctypes.CDLL(bench.PROBE_LIB)
    lib.probe_mfma.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p, ctypes.c_void_p]
    dummy = ctypes.c_void_p(0x10000000)
    invalid = 1   # hipErrorInvalidValue
    for shape, nacc, grid, block, iters in ((8, 1, 1, 64, 1), (32, 3, 1, 64, 1), (16, 1, 0, 64, 1),
                                            (32, 1, 1, 96, 1), (32, 1, 1, 2048, 1),
                                            (16, 2, 1, 64, -1)):
        assert lib.probe_mfma(shape, nacc, grid, block, iters, dummy, None) == invalid
