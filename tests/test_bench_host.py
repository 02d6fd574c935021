"""Host logic of bench.py (no GPU): the profile summarizers read rocprofv3
databases built here with the tables and columns they query, and more than
one GPU is refused with a message."""
import os
import re
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _counters_db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (dispatch_id integer, kernel_name text, grid_size integer, "
                "counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?, ?)", rows)
    con.commit()
    con.close()
    return str(path)


def test_summarize_traffic_scales_each_counter_by_the_known_copy(tmp_path):
    known_kib = (64 << 20) * 4 / 1024
    grid = (64 << 20) // 4
    gemv = "void w4a16::gemv_kernel<1, 1, 4, 4, 0, 4>(...)"
    ew = "void at::native::vectorized_elementwise_kernel<...>"
    # the FETCH counter reads half the copy's bytes (scale 2), WRITE all (scale 1)
    fetch = _counters_db(tmp_path / "f.db", [
        (1, gemv, 1024, "FETCH_SIZE", 100.0), (2, gemv, 1024, "FETCH_SIZE", 300.0),
        (3, ew, grid, "FETCH_SIZE", known_kib / 2), (4, ew, 64, "FETCH_SIZE", 1.0)])
    write = _counters_db(tmp_path / "w.db", [
        (1, gemv, 1024, "WRITE_SIZE", 2.0), (2, gemv, 1024, "WRITE_SIZE", 6.0),
        (3, ew, grid, "WRITE_SIZE", known_kib)])
    parts, traffic = bench.summarize_traffic(fetch, write)
    assert parts["FETCH_SIZE"][1] == pytest.approx(2.0)
    assert parts["WRITE_SIZE"][1] == pytest.approx(1.0)
    assert parts["FETCH_SIZE"][2] == 2 and parts["FETCH_SIZE"][3] == 1
    assert traffic == round((200.0 * 2 + 4.0) * 1024)


def test_summarize_traffic_needs_both_kernels(tmp_path):
    db = _counters_db(tmp_path / "x.db", [(1, "gemv_kernel", 8, "FETCH_SIZE", 1.0)])
    with pytest.raises(SystemExit):
        bench.summarize_traffic(db, db)


def test_summarize_sq_drops_the_first_dispatch_and_normalises_per_wave(tmp_path):
    k = "void w4a16::gemm8_kernel<2, true, 4>(w4a16::GemmArgs)"
    p1 = _counters_db(tmp_path / "p1.db", [
        (d, k, 0, c, v) for d in (1, 2, 3) for c, v in
        (("SQ_WAVES", 4096.0), ("SQ_WAVE_CYCLES", 1000.0 * d), ("SQ_WAIT_ANY", 400.0 * d),
         ("SQ_INSTS_MFMA", 8192.0), ("SQ_VALU_MFMA_BUSY_CYCLES", 2048.0))] +
        [(9, "other_kernel", 0, "SQ_WAVES", 1.0)])
    p2 = _counters_db(tmp_path / "p2.db", [(d, k, 0, "SQ_INSTS_LDS", 40960.0) for d in (1, 2)])
    text = bench.summarize_sq([p1, p2])
    assert "`void w4a16::gemm8_kernel<2, true, 4>`" in text
    assert "| SQ_WAVE_CYCLES | 2,500 |" in text  # mean of dispatches 2 and 3
    assert "- MFMA instructions: 2.0" in text
    assert "- LDS instructions: 10.0" in text
    assert "waiting on s_waitcnt or a barrier: 40.0 %" in text
    assert "MFMA busy clocks per SIMD (over 1024 SIMDs): 2" in text


def test_summarize_sq_without_gemm_dispatches_exits(tmp_path):
    db = _counters_db(tmp_path / "n.db", [(1, "gemv_kernel", 0, "SQ_WAVES", 1.0)])
    with pytest.raises(SystemExit):
        bench.summarize_sq([db])


def test_summarize_trace_groups_by_kernel_and_grid(tmp_path):
    path = tmp_path / "t.db"
    con = sqlite3.connect(path)
    con.execute("create table kernels (name text, grid_x integer, duration integer)")
    con.executemany("insert into kernels values (?, ?, ?)", [
        ("void a(int)", 256, 2000), ("void a(int)", 256, 4000), ("void a(int)", 512, 1000), ("b", 64, 500)])
    con.commit()
    con.close()
    lines = bench.summarize_trace(str(path)).splitlines()
    assert lines[2] == "| `void a` | 256 | 2 | 3.00 | 3.00 | 2.00 |"
    assert "| `void a` | 512 | 1 | 1.00 | 1.00 | 1.00 |" in lines
    assert len(lines) == 5


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU only" in proc.stderr


def test_trace_kernel_names_the_planned_kernel(tmp_path):
    import synth
    pat, grid = bench.trace_kernel(synth.case_by_name("c3_gate_up_m1_k2048_n32768"))
    assert grid == 2048 * 4 * 64
    assert re.match(pat, "void w4a16::gemv_kernel<1, 1, 4, 4, 0, 4>")
    assert not re.match(pat, "void w4a16::gemv_kernel<1, 1, 4, 4, 0, 8>")  # INT8 codes
    pat, grid = bench.trace_kernel(synth.case_by_name("c4_m1024_k2048_n32768"))
    assert re.match(pat, "void w4a16::gemm8_kernel<2, true, 4, 256, 256, false>")
    assert not re.match(pat, "void w4a16::gemm8_kernel<2, true, 8, 256, 256, false>")
    assert not re.match(pat, "void w4a16::gemm8_kernel<2, true, 4, 256, 256, true>")  # stream-K
    # a summary row of that kernel is found by pattern and grid, INT8 rows skipped
    table = tmp_path / "t.md"
    table.write_text("| kernel | grid | launches | mean us | total us | share |\n|---|---|---|---|---|---|\n"
                     f"| `void w4a16::gemm8_kernel<2, true, 8, 256, 256, false>` | {grid} | 7 | 99.0 | 693 | 50 |\n"
                     f"| `void w4a16::gemm8_kernel<2, true, 4, 256, 256, false>` | {grid} | 10 | 12.5 | 125 | 50 |\n")
    assert bench.trace_row(str(table), pat, grid)[:2] == (12.5, 10)
