"""Host-side pieces of bench.py that turn rocprofv3 results into the reported
numbers: kernel-name mapping and the HBM-traffic conversion (counter KiB per
dispatch, scaled by what the same counter reads for a copy of known size).
Runs on synthetic result databases with the tables rocprofv3 writes."""
from __future__ import annotations

import contextlib
import io
import json
import sqlite3

import pytest

import bench

ATTN = ("void h3a::(anonymous namespace)::attn_fwd_bf16_kernel<128, false, false, 0, 0>(unsigned short const*, "
        "unsigned short const*, unsigned short const*, unsigned short*, long, long, long, long, h3a::WorkItem const*, "
        "float, int, h3a::QNormArgs)")
NORM = ("void h3a::(anonymous namespace)::qk_norm_rope_kernel<h3a::(anonymous namespace)::Bf16Tag, 128, 0, 0>"
        "(char const*, char const*, char*, char*, long, long, long, long, int, int, int, float const*, "
        "float const*, float, float const*, int)")
TABLE = "h3a::(anonymous namespace)::rope_table_kernel(h3a::(anonymous namespace)::RopeArgs, float*, int, int)"
COPY = "__amd_rocclr_copyBuffer"


@pytest.mark.parametrize("name,short", [
    (ATTN, "attn_fwd_bf16_kernel<128>"),
    (ATTN.replace("<128, false, false, 0, 0>", "<128, true, false, 0, 0>"), "attn_fwd_bf16_kernel<128, causal>"),
    (ATTN.replace("<128, false, false, 0, 0>", "<128, false, false, 0, 2>"), "attn_fwd_bf16_kernel<128, fp8>"),
    (ATTN.replace("<128, false, false, 0, 0>", "<128, false, false, 0, 1>"), "attn_fwd_bf16_kernel<128, fp8qk>"),
    (ATTN.replace("<128, false, false, 0, 0>", "<128, false, true, 3, 0>"), "attn_fwd_bf16_kernel<128, qnorm r96>"),
    (ATTN.replace("<128, false, false, 0, 0>", "<128, false, false, 0, 3>"), "attn_fwd_bf16_kernel<128, i8qk>"),
    (ATTN.replace("<128, false, false, 0, 0>", "<128, true, false, 0, 4>"), "attn_fwd_bf16_kernel<128, causal, i8qk fp8pv>"),
    (NORM, bench.NORM_KERNEL),
    (TABLE, "rope_table_kernel"),
    (COPY, COPY),
])
def test_short_kernel_names(name, short):
    assert bench._short_kernel(name) == short


def _counter_db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?)", rows)
    con.commit()
    con.close()
    return str(path)


def test_traffic_conversion(tmp_path):
    """A 1 GiB copy whose FETCH_SIZE reads 0.5 GiB and WRITE_SIZE 1 GiB sets the
    scales to 2 and 1; per-kernel bytes are the dispatch average times the scale."""
    gib_kib = float(1 << 20)
    fetch = _counter_db(tmp_path / "f.db", [(ATTN, "FETCH_SIZE", 1000.0), (ATTN, "FETCH_SIZE", 3000.0),
                                            (NORM, "FETCH_SIZE", 500.0), (COPY, "FETCH_SIZE", 7.0)])
    write = _counter_db(tmp_path / "w.db", [(ATTN, "WRITE_SIZE", 100.0), (NORM, "WRITE_SIZE", 400.0)])
    cfetch = _counter_db(tmp_path / "cf.db", [(COPY, "FETCH_SIZE", gib_kib / 2)])
    cwrite = _counter_db(tmp_path / "cw.db", [(COPY, "WRITE_SIZE", gib_kib)])
    buf = io.StringIO()
    with contextlib.redirect_stdout(buf):
        assert bench.rocprof_traffic(fetch, write, cfetch, cwrite) == 0
    out = json.loads(buf.getvalue())
    assert out["fetch_scale"] == pytest.approx(2.0) and out["write_scale"] == pytest.approx(1.0)
    a = out["kernels"][bench.ATTN_KERNEL]
    assert a["hbm_read_bytes"] == pytest.approx(2000.0 * 1024 * 2)
    assert a["hbm_write_bytes"] == pytest.approx(100.0 * 1024)
    assert a["hbm_bytes_per_launch"] == pytest.approx(a["hbm_read_bytes"] + a["hbm_write_bytes"])
    n = out["kernels"][bench.NORM_KERNEL]
    assert n["hbm_read_bytes"] == pytest.approx(500.0 * 1024 * 2)
    assert COPY not in out["kernels"]  # only the library's kernels are reported
    assert set(out["source_sha256_16"]) == {"attn_fwd_bf16.hip", "qk_norm_rope.hip", "rope_table.hip"}



def test_kernel_trace_summary(tmp_path):
    """The kernel-trace table: rocprofv3's own per-kernel totals (microseconds) plus
    the average of the last N dispatches from their start/end stamps (nanoseconds)."""
    db = tmp_path / "t.db"
    con = sqlite3.connect(db)
    con.execute("create table top_kernels (name text, total_calls int, total_duration real, average real, "
                "percentage real)")
    con.execute("create table kernels (name text, start int, end int)")
    con.executemany("insert into top_kernels values (?, ?, ?, ?, ?)",
                    [(ATTN, 4, 11000.0, 2750.0, 97.0), (NORM, 4, 340.0, 85.0, 3.0)])
    t, rows = 0, []
    for dur_us in (3000.0, 2800.0, 2600.0, 2600.0):  # ATTN, then NORM after each
        rows.append((ATTN, t, t + int(dur_us * 1e3)))
        t += int(dur_us * 1e3) + 1000
        rows.append((NORM, t, t + 85000))
        t += 86000
    con.executemany("insert into kernels values (?, ?, ?)", rows)
    con.commit()
    con.close()
    buf = io.StringIO()
    with contextlib.redirect_stdout(buf):
        assert bench.rocprof_summary(str(db), 2) == 0
    lines = buf.getvalue().splitlines()
    attn = next(line for line in lines if line.startswith(f"| {bench.ATTN_KERNEL} |"))
    cells = [c.strip() for c in attn.strip("|").split("|")]
    assert cells == [bench.ATTN_KERNEL, "4", "11000.0", "2750.0", "2600.0", "97.00%"]
    assert any(line.startswith(f"| {bench.NORM_KERNEL} | 4 |") for line in lines)


def test_more_than_one_gpu_is_refused():
    """`bench.py --gpus N` with N > 1 stops with a message before touching a GPU."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout + r.stderr
