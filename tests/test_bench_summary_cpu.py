"""Host logic of the measurement tooling (no GPU): bench.py --summarize on a small result
database with the columns rocprofv3 writes, checking the copy-probe calibration of the
traffic counters, the matrix-core busy fraction and the grouping by launch shape."""
import json
import sqlite3
import subprocess
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]

FC1 = "_ZN2rs12_GLOBAL__N_111gemm_kernelIDF16bLi2ENS0_4TileIDF16bLi2ELi2ELi4ELi4ELi1ELi8ELi2ELi1EEELb0EEEvPKT_S6_iiiiNS_11GemmEpiArgsE"
TOPK = "_ZN2rs12_GLOBAL__N_111topk_kernelEPKfS2_iiiiiPfPiPKiS4_NS0_7RowCopyES6_i"


def _db(path, dispatches, counters):
    """dispatches: (id, kernel_id, duration_ns, grid); counters: (dispatch_id, name, value)."""
    con = sqlite3.connect(path)
    con.execute("create table kernel_symbols (id integer, kernel_name text)")
    con.executemany("insert into kernel_symbols values (?, ?)", [(1, FC1), (2, TOPK)])
    con.execute("create table kernels (dispatch_id integer, kernel_id integer, duration integer, "
                "grid_x integer, grid_y integer, grid_z integer)")
    con.executemany("insert into kernels values (?, ?, ?, ?, 1, 1)", dispatches)
    con.execute("create table pmc_events (dispatch_id integer, counter_name text, counter_value real)")
    con.executemany("insert into pmc_events values (?, ?, ?)", counters)
    con.commit()
    con.close()


def _summarize(*dirs):
    out = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--summarize", *map(str, dirs)],
                         capture_output=True, text=True, check=True, cwd=ROOT).stdout
    return json.loads(out)


def test_traffic_calibrated_by_the_copy_probe(tmp_path):
    known = 8 * 16384 * 8192 * 2
    fetch, write = tmp_path / "fetch", tmp_path / "write"
    fetch.mkdir()
    write.mkdir()
    # two fc1 dispatches and a 2 GiB probe (a top-k dispatch of over 100 us) whose counters
    # read half (FETCH_SIZE) and all (WRITE_SIZE) of the copied KiB
    disp = [(1, 1, 40000, 256 * 100), (2, 1, 42000, 256 * 100), (3, 2, 600000, 1024 * 128)]
    _db(fetch / "a.db", disp, [(1, "FETCH_SIZE", 1000.0), (2, "FETCH_SIZE", 3000.0),
                               (3, "FETCH_SIZE", known / 1024 / 2)])
    _db(write / "a.db", disp, [(1, "WRITE_SIZE", 500.0), (2, "WRITE_SIZE", 500.0),
                               (3, "WRITE_SIZE", known / 1024)])
    s = _summarize(fetch, write)
    assert abs(s["copy_probe"]["scale"]["FETCH_SIZE"] - 2.0) < 1e-12
    assert abs(s["copy_probe"]["scale"]["WRITE_SIZE"] - 1.0) < 1e-12
    k = s["kernels"]["fc1"]
    assert k["dispatches"] == 2
    assert abs(k["FETCH_SIZE_bytes"] - 2000.0 * 1024 * 2.0) < 1e-6
    assert abs(k["WRITE_SIZE_bytes"] - 500.0 * 1024) < 1e-6
    assert abs(k["traffic_bytes_per_launch"] - (4096000.0 + 512000.0)) < 1e-6
    assert "topk" not in s["kernels"]          # the probe is not an encoder dispatch


def test_busy_fraction_overall_and_per_launch_shape(tmp_path):
    d = tmp_path / "mfma"
    d.mkdir()
    # 1024 SIMDs x 10 us x 2.4 GHz = 24.576e6 cycles; busy 6.144e6 -> 0.25
    disp = [(1, 1, 10000, 256 * 1773), (2, 1, 10000, 256 * 1773), (3, 1, 20000, 256 * 612)]
    _db(d / "a.db", disp, [(1, "SQ_VALU_MFMA_BUSY_CYCLES", 6.144e6),
                           (2, "SQ_VALU_MFMA_BUSY_CYCLES", 6.144e6),
                           (3, "SQ_VALU_MFMA_BUSY_CYCLES", 6.144e6)])
    k = _summarize(d)["kernels"]["fc1"]
    g = k["by_grid"]
    assert set(g) == {str(256 * 1773), str(256 * 612)}
    assert g[str(256 * 1773)]["dispatches"] == 2
    assert abs(g[str(256 * 1773)]["mfma_busy_frac"] - 0.25) < 1e-12
    assert abs(g[str(256 * 612)]["mfma_busy_frac"] - 0.125) < 1e-12
    # overall: mean counter over mean duration
    assert abs(k["mfma_busy_frac"] - 6.144e6 / (1024 * (40000 / 3) * 2.4)) < 1e-12
