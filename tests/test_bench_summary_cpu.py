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


SCORE = "_ZN2rs12_GLOBAL__N_112score_kernelIDF16bEEvPKT_S4_Pfiii"
TOPK1 = "rs::(anonymous namespace)::topk_kernel<1>(float const*, float const*, int, int, int, int, int, float*, int*, int const*, int*, rs::(anonymous namespace)::RowCopy, rs::(anonymous namespace)::RowCopy, int)"


def _sa_db(path, dispatches, counters):
    """dispatches: (id, kernel_id, duration_ns, grid_x, lds, start); kernel 1 = rs_score's,
    2 = the top-k's; counters: (dispatch_id, name, value)."""
    con = sqlite3.connect(path)
    con.execute("create table kernel_symbols (id integer, kernel_name text)")
    con.executemany("insert into kernel_symbols values (?, ?)", [(1, SCORE), (2, TOPK1)])
    con.execute("create table kernels (dispatch_id integer, kernel_id integer, duration integer, "
                "grid_x integer, grid_y integer, grid_z integer, lds_size integer, start integer)")
    con.executemany("insert into kernels values (?, ?, ?, ?, 1, 1, ?, ?)", dispatches)
    con.execute("create table pmc_events (dispatch_id integer, counter_name text, counter_value real)")
    con.executemany("insert into pmc_events values (?, ?, ?)", counters)
    con.commit()
    con.close()


def test_standalone_summary_per_stage(tmp_path):
    """bench.py --summarize-standalone: stages told apart by launch shape in order of first
    appearance, median durations against the algorithmic bytes of each stage, and traffic
    calibrated by the copy probe (the top-k dispatch of over 100 us)."""
    known = 8 * 16384 * 8192 * 2
    d = tmp_path / "sa"
    d.mkdir()
    # DeiT-S stages: L 197 -> 138 -> 97 -> 68 (batch 256, C 384, bf16)
    disp, ctr, t = [], [], 0
    did = 0
    for stage, (grid, lds) in enumerate(((256 * 3152, 138 * 4), (256 * 2208, 97 * 4), (256 * 1552, 68 * 4))):
        for rep, dur in enumerate((10000, 12000, 14000)):     # score: median 12 us
            did += 1; t += 1
            disp.append((did, 1, dur + 1000 * stage, grid, 0, t))
            ctr += [(did, "FETCH_SIZE", 1000.0 * (stage + 1)), (did, "WRITE_SIZE", 10.0)]
        for rep, dur in enumerate((8000, 9000, 30000)):       # top-k: median 9 us
            did += 1; t += 1
            disp.append((did, 2, dur, 512 * 512, lds, t))
            ctr += [(did, "FETCH_SIZE", 500.0), (did, "WRITE_SIZE", 400.0)]
    did += 1; t += 1
    disp.append((did, 2, 700000, 512 * 512, 16384 * 4, t))        # the copy probe
    ctr += [(did, "FETCH_SIZE", known / 1024 / 2), (did, "WRITE_SIZE", known / 1024)]
    _sa_db(d / "a.db", disp, ctr)
    out = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--summarize-standalone", str(d),
                          "--workload", "deit_s"], capture_output=True, text=True, check=True, cwd=ROOT).stdout
    s = json.loads(out)
    assert abs(s["copy_probe_scale"]["FETCH_SIZE"] - 2.0) < 1e-12
    assert [(st["L"], st["k"]) for st in s["stages"]] == [(197, 138), (138, 97), (97, 68)]
    st0 = s["stages"][0]
    assert st0["score"]["dispatches"] == 3 and st0["score"]["median_us"] == 12.0
    assert st0["topk"]["dispatches"] == 3 and st0["topk"]["median_us"] == 9.0   # probe excluded
    algo_score = 2.0 * 256 * 197 * 384 * 2 + 4.0 * 256 * 197
    algo_topk = 256 * (4.0 * 197 + 2.0 * 138 * 384 * 2 + 4.0 * 138)
    assert st0["score"]["algorithmic_bytes"] == int(algo_score)
    assert st0["topk"]["algorithmic_bytes"] == int(algo_topk)
    assert abs(st0["score"]["frac_hbm_median"] - round(algo_score / 12e-6 / 8e12, 4)) < 1e-9
    assert st0["score"]["FETCH_SIZE_bytes"] == int(1000.0 * 1024 * 2)
    assert s["stages"][2]["score"]["FETCH_SIZE_bytes"] == int(3000.0 * 1024 * 2)
    t0 = st0["topk"]
    assert abs(t0["traffic_over_algorithmic"] - round((500.0 * 2 + 400.0) * 1024 / algo_topk, 3)) < 1e-9


def test_trace_table(tmp_path):
    """bench.py --summarize-trace: per-class totals of a kernel trace, split-K partial and
    reduction dispatches and the two LayerNorm preparation kernels listed apart."""
    d = tmp_path / "tr"
    d.mkdir()
    fc2 = FC1.replace("Li2ENS0_4Tile", "Li3ENS0_4Tile")
    fc2_split = fc2.replace("ELb0EEEvPKT_", "ELb1EEEvPKT_")
    rows = [(FC1, 0, 30000), (FC1, 100000, 150000), (fc2, 0, 60000), (fc2_split, 0, 20000),
            ("_ZN2rs12_GLOBAL__N_111fold_kernelIDF16bEEvNS0_8FoldArgsE", 0, 7000),
            ("_ZN2rs12_GLOBAL__N_116row_stats_kernelIDF16bEEvPKT_Pfii", 0, 9000),
            ("void at::native::elementwise_kernel<...>", 0, 999999)]
    with open(d / "x_kernel_trace.csv", "w") as f:
        f.write('"Kind","Kernel_Name","Start_Timestamp","End_Timestamp"\n')
        for name, a, b in rows:
            f.write(f'"KERNEL_DISPATCH","{name}",{a},{b}\n')
    out = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--summarize-trace", str(d)],
                         capture_output=True, text=True, check=True, cwd=ROOT).stdout
    lines = {l.split("|")[1].strip(): [c.strip() for c in l.split("|")[2:-1]]
             for l in out.splitlines() if l.startswith("| ") and not l.startswith("| kernel")}
    assert set(lines) == {"fc1", "fc2_score", "fc2_score (split-K partial)", "ln_prep (fold)",
                          "ln_prep (row stats)"}
    assert lines["fc1"][:3] == ["2", "0.080", "40.00"]           # 30 + 50 us
    total = 30000 + 50000 + 60000 + 20000 + 7000 + 9000
    assert abs(float(lines["fc2_score"][-1]) - 100.0 * 60000 / total) < 0.01
