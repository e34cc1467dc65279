"""Host logic of bench.py that runs without a GPU: the one-GPU contract and the HBM-counter
calibration on a synthetic rocprofv3 counter database."""
import json
import os
import sqlite3
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (dispatch_id integer, kernel_name text, "
                "counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def test_counter_summary_calibrates_on_the_last_copy(tmp_path, monkeypatch):
    # a pool clone (a large copy) comes first, the 1 GiB calibration copy last: the scale must
    # come from the last one (FETCH reads half the copy's bytes, WRITE all of them). A part of two
    # kernels (attend + combine) adds its launches within a step; the median is over steps.
    fetch, write = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    sc = "void (anonymous namespace)::index_scores_mfma<2, true, 0>(DevPlan, RowMap)"
    _db(fetch, [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 1048576.0),
                (2, sc, "FETCH_SIZE", 1000.0),
                (3, "attend_f8_split", "FETCH_SIZE", 300.0),
                (4, "attend_combine", "FETCH_SIZE", 50.0),
                (5, sc, "FETCH_SIZE", 1002.0),
                (6, "attend_f8_split", "FETCH_SIZE", 310.0),
                (7, "attend_combine", "FETCH_SIZE", 60.0),
                (8, sc, "FETCH_SIZE", 1001.0),
                (9, "attend_f8_split", "FETCH_SIZE", 305.0),
                (10, "attend_combine", "FETCH_SIZE", 40.0),
                (11, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288.0)])
    _db(write, [(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 2097152.0),
                (2, sc, "WRITE_SIZE", 10.0),
                (3, "attend_f8_split", "WRITE_SIZE", 7.0),
                (4, "attend_combine", "WRITE_SIZE", 1.0),
                (5, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0)])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    bench.summarize_counters("unit", fetch, write)
    d = json.load(open(tmp_path / "profiles" / "unit_hbm_counters.json"))["parts"]
    assert d["score"]["FETCH_SIZE"]["scale"] == 2.0 and d["score"]["WRITE_SIZE"]["scale"] == 1.0
    assert d["score"]["FETCH_SIZE"]["bytes_per_step"] == 1001.0 * 1024 * 2
    assert d["score"]["traffic_bytes_per_step"] == 1001.0 * 1024 * 2 + 10.0 * 1024
    # attend steps: 350, 370, 345 KiB read -> median 350; one step written: 8 KiB
    assert d["attend"]["FETCH_SIZE"]["kib_per_step_median"] == 350.0
    assert d["attend"]["traffic_bytes_per_step"] == 350.0 * 1024 * 2 + 8.0 * 1024
    # the part's sources are hashed, so that later kernel changes make the figures stale
    assert d["attend"]["source_hash"] == bench.kernel_source_hash("attend")
