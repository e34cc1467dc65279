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
    # come from the last one (FETCH reads half the copy's bytes, WRITE all of them)
    fetch, write = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    _db(fetch, [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 1048576.0),
                (2, "index_scores_mfma<2, true>", "FETCH_SIZE", 1000.0),
                (3, "index_scores_mfma<2, true>", "FETCH_SIZE", 1002.0),
                (4, "index_scores_mfma<2, true>", "FETCH_SIZE", 1001.0),
                (5, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288.0)])
    _db(write, [(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 2097152.0),
                (2, "index_scores_mfma<2, true>", "WRITE_SIZE", 10.0),
                (3, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0)])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    bench.summarize_counters("unit", fetch, write)
    d = json.load(open(tmp_path / "profiles" / "index_score_unit_counters.json"))
    assert d["FETCH_SIZE"]["scale"] == 2.0 and d["WRITE_SIZE"]["scale"] == 1.0
    assert d["FETCH_SIZE"]["bytes_per_launch"] == 1001.0 * 1024 * 2
    assert d["traffic_bytes_per_launch"] == 1001.0 * 1024 * 2 + 10.0 * 1024
