"""Host logic of the rocprofv3 summaries (profiling.py) on small synthetic CSV files:
the counter mean per dispatch (rows of one dispatch summed first, optionally only
the last N dispatches), the copy-kernel calibration of the traffic figure, the
source digest that ignores comments, and the grouping of trace rows by launch
shape with the longest uninterrupted run."""
import csv
import json

import pytest

from hybrid_linear_temporal_hta_amd import profiling as pf


def _counters(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        wr.writeheader()
        for d, k, c, v in rows:
            wr.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": c,
                         "Counter_Value": v})


def test_counter_per_dispatch_sums_rows_and_takes_last(tmp_path):
    p = tmp_path / "run_counter_collection.csv"
    k = "hta::win_attn_bf16_kernel<3>(hta::WinLaunch)"
    _counters(p, [
        (1, k, "FETCH_SIZE", 10.0), (1, k, "FETCH_SIZE", 5.0),   # one dispatch, two rows
        (2, "other", "FETCH_SIZE", 1e9),                          # another kernel
        (3, k, "FETCH_SIZE", 30.0),
        (4, k, "WRITE_SIZE", 7.0),                                # another counter
        (5, k, "FETCH_SIZE", 50.0),
    ])
    mean, n = pf.counter_per_dispatch(str(tmp_path), "FETCH_SIZE", "win_attn_bf16_kernel<3>")
    assert n == 3 and mean == pytest.approx((15.0 + 30.0 + 50.0) / 3)
    mean, n = pf.counter_per_dispatch(str(p), "FETCH_SIZE", "win_attn_bf16_kernel<3>", last=2)
    assert n == 2 and mean == pytest.approx(40.0)   # dispatches 3 and 5, by id
    with pytest.raises(ValueError):
        pf.counter_per_dispatch(str(p), "FETCH_SIZE", "win_attn_bf16_kernel<3>", last=4)
    with pytest.raises(ValueError):
        pf.counter_per_dispatch(str(p), "FETCH_SIZE", "absent_kernel")


def test_traffic_scales_by_the_copy_kernel(tmp_path):
    k = "hta::win_attn_bf16_kernel<3>(hta::WinLaunch)"
    cp = "(anonymous namespace)::hbm_copy_kernel(x)"
    for name, counter, kv, cv in (("f", "FETCH_SIZE", 2000.0, 500.0), ("w", "WRITE_SIZE", 300.0, 1000.0)):
        (tmp_path / name).mkdir()
        (tmp_path / ("c" + name)).mkdir()
        _counters(tmp_path / name / "run_counter_collection.csv",
                  [(1, k, counter, kv / 2), (2, k, counter, kv), (3, k, counter, kv)])
        _counters(tmp_path / ("c" + name) / "run_counter_collection.csv", [(1, cp, counter, cv)])
    src = tmp_path / "k.hip"
    src.write_text("int a; // note\n")
    out = tmp_path / "prof" / "t.json"
    out.parent.mkdir()
    pf.main(["traffic", "--kernel", "win_attn_bf16_kernel<3>", "--last", "2",
             "--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w"),
             "--copy-fetch", str(tmp_path / "cf"), "--copy-write", str(tmp_path / "cw"),
             "--copy-bytes", "1000000", "--source", str(src), "--out", str(out),
             "--command", "synthetic"])
    rec = json.loads(out.read_text())
    # the copy moves 1e6 bytes each way: 1e6 / 500 bytes per fetch unit, 1e3 per write unit
    assert rec["bytes_per_fetch_unit"] == pytest.approx(2000.0)
    assert rec["bytes_per_write_unit"] == pytest.approx(1000.0)
    assert rec["hbm_read_bytes_per_launch"] == pytest.approx(2000.0 * 2000.0)
    assert rec["hbm_write_bytes_per_launch"] == pytest.approx(300.0 * 1000.0)
    assert rec["dispatches"] == [2, 2]
    assert rec["source_digest"] == pf.source_digest(str(src))


def test_source_digest_ignores_comments_only(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f() {\n  return 1;  // one\n}\n")
    b.write_text("/* header\n   text */\nint f() {\n\n  return 1;\n}\n")
    c.write_text("int f() {\n  return 2;\n}\n")
    assert pf.source_digest(str(a)) == pf.source_digest(str(b))
    assert pf.source_digest(str(a)) != pf.source_digest(str(c))


def test_trace_by_grid_groups_shapes_and_finds_runs(tmp_path):
    p = tmp_path / "run_kernel_trace.csv"
    rows = []
    t = 0

    def add(name, grid, dur_us):
        nonlocal t
        rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + int(dur_us * 1e3),
                     "Grid_Size_X": grid * 256, "Workgroup_Size_X": 256})
        t += int(dur_us * 1e3) + 1000

    add("hta::a_kernel(x)", 100, 10.0)
    add("hta::a_kernel(x)", 100, 12.0)
    add("hta::b_kernel(x)", 5, 1.0)
    add("hta::a_kernel(x)", 100, 20.0)
    add("hta::a_kernel(x)", 7, 3.0)
    for _ in range(3):
        add("hta::a_kernel(x)", 100, 30.0)
    with open(p, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=list(rows[0]))
        wr.writeheader()
        wr.writerows(rows)
    got = {(r["kernel"], r["workgroups"]): r for r in pf.trace_by_grid(str(tmp_path))}
    a100 = got[("hta::a_kernel", 100)]
    assert a100["calls"] == 6
    assert a100["avg_us"] == pytest.approx((10 + 12 + 20 + 90) / 6)
    assert a100["run_calls"] == 3 and a100["run_avg_us"] == pytest.approx(30.0)
    assert got[("hta::a_kernel", 7)]["calls"] == 1
    assert got[("hta::b_kernel", 5)]["run_calls"] == 1
