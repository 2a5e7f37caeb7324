"""Host tests of profile_summary.py, the tool that turns rocprofv3 output into the summaries under
profiles/: the timed-region split of a kernel trace, per-position statistics of layer-by-layer steps,
per-dispatch counter sums and the copy-scaled traffic, on small synthetic CSV files."""
import csv
import json
import sys
from pathlib import Path
from types import SimpleNamespace

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))
import profile_summary as ps  # noqa: E402


def _trace(path, rows):
    """rows: (kernel name, start ns, end ns)."""
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for i, (name, t0, t1) in enumerate(rows):
            w.writerow(["KERNEL_DISPATCH", i + 1, name, t0, t1])


def _counters(path, rows):
    """rows: (dispatch id, kernel name, counter, value)."""
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow(r)


def test_trace_phases_follow_launch_order(tmp_path):
    # 3 warm-up launches of 10 us, 2 timed of 5 us, 2 isolated of 6 us, listed out of order, plus
    # another kernel in between that must be ignored
    rows, t = [], 1000
    for d in [10, 10, 10, 5, 5, 6, 6]:
        rows.append(("void k<1>(Args)", t, t + d * 1000))
        rows.append(("other_kernel", t + d * 1000, t + d * 1000 + 500))
        t += 20000
    _trace(tmp_path / "t.csv", rows[::-1])
    out = ps.trace(SimpleNamespace(csv=str(tmp_path / "t.csv"), kernel="void k<", phases="3,2,2", period=1))
    assert [p["n"] for p in out["phases"]] == [3, 2, 2]
    assert [p["mean"] for p in out["phases"]] == [10.0, 5.0, 6.0]
    assert out["all"]["n"] == 7


def test_trace_period_splits_launch_positions(tmp_path):
    # 4 steps of 3 launches each (durations 1, 2, 3 us per step), phases of 2 and 2 steps
    rows, t = [], 0
    for step in range(4):
        for pos, name in enumerate(["void a<1>(X)", "void b<2>(X)", "void a<1>(X)"]):
            rows.append((name, t, t + (pos + 1) * 1000))
            t += 10000
    _trace(tmp_path / "t.csv", rows)
    out = ps.trace(SimpleNamespace(csv=str(tmp_path / "t.csv"), kernel="void ", phases="2,2", period=3))
    by = out["by_position"]
    assert [(b["phase"], b["position"], b["n"], b["mean"]) for b in by] == [
        (0, 0, 2, 1.0), (0, 1, 2, 2.0), (0, 2, 2, 3.0), (1, 0, 2, 1.0), (1, 1, 2, 2.0), (1, 2, 2, 3.0)]
    assert by[1]["kernel"] == "b<2>"
    with pytest.raises(SystemExit):
        ps.trace(SimpleNamespace(csv=str(tmp_path / "t.csv"), kernel="void ", phases="3,2", period=3))


def test_counters_sum_per_dispatch_and_skip(tmp_path):
    rows = []
    for d in range(1, 6):  # each dispatch reports its counter in two parts (e.g. per XCD)
        rows += [(d, "void k(A)", "FETCH_SIZE", 10 * d), (d, "void k(A)", "FETCH_SIZE", 1)]
        rows += [(d, "copyBuffer", "FETCH_SIZE", 999)]
    _counters(tmp_path / "c.csv", rows)
    per = ps._per_dispatch(str(tmp_path / "c.csv"), "void k", skip=2)
    assert per["FETCH_SIZE"] == [31.0, 41.0, 51.0]


def test_traffic_scales_each_counter_by_the_copy(tmp_path, monkeypatch):
    kib = ps.COPY_PROBE_BYTES / 1024
    _counters(tmp_path / "f.csv", [(1, "void k(A)", "FETCH_SIZE", 100.0), (2, "void k(A)", "FETCH_SIZE", 100.0)])
    _counters(tmp_path / "w.csv", [(1, "void k(A)", "WRITE_SIZE", 50.0), (2, "void k(A)", "WRITE_SIZE", 50.0)])
    _counters(tmp_path / "cf.csv", [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", kib / 2)])
    _counters(tmp_path / "cw.csv", [(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", kib)])
    monkeypatch.setattr(ps, "kernel_source_hash", lambda: "0123456789abcdef")
    monkeypatch.setattr(ps, "ROOT", tmp_path)
    (tmp_path / "profiles").mkdir()
    rec = ps.traffic(SimpleNamespace(fetch=str(tmp_path / "f.csv"), write=str(tmp_path / "w.csv"),
                                     copy_fetch=str(tmp_path / "cf.csv"), copy_write=str(tmp_path / "cw.csv"),
                                     kernel="void k", workload="wl", label="k<>", algorithmic_bytes=300 * 1024,
                                     update=True))
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["bytes_per_launch"] == (200 + 50) * 1024
    saved = json.loads((tmp_path / "profiles" / "traffic.json").read_text())
    assert saved["wl"]["k<>"]["source_hash"] == "0123456789abcdef"
