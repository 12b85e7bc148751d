"""Host-side checks of the counter summaries behind roofline.traffic (no GPU)."""
from __future__ import annotations

import csv
import importlib.util
import os

import pytest

from cross_model_sparse_amd import profile_summary as ps

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, v) in enumerate(rows, 1):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": name,
                        "Counter_Name": counter, "Counter_Value": v})


def _run(fetch_ref, write_ref, k_fetch, k_write, mib=256):
    """Dispatch order of bench.py --copy-ref-mib: a capacity pass (block mass,
    gather), the copy reference (a fill, three copies), then the timed step."""
    def rows(ref, kval, fill):
        return [("k_block_mass<x>", 5.0), ("k_gather<x>", 7.0),
                ("vectorized_elementwise_kernel<FillFunctor>", fill),
                ("vectorized_elementwise_kernel<MulFunctor>", ref),
                ("vectorized_elementwise_kernel<MulFunctor>", ref),
                ("vectorized_elementwise_kernel<MulFunctor>", ref),
                ("k_block_mass<x>", 5.0), ("k_gather<x>", 7.0),
                ("k_retrieve_mfma<true, 5, 2>", kval),
                ("k_block_mass<x>", 5.0), ("k_gather<x>", 7.0),
                ("k_retrieve_mfma<true, 5, 2>", kval)]
    return rows(fetch_ref, k_fetch, 0.0), rows(write_ref, k_write, mib * 1024.0)


def test_traffic_scales_each_counter_by_the_copy(tmp_path):
    # a fetch counter that reports half the bytes, a write counter that is exact
    f_rows, w_rows = _run(fetch_ref=131072.0, write_ref=262144.0, k_fetch=100000.0, k_write=50000.0)
    _write(tmp_path / "f.csv", "FETCH_SIZE", f_rows)
    _write(tmp_path / "w.csv", "WRITE_SIZE", w_rows)
    rec = ps.traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 256, "k_retrieve_mfma", "a", "b")
    kv = dict(line.split(": ", 1) for line in rec.splitlines() if not line.startswith("#"))
    assert float(kv["fetch_scale"]) == pytest.approx(2.0)
    assert float(kv["write_scale"]) == pytest.approx(1.0)
    assert float(kv["fetch_bytes_per_launch"]) == pytest.approx(100000.0 * 1024 * 2, rel=1e-6)
    assert float(kv["write_bytes_per_launch"]) == pytest.approx(50000.0 * 1024, rel=1e-6)
    assert float(kv["hbm_bytes_per_launch"]) == pytest.approx((200000.0 + 50000.0) * 1024, rel=1e-6)
    assert kv["dispatches_fetch_run"] == "2"


def test_traffic_without_copy_reference_is_an_error(tmp_path):
    f_rows, w_rows = _run(fetch_ref=131072.0, write_ref=262144.0, k_fetch=1.0, k_write=1.0)
    f_rows = [r for r in f_rows if "MulFunctor" not in r[0]]
    _write(tmp_path / "f.csv", "FETCH_SIZE", f_rows)
    _write(tmp_path / "w.csv", "WRITE_SIZE", w_rows)
    with pytest.raises(SystemExit):
        ps.traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 256, "k_retrieve_mfma", "a", "b")


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_bench_reports_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    bench = _bench()
    rec = tmp_path / "traffic.txt"
    body = ("fetch_bytes_per_launch: 300\nwrite_bytes_per_launch: 100\n"
            "hbm_bytes_per_launch: 400\n")
    rec.write_text(f"kernel_source_sha256: {bench.kernel_source_hash()}\n" + body)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    t = bench.recorded_traffic()
    assert t is not None and t["bytes_per_launch"] == 400.0
    rec.write_text("kernel_source_sha256: " + "0" * 64 + "\n" + body)
    assert bench.recorded_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.recorded_traffic() is None


def test_committed_traffic_record_is_well_formed():
    bench = _bench()
    path = bench.TRAFFIC_FILE
    assert os.path.exists(path), path
    kv = dict(line.split(": ", 1) for line in open(path).read().splitlines()
              if line and not line.startswith("#"))
    fb, wb, hb = (float(kv[k]) for k in ("fetch_bytes_per_launch", "write_bytes_per_launch",
                                         "hbm_bytes_per_launch"))
    assert hb == pytest.approx(fb + wb, abs=2)
    assert len(kv["kernel_source_sha256"]) == 64
    # the record is of the kernel the bench names for its roofline
    assert kv["kernel"].startswith("k_retrieve_pair<")


def test_traffic_with_all_layers_compressed_before_the_retrievals(tmp_path):
    # the step compresses every layer, then retrieves every layer, then the
    # warm order runs; only the step's first launches are averaged with first=2
    def rows(ref, fill, k):
        return [("k_block_mass<x>", 5.0), ("k_gather<x>", 7.0), ("k_block_mass<x>", 5.0),
                ("k_gather<x>", 7.0),
                ("vectorized_elementwise_kernel<FillFunctor>", fill),
                ("vectorized_elementwise_kernel<MulFunctor>", ref),
                ("vectorized_elementwise_kernel<MulFunctor>", ref),
                ("k_block_mass<x>", 5.0), ("k_gather<x>", 7.0),
                ("k_block_mass<x>", 5.0), ("k_gather<x>", 7.0),
                ("k_retrieve_pair<true, 5, 2, false, false>", k),
                ("k_retrieve_pair<true, 5, 2, false, false>", k),
                ("k_block_mass<x>", 5.0), ("k_gather<x>", 7.0),
                ("k_retrieve_pair<true, 5, 2, false, false>", 10 * k)]
    _write(tmp_path / "f.csv", "FETCH_SIZE", rows(131072.0, 0.0, 1000.0))
    _write(tmp_path / "w.csv", "WRITE_SIZE", rows(262144.0, 262144.0, 100.0))
    rec = ps.traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 256, "k_retrieve_pair",
                     "a", "b", first=2)
    kv = dict(line.split(": ", 1) for line in rec.splitlines() if not line.startswith("#"))
    assert kv["dispatches_fetch_run"] == "2"
    assert float(kv["fetch_bytes_per_launch"]) == pytest.approx(1000.0 * 1024 * 2)
    assert float(kv["write_bytes_per_launch"]) == pytest.approx(100.0 * 1024)
    rec = ps.traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 256, "k_retrieve_pair",
                     "a", "b")
    kv = dict(line.split(": ", 1) for line in rec.splitlines() if not line.startswith("#"))
    assert kv["dispatches_fetch_run"] == "3"


def _write_pmc(path, dispatches):
    """dispatches: [(name, duration ns, {counter: value})]"""
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
              "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for i, (name, dur, cs) in enumerate(dispatches, 1):
            for c, v in cs.items():
                w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": c,
                            "Counter_Value": v, "Start_Timestamp": 1000,
                            "End_Timestamp": 1000 + dur})


def test_counter_fractions_use_per_xcd_cycles_and_unit_counts(tmp_path):
    # 100 us at 2 GHz: 200000 cycles per XCD, 1.6e6 summed over 8 XCDs
    cyc = 200000.0
    p1 = {"GRBM_GUI_ACTIVE": 8 * cyc, "TA_TA_BUSY_sum": 0.5 * cyc * 256,
          "TD_TD_BUSY_sum": 0.25 * cyc * 256, "TCP_TCC_READ_REQ_LATENCY_sum": 4000.0,
          "TCP_TCC_READ_REQ_sum": 10.0}
    p2 = {"GRBM_GUI_ACTIVE": 8 * cyc, "SQ_VALU_MFMA_BUSY_CYCLES": 0.75 * cyc * 1024,
          "SQ_LDS_IDX_ACTIVE": 0.125 * cyc * 256}
    _write_pmc(tmp_path / "p1.csv", [("other", 5, {"GRBM_GUI_ACTIVE": 1.0}),
                                     ("k_retrieve_pair<x>", 100000, p1)])
    _write_pmc(tmp_path / "p2.csv", [("k_retrieve_pair<x>", 100000, p2)])
    rec = ps.counters([str(tmp_path / "p1.csv"), str(tmp_path / "p2.csv")], "k_retrieve_pair",
                      ["one", "two"])
    frac = {}
    for line in rec.split("fraction of the kernel's active cycles:")[1].splitlines():
        parts = line.rsplit(None, 1)
        if len(parts) == 2 and line.startswith("  "):
            frac[parts[0].strip()] = float(parts[1])
    assert frac["TA busy"] == pytest.approx(0.5, abs=1e-3)
    assert frac["TD busy"] == pytest.approx(0.25, abs=1e-3)
    assert frac["MFMA busy (MfmaUtil)"] == pytest.approx(0.75, abs=1e-3)
    assert frac["LDS active (LdsUtil)"] == pytest.approx(0.125, abs=1e-3)
    assert "busiest unit: MFMA busy (MfmaUtil)" in rec
    assert "2.00 GHz" in rec and "400.0" in rec          # clock and L1->L2 latency
    assert "# pass 2: two" in rec


def test_traffic_of_a_kernel_that_also_runs_in_the_capacity_pass(tmp_path):
    # block mass runs before the copy reference too; only the step's dispatches count
    f_rows, w_rows = _run(fetch_ref=131072.0, write_ref=262144.0, k_fetch=1.0, k_write=1.0)
    f_rows[0] = ("k_block_mass<x>", 999.0)       # capacity pass: excluded
    _write(tmp_path / "f.csv", "FETCH_SIZE", f_rows)
    _write(tmp_path / "w.csv", "WRITE_SIZE", w_rows)
    rec = ps.traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 256, "k_block_mass", "a", "b",
                     source=ps.__file__)
    kv = dict(line.split(": ", 1) for line in rec.splitlines() if not line.startswith("#"))
    assert float(kv["FETCH_SIZE_KiB_per_dispatch"]) == pytest.approx(5.0)
    assert kv["dispatches_fetch_run"] == "2"
    assert kv["kernel_source"].endswith("profile_summary.py")
