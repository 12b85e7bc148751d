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
    path = os.path.join(ROOT, "profiles", "k_retrieve_mfma_pair14b8b_bf16_N8192_traffic.txt")
    kv = dict(line.split(": ", 1) for line in open(path).read().splitlines()
              if line and not line.startswith("#"))
    fb, wb, hb = (float(kv[k]) for k in ("fetch_bytes_per_launch", "write_bytes_per_launch",
                                         "hbm_bytes_per_launch"))
    assert hb == pytest.approx(fb + wb, abs=2)
    assert len(kv["kernel_source_sha256"]) == 64


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
