"""Short text summaries of rocprofv3 output for the profiles/ folder.

    python -m cross_model_sparse_amd.profile_summary stats STATS_CSV --command CMD [--match TEXT ...]
        per-kernel call count and average / total duration from a
        `rocprofv3 --kernel-trace --stats` run (run_kernel_stats.csv),
        optionally only for kernels whose names contain one of the TEXTs

    python -m cross_model_sparse_amd.profile_summary counters PASS_CSV... --kernel NAME \\
        --command CMD [--command CMD ...] [--first K] [--skip S]
        per-dispatch means of the counters of several `rocprofv3 --pmc` passes
        over the same command, and the fraction of the kernel's active cycles
        each texture-path, LDS, VALU and MFMA unit was busy or stalled

    python -m cross_model_sparse_amd.profile_summary traffic \\
        --fetch FETCH_CSV --write WRITE_CSV --copy-mib M --kernel NAME \\
        --fetch-command CMD --write-command CMD
        HBM bytes per launch of NAME from two `rocprofv3 --pmc` runs (one with
        FETCH_SIZE, one with WRITE_SIZE, both KiB per dispatch).  Each counter is
        scaled by what it reads for a plain copy kernel of known size run in the
        same command (M MiB read and M MiB written per launch, run by
        bench.py --copy-ref-mib M).  The record carries the SHA-256 of the kernel's
        source (--source, default the retrieval kernel's) so a reader can tell
        whether the kernel changed since.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SRC = os.path.join(HERE, "csrc", "k_retrieve.hip")


def _short(name: str, n: int = 90) -> str:
    name = name.replace("(anonymous namespace)::", "")
    return name if len(name) <= n else name[: n - 3] + "..."


def stats(path: str, command: str, top: int = 12, match=None) -> str:
    rows = list(csv.DictReader(open(path)))
    if match:
        rows = [r for r in rows if any(m in r["Name"] for m in match)]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"# rocprofv3 --kernel-trace --stats summary", f"command: {command}", "",
           f"{'calls':>6} {'avg_us':>10} {'total_ms':>10} {'pct':>6}  kernel"]
    for r in rows[:top]:
        out.append(f"{int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} "
                   f"{float(r['TotalDurationNs']) / 1e6:>10.3f} {float(r['Percentage']):>6.2f}  "
                   f"{_short(r['Name'])}")
    return "\n".join(out) + "\n"


def _dispatches(path: str, counter: str):
    """[(dispatch id, kernel name, value KiB)] in dispatch order."""
    rows = [(int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"]))
            for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    rows.sort()
    return rows


def _reference_window(rows, want: float):
    """(lo, hi): bench.py --copy-ref-mib runs the copy reference after the
    capacity pass and before the first timed step, so it lies between two
    consecutive gather dispatches -- the capacity pass's last (lo) and the
    step's first (hi) -- that precede the first retrieval launch, and it is
    the only pair of them with a large elementwise dispatch in between."""
    first = next(i for i, r in enumerate(rows) if "k_retrieve_" in r[1])
    g = [i for i in range(first) if "k_gather" in rows[i][1]]
    for lo, hi in zip(g, g[1:]):
        if any("elementwise" in rows[k][1] and rows[k][2] > 0.25 * want for k in range(lo + 1, hi)):
            return lo, hi
    raise SystemExit("no copy-reference dispatch found between the capacity pass and the step")


def _copy_reference(rows, mib: int):
    """Counter value of the copy reference: the median of the elementwise
    dispatches in the reference window (the fill that creates the source reads
    nothing and is skipped by the > 1/4 size test in the fetch run)."""
    want = mib * 1024.0
    lo, hi = _reference_window(rows, want)
    vals = [v for _, name, v in rows[lo + 1:hi]
            if "elementwise" in name and v > 0.25 * want]
    if not vals:
        raise SystemExit("no copy-reference dispatch found in the counter file")
    vals.sort()
    return vals[len(vals) // 2]


def _kernel_mean(rows, kernel: str, want: float, first=None):
    """Mean counter value (KiB) and count of `kernel`'s dispatches after the
    capacity pass (the timed steps' launches; only the first `first` of them
    when given)."""
    lo, _ = _reference_window(rows, want)
    vals = [v for _, name, v in rows[lo + 1:] if kernel in name]
    if first:
        vals = vals[:first]
    if not vals:
        raise SystemExit(f"no dispatch of {kernel} after the capacity pass")
    return sum(vals) / len(vals), len(vals)


def traffic(fetch_csv, write_csv, mib, kernel, fetch_cmd, write_cmd, source=KERNEL_SRC,
            first=None) -> str:
    fetch = _dispatches(fetch_csv, "FETCH_SIZE")
    write = _dispatches(write_csv, "WRITE_SIZE")
    want = mib * 1024.0
    f_ref = _copy_reference(fetch, mib)
    w_ref = _copy_reference(write, mib)
    f_scale = want / f_ref
    w_scale = want / w_ref
    f_kib, nf = _kernel_mean(fetch, kernel, want, first)
    w_kib, nw = _kernel_mean(write, kernel, want, first)
    fb = f_kib * 1024 * f_scale
    wb = w_kib * 1024 * w_scale
    src_hash = hashlib.sha256(open(source, "rb").read()).hexdigest()
    lines = [
        f"# HBM traffic of {kernel} from hardware counters",
        "# REPO = repository root",
        f"# fetch run: {fetch_cmd}",
        f"# write run: {write_cmd}",
        f"kernel: {kernel}",
        f"kernel_source: {os.path.relpath(source, os.path.dirname(HERE))}",
        f"kernel_source_sha256: {src_hash}",
        f"dispatches_fetch_run: {nf}",
        f"dispatches_write_run: {nw}",
        f"FETCH_SIZE_KiB_per_dispatch: {f_kib:.1f}",
        f"WRITE_SIZE_KiB_per_dispatch: {w_kib:.1f}",
        f"copy_reference_MiB_read_and_written: {mib}",
        f"copy_reference_FETCH_SIZE_KiB: {f_ref:.1f}",
        f"copy_reference_WRITE_SIZE_KiB: {w_ref:.1f}",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        f"fetch_bytes_per_launch: {fb:.0f}",
        f"write_bytes_per_launch: {wb:.0f}",
        f"hbm_bytes_per_launch: {fb + wb:.0f}",
    ]
    return "\n".join(lines) + "\n"


# Unit counts of the MI355X (gfx950) used to turn summed counters into
# fractions of the kernel's time: 8 XCDs (each reports its own
# GRBM_GUI_ACTIVE), 256 active CUs, 4 SIMDs per CU.
XCDS, CUS, SIMDS = 8, 256, 1024


def _pmc_rows(path: str):
    """{dispatch id: (kernel name, duration ns, {counter: value})}."""
    out = {}
    for r in csv.DictReader(open(path)):
        d = int(r["Dispatch_Id"])
        if d not in out:
            dur = int(r.get("End_Timestamp") or 0) - int(r.get("Start_Timestamp") or 0)
            out[d] = (r["Kernel_Name"], dur, {})
        out[d][2][r["Counter_Name"]] = float(r["Counter_Value"])
    return out


def unit_fractions(c: dict) -> dict:
    """Busy / stall fractions of the kernel's active time from one dispatch's
    summed counters (only those whose counters are present).  Per-XCD active
    cycles = GRBM_GUI_ACTIVE / 8; the formulas follow rocprofv3's derived
    metrics (MfmaUtil, LdsUtil, LDSBankConflict, VALUBusy) with CU_NUM = 256
    and SIMD_NUM = 1024, and divide the per-CU texture-path counters (summed
    over instances) by 256 CUs."""
    g = c.get("GRBM_GUI_ACTIVE")
    if not g:
        return {}
    cyc = g / XCDS
    per_cu = {"TA busy": "TA_TA_BUSY_sum", "TA address stalled by L1": "TA_ADDR_STALLED_BY_TC_CYCLES_sum",
              "TD busy": "TD_TD_BUSY_sum", "TD stalled by L1": "TD_TC_STALL_sum",
              "L1 pending-request stall": "TCP_PENDING_STALL_CYCLES_sum",
              "L1 stalls TA data": "TCP_TCP_TA_DATA_STALL_CYCLES_sum",
              "LDS active (LdsUtil)": "SQ_LDS_IDX_ACTIVE",
              "LDS bank conflict": "SQ_LDS_BANK_CONFLICT",
              "LDS data FIFO full": "SQ_LDS_DATA_FIFO_FULL",
              "VALU busy (VALUBusy)": "SQ_ACTIVE_INST_VALU"}
    f = {k: c[v] / (cyc * CUS) for k, v in per_cu.items() if v in c}
    if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
        f["MFMA busy (MfmaUtil)"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * SIMDS)
    return f


def counters(csvs, kernel: str, commands, first=None, skip=0) -> str:
    """Average of each counter over `kernel`'s dispatches (after skipping
    `skip`, then the first `first`) in every pass, the unit fractions derived
    from them, and the unit with the largest busy fraction."""
    merged, fr, durs, n_disp, clk = {}, {}, [], [], []
    for path in csvs:
        disp = [v for _, v in sorted(_pmc_rows(path).items()) if kernel in v[0]][skip:]
        disp = disp[:first] if first else disp
        if not disp:
            raise SystemExit(f"no dispatch of {kernel} in {path}")
        n_disp.append(len(disp))
        for name in disp[0][2]:
            merged.setdefault(name, sum(d[2].get(name, 0.0) for d in disp) / len(disp))
        per = [unit_fractions(d[2]) for d in disp]
        for k in per[0]:
            fr.setdefault(k, sum(p[k] for p in per) / len(per))
        durs += [d[1] for d in disp]
        clk += [d[2]["GRBM_GUI_ACTIVE"] / XCDS / d[1] for d in disp
                if d[1] > 0 and "GRBM_GUI_ACTIVE" in d[2]]
    lat = None
    if "TCP_TCC_READ_REQ_LATENCY_sum" in merged and merged.get("TCP_TCC_READ_REQ_sum"):
        lat = merged["TCP_TCC_READ_REQ_LATENCY_sum"] / merged["TCP_TCC_READ_REQ_sum"]
    out = [f"# rocprofv3 --pmc counters of {kernel}", "# REPO = repository root"]
    out += [f"# pass {i + 1}: {cmd}" for i, cmd in enumerate(commands)]
    out += [f"kernel: {kernel}",
            f"dispatches per pass: {', '.join(map(str, n_disp))}"
            + (f" (first {first} after skipping {skip})" if first else ""),
            f"mean duration under counters: {sum(durs) / max(1, len(durs)) / 1e3:.1f} us"]
    if clk:
        out.append(f"active clock implied by GRBM_GUI_ACTIVE / 8 / duration: {sum(clk) / len(clk):.2f} GHz")
    out += ["", "counter means per dispatch:"]
    out += [f"  {k:36s} {v:16.4g}" for k, v in sorted(merged.items())]
    if lat is not None:
        out.append(f"  {'L1->L2 read latency (cycles)':36s} {lat:16.1f}")
    if "TCC_HIT_sum" in merged and "TCC_MISS_sum" in merged:
        h, m = merged["TCC_HIT_sum"], merged["TCC_MISS_sum"]
        out.append(f"  {'L2 hit rate':36s} {h / max(1.0, h + m):16.3f}")
    out += ["", "fraction of the kernel's active cycles:"]
    out += [f"  {k:36s} {v:8.3f}" for k, v in sorted(fr.items(), key=lambda kv: -kv[1])]
    busy = {k: v for k, v in fr.items() if "busy" in k or "active" in k}
    if busy:
        top = max(busy, key=busy.get)
        out += ["", f"busiest unit: {top} ({busy[top]:.3f})"]
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    s.add_argument("--top", type=int, default=12)
    s.add_argument("--match", action="append",
                   help="keep only kernels whose name contains this text (repeatable)")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--kernel", default="k_retrieve_mfma")
    t.add_argument("--fetch-command", required=True)
    t.add_argument("--write-command", required=True)
    t.add_argument("--source", default=KERNEL_SRC,
                   help="kernel source file whose SHA-256 the record carries "
                        "(default: the retrieval kernel's)")
    t.add_argument("--first", type=int, default=None,
                   help="average only the first FIRST dispatches after the capacity pass")
    c = sub.add_parser("counters")
    c.add_argument("csvs", nargs="+", help="pmc_counter_collection.csv of each pass")
    c.add_argument("--kernel", required=True)
    c.add_argument("--command", action="append", required=True,
                   help="the command of each pass, in order (repeat per pass)")
    c.add_argument("--first", type=int, default=None)
    c.add_argument("--skip", type=int, default=0)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        sys.stdout.write(stats(a.csv, a.command, a.top, a.match))
    elif a.cmd == "traffic":
        sys.stdout.write(traffic(a.fetch, a.write, a.copy_mib, a.kernel, a.fetch_command,
                                 a.write_command, a.source, a.first))
    else:
        sys.stdout.write(counters(a.csvs, a.kernel, a.command, a.first, a.skip))


if __name__ == "__main__":
    main()
