"""Short text summaries of rocprofv3 output for the profiles/ folder.

    python -m cross_model_sparse_amd.profile_summary stats STATS_CSV --command CMD [--match TEXT ...]
        per-kernel call count and average / total duration from a
        `rocprofv3 --kernel-trace --stats` run (run_kernel_stats.csv),
        optionally only for kernels whose names contain one of the TEXTs

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


def _reference_window(rows):
    """(lo, hi): bench.py --copy-ref-mib runs the copy reference after the
    capacity pass and before the first timed step, so it lies strictly between
    the capacity pass's last gather (lo) and the step's first block-mass
    launches (hi: the last block-mass dispatch before the step's first
    retrieval launch)."""
    first = next(i for i, r in enumerate(rows) if "k_retrieve_mfma" in r[1])
    hi = max(i for i in range(first) if "k_block_mass" in rows[i][1])
    lo = max(i for i in range(hi) if "k_gather" in rows[i][1])
    return lo, hi


def _copy_reference(rows, mib: int):
    """Counter value of the copy reference: the median of the elementwise
    dispatches in the reference window (the fill that creates the source reads
    nothing and is skipped by the > 1/4 size test in the fetch run)."""
    want = mib * 1024.0
    lo, hi = _reference_window(rows)
    vals = [v for _, name, v in rows[lo + 1:hi]
            if "elementwise" in name and v > 0.25 * want]
    if not vals:
        raise SystemExit("no copy-reference dispatch found in the counter file")
    vals.sort()
    return vals[len(vals) // 2]


def _kernel_mean(rows, kernel: str):
    """Mean counter value (KiB) and count of `kernel`'s dispatches after the
    capacity pass (the timed steps' launches)."""
    lo, _ = _reference_window(rows)
    vals = [v for _, name, v in rows[lo + 1:] if kernel in name]
    if not vals:
        raise SystemExit(f"no dispatch of {kernel} after the capacity pass")
    return sum(vals) / len(vals), len(vals)


def traffic(fetch_csv, write_csv, mib, kernel, fetch_cmd, write_cmd, source=KERNEL_SRC) -> str:
    fetch = _dispatches(fetch_csv, "FETCH_SIZE")
    write = _dispatches(write_csv, "WRITE_SIZE")
    want = mib * 1024.0
    f_ref = _copy_reference(fetch, mib)
    w_ref = _copy_reference(write, mib)
    f_scale = want / f_ref
    w_scale = want / w_ref
    f_kib, nf = _kernel_mean(fetch, kernel)
    w_kib, nw = _kernel_mean(write, kernel)
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
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        sys.stdout.write(stats(a.csv, a.command, a.top, a.match))
    else:
        sys.stdout.write(traffic(a.fetch, a.write, a.copy_mib, a.kernel, a.fetch_command,
                                 a.write_command, a.source))


if __name__ == "__main__":
    main()
