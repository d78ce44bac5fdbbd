"""Summarise rocprofv3 CSV output into the short Markdown files kept under profiles/.

    python -m sparse_top_kv_head_amd.prof_summary stats <dir> "<command>" <out.md> "<title>"
    python -m sparse_top_kv_head_amd.prof_summary traffic <fetch_dir> <write_dir> "<cmd1>||<cmd2>" <out.md> "<title>" [--no-scan-line]
    python -m sparse_top_kv_head_amd.prof_summary counters <dir> "<command>" <out.md> "<title>"

``stats`` reads ``run_kernel_stats.csv`` of a ``--kernel-trace --stats`` run.
``traffic`` reads the ``run_counter_collection.csv`` of one FETCH_SIZE and one
WRITE_SIZE run of ``bench.py --calibrate-copy`` and scales each counter by what
it reads for the plain 256 MiB device copies of that run (the last three copy
dispatches; bytes moved per KiB counted), giving HBM bytes per dispatch. The scan kernel's figure is written
with a hash of its sources, so that ``bench.py`` uses it only while the kernel
is unchanged. ``counters`` tabulates every counter of a ``--pmc`` run per kernel
(mean over dispatches).
"""

from __future__ import annotations

import collections
import csv
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SCAN_SOURCES = ["sparse_top_kv_head_amd/csrc/score.hip", "sparse_top_kv_head_amd/csrc/prhs_device.hpp",
                "sparse_top_kv_head_amd/csrc/prhs_launch.hpp"]
COPY_KERNEL = "__amd_rocclr_copyBuffer"
CALIBRATION_KIB = 256 * 1024


def source_hash(files=SCAN_SOURCES):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def short_name(name):
    for p in ("prhs::(anonymous namespace)::", "at::native::(anonymous namespace)::", "void "):
        name = name.replace(p, "")
    return name.split("(")[0]


def _ours(name):
    return "prhs" in name or "stream_read" in name


def stats(statsdir, cmd, out, title):
    rows = list(csv.DictReader(open(os.path.join(statsdir, "run_kernel_stats.csv"))))
    lines = [f"# {title}\n",
             "Command (repository root, MI355X, one GPU; `cd /tmp && export TMPDIR=/tmp` first):\n",
             "```", cmd, "```\n",
             "Kernel statistics over the whole run (warm-up, eager steps, graph-replayed steps and the "
             "separate scan loop; this library's kernels first). Durations in microseconds.\n",
             "| kernel | calls | mean | min | max |", "|---|---|---|---|---|"]
    rows.sort(key=lambda r: (0 if _ours(r["Name"]) else 1, -float(r["TotalDurationNs"])))
    for r in rows:
        if not _ours(r["Name"]) and float(r["TotalDurationNs"]) < 1e5:
            continue
        lines.append(f"| `{short_name(r['Name'])[:80]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def _counter_means(d, ours=None):
    """Counter values per kernel (short name) and counter; `ours` collects the
    short names of this library's kernels."""
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
        k = short_name(r["Kernel_Name"])
        agg[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        if ours is not None and _ours(r["Kernel_Name"]):
            ours.add(k)
    return agg


def _calibration_copy(d, counter, n=3):
    """Mean counter value of the calibration copies: the last n copy dispatches of
    the run (bench.py --calibrate-copy issues them after all other GPU work)."""
    rows = [r for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv")))
            if short_name(r["Kernel_Name"]) == COPY_KERNEL and r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    last = rows[-n:]
    return sum(float(r["Counter_Value"]) for r in last) / len(last)


def traffic(fetch_dir, write_dir, cmds, out, title, scan_line=True):
    ours = set()
    f = _counter_means(fetch_dir, ours)
    w = _counter_means(write_dir)
    copy_f = _calibration_copy(fetch_dir, "FETCH_SIZE")
    copy_w = _calibration_copy(write_dir, "WRITE_SIZE")
    ff, fw = CALIBRATION_KIB / copy_f, CALIBRATION_KIB / copy_w
    lines = [f"# {title}\n", "Commands (repository root, MI355X, one GPU; each counter in its own run):\n",
             "```"] + cmds + ["```\n",
             f"Calibration: a plain device copy of 256 MiB (`--calibrate-copy`, torch `copy_`, dispatched as "
             f"`{COPY_KERNEL}`) reads FETCH_SIZE = {copy_f:.1f} KiB and WRITE_SIZE = {copy_w:.1f} KiB per "
             f"dispatch, so the scale factors to bytes moved are fetch x{ff:.4f}, write x{fw:.4f}.\n",
             (f"Scan kernel sources hash (sha256 of {', '.join(SCAN_SOURCES)}, first 16 hex): "
              f"`{source_hash()}`\n" if scan_line else ""),
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled fetch MiB | scaled write MiB |",
             "|---|---|---|---|---|---|"]
    per = {}
    for k in sorted(f):
        if k not in ours:
            continue
        fv = f[k]["FETCH_SIZE"]
        wv = w.get(k, {}).get("WRITE_SIZE", [0.0])
        fm, wm = sum(fv) / len(fv), sum(wv) / len(wv)
        lines.append(f"| `{k[:70]}` | {len(fv)} | {fm:.1f} | {wm:.1f} | {fm * ff / 1024:.2f} | {wm * fw / 1024:.2f} |")
        per[k] = fm * ff * 1024 + wm * fw * 1024
    if scan_line:
        scan = [k for k in per if "score_scan" in k][0]
        lines.append(f"\nscan_traffic_bytes_per_launch: {per[scan]:.0f}")
        lines.append(f"scan_source_hash: {source_hash()}")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


# MI355X: 32 shader engines (8 XCDs x 4) of 8 CUs, 4 SIMDs per CU.
SIMDS_PER_SE = 32


def counters(d, cmd, out, title):
    ours = set()
    agg = _counter_means(d, ours)
    names = sorted({c for k in agg for c in agg[k]})
    occ = "SQ_WAVE_CYCLES" in names and "SQ_BUSY_CYCLES" in names
    lines = [f"# {title}\n", "Command (repository root, MI355X, one GPU):\n", "```", cmd, "```\n",
             "Mean counter value per dispatch."]
    if occ:
        lines.append(
            "waves/SIMD (achieved occupancy, estimated) = 4 * SQ_WAVE_CYCLES / SQ_BUSY_CYCLES / "
            f"{SIMDS_PER_SE}: SQ_WAVE_CYCLES counts resident waves in 4-cycle units and "
            "SQ_BUSY_CYCLES is summed over the 32 shader engines of 32 SIMDs each. As a check, "
            "the plain streaming read (limit 8 waves/SIMD) comes out near 7.5, and the select "
            "kernel (one 16-wave workgroup per CU on half of the CUs) near 2.")
    lines += ["", "| kernel | dispatches | " + " | ".join(names) + (" | waves/SIMD |" if occ else " |"),
              "|---|---|" + "---|" * (len(names) + (1 if occ else 0))]
    for k in sorted(agg):
        if k not in ours and COPY_KERNEL not in k:
            continue
        n = max(len(v) for v in agg[k].values())
        mean = {c: sum(agg[k][c]) / len(agg[k][c]) for c in names if agg[k].get(c)}
        vals = [f"{mean[c]:.4g}" if c in mean else "" for c in names]
        if occ:
            b = mean.get("SQ_BUSY_CYCLES", 0.0)
            vals.append(f"{4 * mean.get('SQ_WAVE_CYCLES', 0.0) / b / SIMDS_PER_SE:.2f}" if b else "")
        lines.append(f"| `{k[:60]}` | {n} | " + " | ".join(vals) + " |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    what = sys.argv[1]
    if what == "stats":
        stats(*sys.argv[2:6])
    elif what == "traffic":
        traffic(sys.argv[2], sys.argv[3], sys.argv[4].split("||"), sys.argv[5], sys.argv[6],
                scan_line=not (len(sys.argv) > 7 and sys.argv[7] == "--no-scan-line"))
    elif what == "counters":
        counters(*sys.argv[2:6])
    else:
        raise SystemExit(__doc__)
