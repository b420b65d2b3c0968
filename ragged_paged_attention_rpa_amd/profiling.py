"""Summaries of rocprofv3 output for the committed profiles.

Two text products, both computed from the CSV files rocprofv3 writes with
``-f csv``:

* ``trace``: per-kernel call count and mean/min/max duration from a
  ``--kernel-trace --stats`` run (``*_kernel_stats.csv``);
* ``traffic``: HBM bytes per dispatch of one kernel from two ``--pmc`` runs
  (``FETCH_SIZE``, then ``WRITE_SIZE``; both in KiB per dispatch), each scaled
  by the factor that makes the same counter agree with a plain device copy of
  known size (``bench.py --copy-bytes N`` reads N bytes and writes N bytes).
  The result is written as JSON keyed by a hash of the kernel's source, so
  ``bench.py`` reports it only while the kernel is unchanged.

* ``mfma``: matrix-core use of one kernel from one ``--pmc`` run of
  ``SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CYCLES
  GRBM_GUI_ACTIVE``: MFMA-busy share of the SIMD cycles while the kernel ran
  (busy cycles summed over SIMDs / (GPU-active cycles x 1024 SIMDs)) and the
  bf16 MFMA flops executed (MOPS x 512) against the kernel's algorithmic flops.
  rocprofv3's CSV gives GRBM_GUI_ACTIVE summed over the 8 XCDs (its value / 8
  over the dispatch's own start-end span comes out at the shader clock), so
  the active cycles of one XCD are that value / 8.

Usage:
  python -m ragged_paged_attention_rpa_amd.profiling trace STATS_CSV OUT_TXT "TITLE" "COMMAND"
  python -m ragged_paged_attention_rpa_amd.profiling mfma PMC_CSV KERNEL ALGO_FLOPS OUT_TXT \
      "TITLE" "COMMAND"
  python -m ragged_paged_attention_rpa_amd.profiling traffic CONFIG KERNEL \\
      FETCH_CSV WRITE_CSV COPY_FETCH_CSV COPY_WRITE_CSV COPY_BYTES "COMMAND"
"""
from __future__ import annotations

import collections
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _short(name: str, width: int = 72) -> str:
    return name if len(name) <= width else name[: width - 3] + "..."


def trace_summary(stats_csv: str, title: str, command: str) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"# rocprofv3 kernel summary — {title}",
           "# command (run from the repo root):",
           f"#   {command}",
           f"{'kernel':72s} {'calls':>6s} {'mean_us':>10s} {'min_us':>10s} {'max_us':>10s} {'total_us':>11s}"]
    for r in rows:
        out.append(f"{_short(r['Name']):72s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                   f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                   f"{float(r['TotalDurationNs']) / 1e3:11.1f}")
    return "\n".join(out) + "\n"


def counter_per_dispatch(pmc_csv: str, kernel_substr: str, counter: str) -> tuple[float, int]:
    """Mean over dispatches of `counter` (summed over its instances) for the
    kernels whose name contains `kernel_substr`."""
    per = collections.defaultdict(float)
    for r in csv.DictReader(open(pmc_csv)):
        if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
            per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for kernels matching {kernel_substr!r} in {pmc_csv}")
    return sum(per.values()) / len(per), len(per)


def _largest_kernel_value(pmc_csv: str, counter: str) -> float:
    """Counter value of the dispatch with the largest reading (the copy)."""
    per = collections.defaultdict(float)
    for r in csv.DictReader(open(pmc_csv)):
        if r["Counter_Name"] == counter:
            per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    return max(per.values())


def traffic_summary(config, kernel, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv,
                    copy_bytes, command):
    sys.path.insert(0, ROOT)
    from bench import source_sha  # noqa: E402  (hash of the kernel source)

    fetch_kib, nf = counter_per_dispatch(fetch_csv, kernel, "FETCH_SIZE")
    write_kib, nw = counter_per_dispatch(write_csv, kernel, "WRITE_SIZE")
    cf = copy_bytes / (_largest_kernel_value(copy_fetch_csv, "FETCH_SIZE") * 1024.0)
    cw = copy_bytes / (_largest_kernel_value(copy_write_csv, "WRITE_SIZE") * 1024.0)
    fetch_b = fetch_kib * 1024.0 * cf
    write_b = write_kib * 1024.0 * cw
    return {
        "config": config, "kernel": kernel, "kernel_source_sha": source_sha(config),
        "fetch_kib_per_dispatch": fetch_kib, "write_kib_per_dispatch": write_kib,
        "dispatches": [nf, nw],
        "copy_calibration": {"bytes": copy_bytes, "fetch_factor": cf, "write_factor": cw},
        "hbm_fetch_bytes_per_launch": fetch_b, "hbm_write_bytes_per_launch": write_b,
        "hbm_bytes_per_launch": fetch_b + write_b,
        "command": command,
    }


SIMDS = 1024  # 256 CUs x 4 SIMDs on MI355X
XCDS = 8


def _per_dispatch(pmc_csv, kernel_substr, counter, spans=None):
    """{dispatch id: [instance values]} of `counter` for the matching kernels;
    fills `spans` with each dispatch's (start, end) timestamps in ns."""
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(pmc_csv)):
        if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
            per[r["Dispatch_Id"]].append(float(r["Counter_Value"]))
            if spans is not None:
                spans[r["Dispatch_Id"]] = (int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
    if not per:
        raise SystemExit(f"no {counter} rows for kernels matching {kernel_substr!r} in {pmc_csv}")
    return per


def mfma_summary(pmc_csv, kernel, algo_flops, title, command):
    busy = _per_dispatch(pmc_csv, kernel, "SQ_VALU_MFMA_BUSY_CYCLES")
    mops = _per_dispatch(pmc_csv, kernel, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    sqb = _per_dispatch(pmc_csv, kernel, "SQ_BUSY_CYCLES")
    spans = {}
    gui = _per_dispatch(pmc_csv, kernel, "GRBM_GUI_ACTIVE", spans)
    ids = sorted(set(busy) & set(mops) & set(gui), key=lambda x: int(x))
    xcd_cyc = {i: sum(gui[i]) / XCDS for i in ids}
    util = [sum(busy[i]) / (xcd_cyc[i] * SIMDS) for i in ids]
    flops = [sum(mops[i]) * 512 for i in ids]
    out = [f"# rocprofv3 MFMA counters — {title}",
           "# command (run from the repo root):",
           f"#   {command}",
           f"# kernel: {kernel}; dispatches: {len(ids)}",
           "# mfma_busy_pct = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE/8 x 1024 SIMDs); "
           "clock = GRBM_GUI_ACTIVE/8 / dispatch span",
           f"{'dispatch':>9s} {'span_us':>9s} {'clock_GHz':>9s} {'mfma_busy_pct':>14s} "
           f"{'mfma_bf16_flops':>16s} {'exec/algo':>10s} {'sq_busy_cyc':>12s}"]
    for i, u, f in zip(ids, util, flops):
        t0, t1 = spans[i]
        span_ns = max(1, t1 - t0)
        out.append(f"{i:>9s} {span_ns / 1e3:9.1f} {xcd_cyc[i] / span_ns:9.2f} {100 * u:14.1f} "
                   f"{f:16.4e} {f / algo_flops:10.3f} {sum(sqb[i]):12.0f}")
    mu, mf = sum(util) / len(util), sum(flops) / len(flops)
    out.append(f"# mean: MFMA busy {100 * mu:.1f}% of SIMD cycles; executed bf16 MFMA flops "
               f"{mf:.4e} = {mf / algo_flops:.3f} x the algorithmic {algo_flops:.4e}")
    return "\n".join(out) + "\n"


def main(argv):
    if len(argv) >= 5 and argv[0] == "trace":
        stats, out, title, command = argv[1:5]
        open(out, "w").write(trace_summary(stats, title, command))
        return
    if len(argv) >= 9 and argv[0] == "traffic":
        config, kernel, f, w, cf, cw, nbytes, command = argv[1:9]
        d = traffic_summary(config, kernel, f, w, cf, cw, int(nbytes), command)
        out = os.path.join(ROOT, "profiles", f"traffic_{config}.json")
        json.dump(d, open(out, "w"), indent=1)
        print(json.dumps(d))
        return
    if len(argv) >= 7 and argv[0] == "mfma":
        pmc, kernel, flops, out, title, command = argv[1:7]
        text = mfma_summary(pmc, kernel, float(flops), title, command)
        open(out, "w").write(text)
        print(text)
        return
    print(__doc__)
    raise SystemExit(2)


if __name__ == "__main__":
    main(sys.argv[1:])
