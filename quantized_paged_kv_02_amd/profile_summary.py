"""Summaries of rocprofv3 output for the decode kernels (host tooling).

Two commands:

  python -m quantized_paged_kv_02_amd.profile_summary stats <dir> --command CMD --out FILE
        [--workload NAME --times-out JSON --split-tokens N]
      Kernel durations from a ``rocprofv3 --kernel-trace --stats
      --output-format csv`` run (the ``*_kernel_trace.csv`` under <dir>):
      calls, mean, median, min and max per kernel, written as markdown,
      and the decode launches bench.py's roofline times (decode kernel,
      partition reduce, their span), also collected per workload in JSON.

  python -m quantized_paged_kv_02_amd.profile_summary traffic <fetch_dir> <write_dir>
        --workload NAME --command-fetch CMD --command-write CMD --out FILE
      HBM bytes per decode launch from two ``rocprofv3 --pmc FETCH_SIZE``
      and ``--pmc WRITE_SIZE`` runs of ``bench.py --copy-probe-mib M``.
      Both counters are in KiB; each is scaled by what it reads for the
      plain device copy of known size in the same run (copyBuffer
      dispatches of the probe's grid), so the figure is in bytes.  The
      decode launch is the decode kernel plus the partition reduce kernel.

  python -m quantized_paged_kv_02_amd.profile_summary crosscheck <dir> --workload NAME
        --command CMD --out FILE
      The launch's read traffic from L2-to-DRAM and L1-to-L2 read-request
      counters of one ``rocprofv3 --pmc`` run, each calibrated on the run's
      device copy: a second figure beside FETCH_SIZE's.

  python -m quantized_paged_kv_02_amd.profile_summary clock <dir> --kernels REGEX
        --command CMD --out FILE
      Effective engine clock per dispatch of the kernels matching REGEX from
      a ``rocprofv3 --pmc GRBM_GUI_ACTIVE`` run: the counter (GPU-active
      cycles, summed over the agent's XCDs) / the XCD count / the dispatch's
      duration, in dispatch order with the idle gap before each.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = [os.path.join(ROOT, "quantized_paged_kv_02_amd", "csrc", f)
                  for f in ("kvq_decode.hip", "kvq_device.h", "kvq_args.h", "kvq_quant.h",
                            "kvq_kivi_write.h")]


def kernel_source_hash() -> str:
    """Hash of the decode kernel sources; traffic figures are valid only for
    the sources they were measured on."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _find(directory: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    return hits[0]


def _short(name: str) -> str:
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    return name if len(name) <= 90 else name[:87] + "..."


def decode_times(rows):
    """Durations (us) of the decode launches that bench.py's roofline times:
    the kvq_paged_decode dispatches (the decode kernel dispatches with the
    smallest grid: a decode step's kvq_write_decode adds flush workgroups
    on KIVI caches) and the partition reduce dispatched right after each,
    plus each such launch's span from the decode's start to the reduce's
    end."""
    rows = sorted(rows, key=lambda r: int(r["Start_Timestamp"]))
    dec = [i for i, r in enumerate(rows) if "paged_decode" in r["Kernel_Name"]]
    if not dec:
        return None
    grid = min(int(rows[i]["Grid_Size_X"]) for i in dec)   # work-items
    wg_size = int(rows[dec[0]].get("Workgroup_Size_X") or 0)
    d_us, m_us, span = [], [], []
    for i in dec:
        r = rows[i]
        if int(r["Grid_Size_X"]) != grid:
            continue
        t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        d_us.append((t1 - t0) / 1000.0)
        nxt = rows[i + 1] if i + 1 < len(rows) else None
        if nxt is not None and "partition_reduce" in nxt["Kernel_Name"]:
            m_us.append((int(nxt["End_Timestamp"]) - int(nxt["Start_Timestamp"])) / 1000.0)
            span.append((int(nxt["End_Timestamp"]) - t0) / 1000.0)
        else:
            span.append((t1 - t0) / 1000.0)
    out = {"decode_us": round(statistics.mean(d_us), 3),
           "decode_median_us": round(statistics.median(d_us), 3),
           "merge_us": round(statistics.mean(m_us), 3) if m_us else 0.0,
           "merge_median_us": round(statistics.median(m_us), 3) if m_us else 0.0,
           "launch_span_us": round(statistics.mean(span), 3),
           "launch_span_median_us": round(statistics.median(span), 3),
           "dispatches": len(d_us), "decode_grid": grid,
           "decode_workgroups": grid // wg_size if wg_size else None}
    return out


def stats(directory: str, command: str, out: str, workload: str | None = None,
          times_out: str | None = None, split_tokens: int | None = None,
          partition: str = "per-row") -> None:
    rows = list(csv.DictReader(open(_find(directory, "kernel_trace.csv"))))
    dt = decode_times(rows)
    per = {}
    for r in rows:
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        per.setdefault(r["Kernel_Name"], []).append(d)
    lines = ["# rocprofv3 kernel trace summary", "",
             f"Command: `{command}`", "",
             "Durations in microseconds (per dispatch).", "",
             "| kernel | calls | mean | median | min | max | total ms |",
             "|---|---|---|---|---|---|---|"]
    for name, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{_short(name)}` | {len(v)} | {statistics.mean(v):.2f} | "
                     f"{statistics.median(v):.2f} | {min(v):.2f} | {max(v):.2f} | "
                     f"{sum(v) / 1000:.3f} |")
    if dt is not None:
        lines += ["", "Decode launches as bench.py's roofline times them (kvq_paged_decode "
                  f"dispatches, grid {dt['decode_grid']} work-items = "
                  f"{dt.get('decode_workgroups')} workgroups, {dt['dispatches']} of "
                  "them): decode kernel mean / median "
                  f"{dt['decode_us']:.2f} / {dt['decode_median_us']:.2f} us, partition "
                  f"reduce after it {dt['merge_us']:.2f} / {dt['merge_median_us']:.2f} us, "
                  "launch span (decode start to reduce end) "
                  f"{dt['launch_span_us']:.2f} / {dt['launch_span_median_us']:.2f} us."]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out}")
    if times_out and workload and dt is not None:
        data = json.load(open(times_out)) if os.path.exists(times_out) else {}
        if data.get("kernel_source_hash") != kernel_source_hash():
            data = {}
        data["kernel_source_hash"] = kernel_source_hash()
        data["note"] = ("rocprofv3 kernel-trace durations (us) of the decode launches bench.py "
                        "times for its roofline (kvq_paged_decode: decode kernel, then the "
                        "partition reduce when the launch is split), per workload")
        data[workload] = {**dt, "split_tokens": split_tokens, "partition": partition,
                          "command": command, "summary": os.path.relpath(out, ROOT)}
        with open(times_out, "w") as f:
            json.dump(data, f, indent=1)
            f.write("\n")
        print(f"wrote {times_out}: {workload} decode {dt['decode_us']} us, merge "
              f"{dt['merge_us']} us")


def _counter(directory: str, counter: str):
    rows = list(csv.DictReader(open(_find(directory, "counter_collection.csv"))))
    return [r for r in rows if r["Counter_Name"] == counter]


def _per_launch(rows, copy_bytes_kib: float):
    # calibration: the largest copyBuffer dispatches are the probe copies
    copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
    probe = max(copies)
    probe_rows = [c for c in copies if c > 0.9 * probe]
    factor = copy_bytes_kib / statistics.median(probe_rows)
    dec = [float(r["Counter_Value"]) for r in rows if "paged_decode" in r["Kernel_Name"]]
    red = [float(r["Counter_Value"]) for r in rows if "partition_reduce" in r["Kernel_Name"]]
    kib = statistics.median(dec) + (statistics.median(red) if red else 0.0)
    return kib * 1024 * factor, factor, len(dec)


def traffic(fetch_dir: str, write_dir: str, workload: str, copy_mib: int, cmd_fetch: str,
            cmd_write: str, out: str, split_tokens: int | None = None,
            partition: str = "per-row") -> None:
    copy_kib = copy_mib * 1024.0
    rd, rf, n_rd = _per_launch(_counter(fetch_dir, "FETCH_SIZE"), copy_kib)
    wr, wf, n_wr = _per_launch(_counter(write_dir, "WRITE_SIZE"), copy_kib)
    data = {}
    if os.path.exists(out):
        data = json.load(open(out))
    if data.get("kernel_source_hash") != kernel_source_hash():
        data = {}
    data["kernel_source_hash"] = kernel_source_hash()
    data["note"] = ("HBM bytes per kvq_paged_decode launch (decode kernel + partition reduce), "
                    "median over dispatches; FETCH_SIZE and WRITE_SIZE (KiB) scaled by what "
                    "they read for a device copy of known size in the same run")
    data[workload] = {
        "bytes_per_launch": int(rd + wr), "read_bytes": int(rd), "write_bytes": int(wr),
        "fetch_scale": round(rf, 4), "write_scale": round(wf, 4),
        "dispatches": [n_rd, n_wr], "command_fetch": cmd_fetch, "command_write": cmd_write,
        "split_tokens": split_tokens, "partition": partition,
    }
    with open(out, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    print(f"wrote {out}: {workload} read {rd / 1e6:.2f} MB write {wr / 1e6:.2f} MB per launch "
          f"(scales {rf:.3f} / {wf:.3f})")


def crosscheck(directory: str, workload: str, copy_mib: int, command: str, out: str,
               counters=("TCC_EA0_RDREQ_DRAM_sum", "TCP_TCC_READ_REQ_sum")) -> None:
    """Read traffic of one decode launch from request counters of other
    blocks than FETCH_SIZE's: L2-to-DRAM read requests and L1-to-L2 read
    requests.  Each is turned into bytes with the bytes per request the
    same counter shows for the run's device copy (its read side: the copy
    reads ``copy_mib`` MiB), and compared with the launch's algorithmic
    bytes and with the FETCH_SIZE figure in decode_traffic.json."""
    copy_bytes = copy_mib * (1 << 20)
    rows_all = list(csv.DictReader(open(_find(directory, "counter_collection.csv"))))
    lines = ["# Decode read traffic from request counters", "",
             f"Command: `{command}`", "",
             f"Workload {workload}.  Each counter is summed over its instances per "
             "dispatch; bytes per request come from the same counter on the run's "
             f"{copy_mib} MiB device copy (copyBuffer; its reads only).  Per launch = decode "
             "kernel + partition reduce, medians over dispatches.", "",
             "| counter | per copy | bytes per request | per launch | bytes per launch |",
             "|---|---|---|---|---|"]
    figures = {}
    for name in counters:
        rows = [r for r in rows_all if r["Counter_Name"] == name]
        if not rows:
            continue
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        big = max(copies)
        per_copy = statistics.median([c for c in copies if c > 0.9 * big])
        bpr = copy_bytes / per_copy
        dec = [float(r["Counter_Value"]) for r in rows if "paged_decode" in r["Kernel_Name"]]
        red = [float(r["Counter_Value"]) for r in rows if "partition_reduce" in r["Kernel_Name"]]
        n = statistics.median(dec) + (statistics.median(red) if red else 0.0)
        figures[name] = n * bpr
        lines.append(f"| {name} | {per_copy:.0f} | {bpr:.2f} | {n:.0f} | {n * bpr / 1e6:.2f} MB |")
    tfile = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if os.path.exists(tfile):
        t = json.load(open(tfile)).get(workload)
        if t:
            lines += ["", f"FETCH_SIZE-derived read bytes per launch (decode_traffic.json): "
                      f"{t['read_bytes'] / 1e6:.2f} MB."]
    lines.append("")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {out}: " + ", ".join(f"{k} {v / 1e6:.2f} MB" for k, v in figures.items()))


def clock(directory: str, kernels: str, command: str, out: str) -> None:
    """Per-dispatch durations and effective clocks (see the module notes)."""
    agents = list(csv.DictReader(open(_find(directory, "agent_info.csv"))))
    gpu = next(a for a in agents if a.get("Name", "").startswith("gfx"))
    xcc = int(gpu["Num_Xcc"])
    peak = float(gpu["Max_Engine_Clk_Fcompute"]) / 1e3
    rows = [r for r in csv.DictReader(open(_find(directory, "counter_collection.csv")))
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE" and re.search(kernels, r["Kernel_Name"])]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    lines = ["# Engine clock per dispatch", "", f"Command: `{command}`", "",
             f"Kernels matching `{kernels}`, in dispatch order.  Clock = GRBM_GUI_ACTIVE "
             f"(summed over the {xcc} XCDs) / {xcc} / duration; the agent's maximum "
             f"engine clock is {peak:.2f} GHz.  Gap: idle time since the previous "
             "listed dispatch ended.", "",
             "| # | kernel | gap us | duration us | clock GHz |", "|---|---|---|---|---|"]
    prev = None
    clocks, durs = [], []
    for i, r in enumerate(rows):
        s0, e0 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        ghz = float(r["Counter_Value"]) / xcc / (e0 - s0)
        gap = (s0 - prev) / 1e3 if prev is not None else 0.0
        prev = e0
        clocks.append(ghz)
        durs.append((e0 - s0) / 1e3)
        lines.append(f"| {i} | `{_short(r['Kernel_Name'])}` | {gap:.1f} | "
                     f"{(e0 - s0) / 1e3:.1f} | {ghz:.3f} |")
    lines.append("")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {out}: {len(rows)} dispatches, clock {min(clocks):.2f} .. {max(clocks):.2f} "
          f"GHz, duration {min(durs):.1f} .. {max(durs):.1f} us")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--workload", default=None)
    s.add_argument("--times-out", default=None,
                   help="JSON file collecting decode / merge durations per workload")
    s.add_argument("--split-tokens", type=int, default=None,
                   help="the partition length the profiled launches used")
    s.add_argument("--partition", default="per-row", choices=["per-row", "balanced"])
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--workload", required=True)
    t.add_argument("--copy-mib", type=int, default=1024)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--split-tokens", type=int, default=None,
                   help="the partition length the profiled launches used")
    t.add_argument("--partition", default="per-row", choices=["per-row", "balanced"])
    c = sub.add_parser("crosscheck")
    c.add_argument("dir")
    c.add_argument("--workload", required=True)
    c.add_argument("--copy-mib", type=int, default=1024)
    c.add_argument("--command", required=True)
    c.add_argument("--out", required=True)
    k = sub.add_parser("clock")
    k.add_argument("dir")
    k.add_argument("--kernels", required=True, help="regular expression on kernel names")
    k.add_argument("--command", required=True)
    k.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "clock":
        clock(a.dir, a.kernels, a.command, a.out)
        return 0
    if a.cmd == "crosscheck":
        crosscheck(a.dir, a.workload, a.copy_mib, a.command, a.out)
        return 0
    if a.cmd == "stats":
        stats(a.dir, a.command, a.out, a.workload, a.times_out, a.split_tokens, a.partition)
    else:
        traffic(a.fetch_dir, a.write_dir, a.workload, a.copy_mib, a.command_fetch,
                a.command_write, a.out, a.split_tokens, a.partition)


if __name__ == "__main__":
    sys.exit(main())
