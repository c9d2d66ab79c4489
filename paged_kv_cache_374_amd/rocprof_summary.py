"""Summarise rocprofv3 CSV output for the decode kernels.

    python -m paged_kv_cache_374_amd.rocprof_summary --trace DIR [--fetch DIR --write DIR]
        --kernel NAME_SUBSTRING --bytes-per-launch N --command "..." --out profiles/NAME.md
        [--traffic-json profiles/NAME.traffic.json]

--trace: a `rocprofv3 --kernel-trace --stats --output-format csv` output directory
(its *_kernel_stats.csv gives per-kernel call counts and durations).
--fetch / --write: `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` directories.
--pmc-extra (repeatable): further `--pmc` directories; every counter they hold for the
kernel is listed, with LDS bank-conflict share and mean resident waves per CU derived
where their counters are present.
The counters are calibrated with the copy_blocks kernel profiled in the same run
(`bench.py --calibrate` issues it on a known number of bytes): true bytes / counter
reading of that kernel is the factor applied to the decode kernel's readings.

The traffic record stores a hash of the kernel sources it was measured on; bench.py
reports it only while the sources are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("csrc/attn_mfma.hip", "csrc/attn_generic.hip", "csrc/cache_ops.hip",
                  "csrc/plan.cpp", "csrc/plan.h", "csrc/capi.hip", "csrc/device_common.h",
                  "csrc/read_probe.hip")
CALIBRATION_KERNEL = "copy_blocks_kernel"


def sources_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _one(pattern: str) -> str:
    """The newest file matching `pattern` (an output folder may hold several runs)."""
    hits = glob.glob(pattern, recursive=True)
    if not hits:
        raise FileNotFoundError(pattern)
    return max(hits, key=os.path.getmtime)


def kernel_stats(trace_dir: str):
    path = _one(os.path.join(trace_dir, "**", "*kernel_stats.csv"))
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append({"name": r["Name"], "calls": int(r["Calls"]),
                         "avg_us": float(r["AverageNs"]) / 1e3,
                         "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3,
                         "pct": float(r["Percentage"])})
    return path, rows


def counter_means(pmc_dir: str, counter: str, calibration: str = CALIBRATION_KERNEL):
    """Mean counter value (KiB as rocprofv3 reports it) per kernel name. For the
    calibration kernel only the dispatches within half of its largest reading count:
    a workload may run the same kernel on far fewer bytes (copy-on-write copies), and
    the calibration call is the one of known size."""
    path = _one(os.path.join(pmc_dir, "**", "*counter_collection.csv"))
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    out = {}
    for k, v in per.items():
        if calibration in k:
            v = [x for x in v if x >= 0.5 * max(v)]
        out[k] = statistics.mean(v)
    return path, out


def all_counter_means(pmc_dir: str, needle: str):
    """Mean value per dispatch of every counter collected for the kernel matching
    `needle`, plus the agent's CU and XCC counts and wave slots per CU."""
    path = _one(os.path.join(pmc_dir, "**", "*counter_collection.csv"))
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if needle in r["Kernel_Name"]:
                per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    agent = {}
    with open(_one(os.path.join(pmc_dir, "**", "*agent_info.csv"))) as f:
        for r in csv.DictReader(f):
            if r.get("Cu_Count", "0") not in ("", "0"):
                agent = {"cus": int(r["Cu_Count"]), "xcc": int(r["Num_Xcc"]),
                         "slots": int(r["Max_Waves_Per_Cu"])}
    return path, {k: statistics.mean(v) for k, v in per.items()}, agent


def derived_rows(c, agent):
    """Readings derived from the SQ/GRBM counters, where present. SQ_WAVE_CYCLES counts
    in units of four cycles; GRBM_GUI_ACTIVE comes summed over the XCCs."""
    out = []
    if "SQ_LDS_BANK_CONFLICT" in c and c.get("SQ_LDS_IDX_ACTIVE"):
        out.append(("LDS bank-conflict cycles / LDS active cycles",
                    f"{100 * c['SQ_LDS_BANK_CONFLICT'] / c['SQ_LDS_IDX_ACTIVE']:.1f}%"))
    if "SQ_WAVE_CYCLES" in c and c.get("GRBM_GUI_ACTIVE") and agent:
        gui = c["GRBM_GUI_ACTIVE"] / agent["xcc"]
        waves = 4 * c["SQ_WAVE_CYCLES"] / gui / agent["cus"]
        out.append(("mean resident waves per CU over the kernel",
                    f"{waves:.2f} of {agent['slots']} ({100 * waves / agent['slots']:.1f}%)"))
    if "SQ_INSTS_VALU" in c and c.get("SQ_WAVES"):
        out.append(("VALU instructions per wave", f"{c['SQ_INSTS_VALU'] / c['SQ_WAVES']:.0f}"))
    if "SQ_INSTS_MFMA" in c and c.get("SQ_WAVES"):
        out.append(("MFMA instructions per wave", f"{c['SQ_INSTS_MFMA'] / c['SQ_WAVES']:.0f}"))
    return out


def pick(names, needle):
    hits = [n for n in names if needle in n]
    if not hits:
        raise KeyError(f"no kernel matching {needle!r}")
    return hits[0]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--kernel", required=True, help="substring of the dominant kernel's name")
    ap.add_argument("--bytes-per-launch", type=float, required=True,
                    help="algorithmic bytes one launch of that kernel moves")
    ap.add_argument("--calib-read-bytes", type=float, default=0.0)
    ap.add_argument("--calib-write-bytes", type=float, default=0.0)
    ap.add_argument("--command", required=True, help="command line that produced the trace")
    ap.add_argument("--pmc-command", default="")
    ap.add_argument("--out", required=True)
    ap.add_argument("--traffic-json")
    ap.add_argument("--pmc-extra", action="append", default=[],
                    help="further `rocprofv3 --pmc` output directories (LDS, occupancy, ...)")
    ap.add_argument("--pmc-extra-command", default="")
    args = ap.parse_args()

    tpath, rows = kernel_stats(args.trace)
    dom = [r for r in rows if args.kernel in r["name"]]
    if not dom:
        raise SystemExit(f"kernel {args.kernel!r} not in {tpath}")
    d = dom[0]
    achieved = args.bytes_per_launch / (d["avg_us"] * 1e-6) / 1e9
    lines = [f"# rocprofv3 summary: {args.kernel}", "",
             f"Command: `{args.command}`", "",
             f"Trace file: `{os.path.basename(tpath)}`", "",
             f"Source hash (kernel sources): `{sources_sha()}`", "",
             "| kernel | calls | avg us | min us | max us | % of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in rows[:8]:
        name = r["name"] if len(r["name"]) < 90 else r["name"][:87] + "..."
        lines.append(f"| `{name}` | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | "
                     f"{r['max_us']:.2f} | {r['pct']:.1f} |")
    lines += ["", f"Dominant kernel average: {d['avg_us']:.2f} us; algorithmic bytes per launch "
              f"{args.bytes_per_launch:.0f} -> {achieved:.0f} GB/s "
              f"({100 * achieved / 8000:.1f}% of 8 TB/s)."]
    traffic = None
    if args.fetch and args.write:
        fpath, fetch = counter_means(args.fetch, "FETCH_SIZE")
        wpath, write = counter_means(args.write, "WRITE_SIZE")
        kf, kw = pick(fetch, args.kernel), pick(write, args.kernel)
        cf, cw = pick(fetch, CALIBRATION_KERNEL), pick(write, CALIBRATION_KERNEL)
        f_factor = args.calib_read_bytes / (fetch[cf] * 1024.0)
        w_factor = args.calib_write_bytes / (write[cw] * 1024.0)
        fb = fetch[kf] * 1024.0 * f_factor
        wb = write[kw] * 1024.0 * w_factor
        traffic = fb + wb
        lines += ["", f"PMC command: `{args.pmc_command}`", "",
                  f"Counter files: `{os.path.basename(fpath)}`, `{os.path.basename(wpath)}`", "",
                  "| counter | calibration kernel reading (KiB) | true bytes | factor | "
                  "decode reading (KiB) | decode bytes/launch |", "|---|---|---|---|---|---|",
                  f"| FETCH_SIZE | {fetch[cf]:.0f} | {args.calib_read_bytes:.0f} | "
                  f"{f_factor:.3f} | {fetch[kf]:.0f} | {fb:.0f} |",
                  f"| WRITE_SIZE | {write[cw]:.0f} | {args.calib_write_bytes:.0f} | "
                  f"{w_factor:.3f} | {write[kw]:.0f} | {wb:.0f} |", "",
                  f"HBM traffic per launch {traffic:.0f} B = "
                  f"{traffic / args.bytes_per_launch:.3f} x the algorithmic bytes."]
    if args.pmc_extra:
        lines += ["", f"Further counter passes: `{args.pmc_extra_command}`", "",
                  "| counter | mean per dispatch of the kernel |", "|---|---|"]
        merged, agent = {}, {}
        for d_ in args.pmc_extra:
            _, c, ag = all_counter_means(d_, args.kernel)
            merged.update(c)
            agent = agent or ag
        for k in sorted(merged):
            lines.append(f"| {k} | {merged[k]:.0f} |")
        rows_d = derived_rows(merged, agent)
        if rows_d:
            lines += ["", "| derived | value |", "|---|---|"]
            lines += [f"| {k} | {v} |" for k, v in rows_d]
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    if args.traffic_json and traffic is not None:
        with open(args.traffic_json, "w") as f:
            json.dump({"kernel": args.kernel, "source_sha": sources_sha(),
                       "traffic_bytes_per_launch": traffic,
                       "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
                       "algorithmic_bytes_per_launch": args.bytes_per_launch,
                       "avg_us": d["avg_us"]}, f, indent=1)
    print("\n".join(lines))


if __name__ == "__main__":
    main()
