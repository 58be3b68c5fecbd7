"""Turn rocprofv3 CSV output into the short text summaries kept in profiles/.

    python -m paged_kv_cache_157_amd.rocprof_summary stats  <kernel_stats.csv> <out.md> <command>
    python -m paged_kv_cache_157_amd.rocprof_summary traffic <fetch_dir> <write_dir> <workload> <out.md> <command...>

`traffic` reads two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of
`bench.py --copy-probe-mib N` (a plain N-MiB device copy is the last large
copy dispatch), derives the counter-to-byte factors from that copy, scales the
decode kernels' per-dispatch counters, and records bytes per decode launch in
profiles/traffic.json together with a hash of the decode source, so the bench
reports the figure only while the kernel is unchanged.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def decode_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("decode.hip", "decode_hg.h", "decode_hg4.hip", "pa_device.h"):
        h.update(open(os.path.join(HERE, "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    return name.split("(")[0].replace("void ", "")[:70]


def stats(csv_path: str, out_md: str, command: str) -> None:
    rows = list(csv.DictReader(open(csv_path)))
    lines = [f"# rocprofv3 kernel statistics", "", f"Command: `{command}`", "",
             "| kernel | calls | avg µs | min µs | max µs | % time |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | "
                     f"{float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_rows(d: str):
    f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not f:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    return list(csv.DictReader(open(f[0])))


def traffic(fetch_dir: str, write_dir: str, workload: str, out_md: str, command: str) -> None:
    res = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d)
        copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"]]
        probe = max(copies, key=lambda r: int(r["Dispatch_Id"]))  # the last copy is the probe
        per = defaultdict(list)
        for r in rows:
            if "pa::" in r["Kernel_Name"]:
                per[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
        res[name] = dict(probe_kib=float(probe["Counter_Value"]),
                         per_kernel={k: sum(v) / len(v) for k, v in per.items()})
    probe_mib = 1024
    factor = {k: probe_mib * 1024.0 / v["probe_kib"] for k, v in res.items()}
    dec = [k for k in res["FETCH_SIZE"]["per_kernel"] if "decode" in k]
    fetch_b = sum(res["FETCH_SIZE"]["per_kernel"][k] for k in dec) * 1024 * factor["FETCH_SIZE"]
    write_b = sum(res["WRITE_SIZE"]["per_kernel"][k] for k in dec) * 1024 * factor["WRITE_SIZE"]
    rec = dict(bytes_per_launch=int(fetch_b + write_b), fetch_bytes=int(fetch_b),
               write_bytes=int(write_b), factors=factor, kernels=dec,
               source_hash=decode_source_hash())
    data = json.load(open(TRAFFIC_JSON)) if os.path.exists(TRAFFIC_JSON) else {}
    data[workload] = rec
    json.dump(data, open(TRAFFIC_JSON, "w"), indent=1, sort_keys=True)
    lines = [f"# HBM traffic of the decode launch ({workload})", "",
             f"Command (one run per counter): `{command}`", "",
             f"Reference: a plain {probe_mib} MiB device copy reads FETCH_SIZE = "
             f"{res['FETCH_SIZE']['probe_kib']:.1f} KiB and WRITE_SIZE = "
             f"{res['WRITE_SIZE']['probe_kib']:.1f} KiB; byte factors "
             f"{factor['FETCH_SIZE']:.4f} (fetch) and {factor['WRITE_SIZE']:.4f} (write).", "",
             "| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch |", "|---|---|---|"]
    for k in res["FETCH_SIZE"]["per_kernel"]:
        lines.append(f"| {k} | {res['FETCH_SIZE']['per_kernel'][k]:.1f} | "
                     f"{res['WRITE_SIZE']['per_kernel'].get(k, float('nan')):.1f} |")
    lines += ["", f"Decode launch (all decode kernels): fetched {fetch_b/1e6:.2f} MB, written "
                  f"{write_b/1e6:.2f} MB, total {(fetch_b+write_b)/1e6:.2f} MB per launch.",
              f"Decode source hash: {rec['source_hash']}"]
    open(out_md, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "stats":
        stats(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]))
    elif mode == "traffic":
        traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], " ".join(sys.argv[6:]))
    else:
        raise SystemExit(__doc__)
