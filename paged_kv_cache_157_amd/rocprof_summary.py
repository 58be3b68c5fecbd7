"""Turn rocprofv3 CSV output into the short text summaries kept in profiles/.

    python -m paged_kv_cache_157_amd.rocprof_summary stats <out_dir> <out.md> <command...>
    python -m paged_kv_cache_157_amd.rocprof_summary traffic <rd_dir> <wr_dir> <workload> <out.md> <command...>
    python -m paged_kv_cache_157_amd.rocprof_summary line <out.md> <title> <json_file>... -- <command...>

`stats` reads the kernel statistics and the kernel trace of one
`rocprofv3 --kernel-trace --stats` run.  Besides the per-kernel table it
splits the launches of each decode kernel by what ran just before them on
the GPU: a launch that follows the 768 MiB eviction read of bench.py's cold
leg (a reduction kernel) ran with the Infinity Cache evicted ("cold"), any
other one back to back with decode and cache-write launches ("warm").

`traffic` reads two `rocprofv3 --pmc` runs of `bench.py --copy-probe-mib N`:
  1. TCC_EA0_RDREQ, TCC_EA0_RDREQ_32B, TCC_EA0_RDREQ_64B, TCC_EA0_RDREQ_128B
     (read requests from the L2 to memory, by size);
  2. TCC_BUBBLE, TCC_EA0_WRREQ, TCC_EA0_WRREQ_64B (128-byte reads as the
     FETCH_SIZE formula counts them; write requests, 64-byte ones apart).
Read bytes = 32 n32 + 64 n64 + 128 n128; write bytes = 64 n64w + 32 (nw -
n64w).  The plain N-MiB device copy (the last large copy dispatch) checks
both against its known size, and the FETCH_SIZE formula's value is shown
beside them.  Bytes per decode launch go to profiles/traffic.json together
with a hash of the decode source, so bench.py reports the figure only while
the kernel is unchanged.

`line` keeps bench.py result lines (the last JSON line of each file) as a
short markdown summary with the command that printed them: the scalar fields
of each line, and those of its nested records, one table per line.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import statistics
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def decode_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("decode.hip", "decode_common.h", "decode_hg.h", "decode_hg4.hip", "pa_device.h"):
        p = os.path.join(HERE, "csrc", f)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    return name.split("(")[0].replace("void ", "")[:70]


def _find(d: str, suffix: str) -> str:
    f = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not f:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return f[0]


def stats(out_dir: str, out_md: str, command: str) -> None:
    rows = list(csv.DictReader(open(_find(out_dir, "kernel_stats.csv"))))
    lines = ["# rocprofv3 kernel statistics", "", f"Command: `{command}`", "",
             "| kernel | calls | avg µs | min µs | max µs | % time |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | "
                     f"{float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} |")
    try:
        trace = list(csv.DictReader(open(_find(out_dir, "kernel_trace.csv"))))
    except FileNotFoundError:
        trace = []
    if trace:
        trace.sort(key=lambda r: int(r["Start_Timestamp"]))
        groups = defaultdict(lambda: {"warm": [], "cold": []})
        prev = ""
        for r in trace:
            name = r["Kernel_Name"]
            if "decode" in name and "pa::" in name:
                # the eviction read is torch's sum: at::native::reduce_kernel
                kind = "cold" if "at::native" in prev and "reduce_kernel" in prev else "warm"
                groups[_short(name)][kind].append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            prev = name
        lines += ["", "Decode launches split by what ran just before them (kernel trace): "
                      "\"cold\" = right after the 768 MiB eviction read, \"warm\" = otherwise "
                      "(back to back with decode or cache-write launches).", "",
                  "| kernel | kind | launches | avg µs | median µs | min µs |", "|---|---|---|---|---|---|"]
        for k, g in groups.items():
            for kind in ("warm", "cold"):
                v = g[kind]
                if v:
                    lines.append(f"| {k} | {kind} | {len(v)} | {sum(v)/len(v):.2f} | "
                                 f"{statistics.median(v):.2f} | {min(v):.2f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_rows(d: str):
    return list(csv.DictReader(open(_find(d, "counter_collection.csv"))))


def _per_dispatch(rows):
    """{dispatch id: (kernel name, {counter: value})}"""
    out = {}
    for r in rows:
        did = int(r["Dispatch_Id"])
        name, vals = out.setdefault(did, (r["Kernel_Name"], {}))
        vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def traffic(rd_dir: str, wr_dir: str, workload: str, out_md: str, command: str) -> None:
    disp = {}
    for d in (rd_dir, wr_dir):
        for did, (name, vals) in _per_dispatch(_counter_rows(d)).items():
            disp.setdefault((d, did), (name, vals))

    def reads(v):
        return 32 * v["TCC_EA0_RDREQ_32B"] + 64 * v["TCC_EA0_RDREQ_64B"] + 128 * v["TCC_EA0_RDREQ_128B"]

    def writes(v):
        return 64 * v["TCC_EA0_WRREQ_64B"] + 32 * (v["TCC_EA0_WRREQ"] - v["TCC_EA0_WRREQ_64B"])

    res = {}
    for d, f in ((rd_dir, "read"), (wr_dir, "write")):
        mine = {did: nv for (dd, did), nv in disp.items() if dd == d}
        copies = [(did, nv) for did, nv in mine.items() if "copyBuffer" in nv[0]]
        probe = max(copies)[1][1]  # the last copy dispatch is the probe
        per = defaultdict(list)
        for did, (name, vals) in mine.items():
            if "pa::" in name:
                per[_short(name)].append(vals)
        res[f] = dict(probe=probe, per=per)
    probe_mib = 1024
    probe_bytes = probe_mib << 20
    rp = res["read"]["probe"]
    wp = res["write"]["probe"]
    probe_read = reads(rp)
    probe_write = writes(wp)
    dec = [k for k in res["read"]["per"] if "decode" in k]

    def mean(xs):
        return sum(xs) / len(xs)

    rd_b = sum(mean([reads(v) for v in res["read"]["per"][k]]) for k in dec)
    wr_b = sum(mean([writes(v) for v in res["write"]["per"][k]]) for k in dec)
    n128 = sum(mean([v["TCC_EA0_RDREQ_128B"] for v in res["read"]["per"][k]]) for k in dec)
    nrd = sum(mean([v["TCC_EA0_RDREQ"] for v in res["read"]["per"][k]]) for k in dec)
    bub = sum(mean([v["TCC_BUBBLE"] for v in res["write"]["per"][k]]) for k in dec)
    n32 = sum(mean([v["TCC_EA0_RDREQ_32B"] for v in res["read"]["per"][k]]) for k in dec)
    # the FETCH_SIZE formula of the counter list: a 128-byte request counts as
    # such only when TCC_BUBBLE sees it, every other non-32-byte one as 64 bytes
    fetch_formula = bub * 128 + (nrd - bub - n32) * 64 + n32 * 32
    rec = dict(bytes_per_launch=int(rd_b + wr_b), read_bytes=int(rd_b), write_bytes=int(wr_b),
               method="read = 32 n32 + 64 n64 + 128 n128 (TCC_EA0_RDREQ_*B); "
                      "write = 64 n64 + 32 (n - n64) (TCC_EA0_WRREQ, TCC_EA0_WRREQ_64B)",
               probe_check=dict(copy_bytes=probe_bytes, read_counted=int(probe_read),
                                write_counted=int(probe_write)),
               fetch_size_formula_bytes=int(fetch_formula),
               kernels=dec, source_hash=decode_source_hash())
    data = json.load(open(TRAFFIC_JSON)) if os.path.exists(TRAFFIC_JSON) else {}
    data[workload] = rec
    json.dump(data, open(TRAFFIC_JSON, "w"), indent=1, sort_keys=True)
    lines = [f"# HBM traffic of the decode launch ({workload})", "",
             f"Command (one run per counter set): `{command}`", "",
             "Read bytes from the L2-to-memory read requests by size: 32 x TCC_EA0_RDREQ_32B + "
             "64 x TCC_EA0_RDREQ_64B + 128 x TCC_EA0_RDREQ_128B; write bytes from "
             "64 x TCC_EA0_WRREQ_64B + 32 x (TCC_EA0_WRREQ - TCC_EA0_WRREQ_64B).", "",
             f"Check on a plain {probe_mib} MiB device copy ({probe_bytes} bytes each way): reads "
             f"counted {probe_read:.0f} bytes ({probe_read / probe_bytes:.4f} of the copy), writes "
             f"{probe_write:.0f} ({probe_write / probe_bytes:.4f}); its read requests: "
             f"{rp['TCC_EA0_RDREQ']:.0f} in all, {rp['TCC_EA0_RDREQ_128B']:.0f} of 128 B, "
             f"{rp['TCC_EA0_RDREQ_64B']:.0f} of 64 B, {rp['TCC_EA0_RDREQ_32B']:.0f} of 32 B.", "",
             "| kernel | read MB/dispatch | write MB/dispatch | 128 B reads | all reads | TCC_BUBBLE |",
             "|---|---|---|---|---|---|"]
    for k in res["read"]["per"]:
        rv = res["read"]["per"][k]
        wv = res["write"]["per"].get(k, [])
        lines.append(f"| {k} | {mean([reads(v) for v in rv]) / 1e6:.2f} | "
                     f"{(mean([writes(v) for v in wv]) / 1e6) if wv else float('nan'):.2f} | "
                     f"{mean([v['TCC_EA0_RDREQ_128B'] for v in rv]):.0f} | "
                     f"{mean([v['TCC_EA0_RDREQ'] for v in rv]):.0f} | "
                     f"{(mean([v['TCC_BUBBLE'] for v in wv])) if wv else float('nan'):.0f} |")
    lines += ["", f"Decode launch (all decode kernels): read {rd_b/1e6:.2f} MB, written "
                  f"{wr_b/1e6:.2f} MB, total {(rd_b+wr_b)/1e6:.2f} MB per launch; "
                  f"128-byte read requests {n128:.0f} of {nrd:.0f}, TCC_BUBBLE {bub:.0f}.",
              f"The FETCH_SIZE formula (TCC_BUBBLE x 128 + other non-32-byte requests x 64 + "
              f"32-byte ones x 32) gives {fetch_formula/1e6:.2f} MB for the same reads, "
              f"{fetch_formula / rd_b if rd_b else float('nan'):.3f} of the request-size count.",
              f"Decode source hash: {rec['source_hash']}"]
    open(out_md, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _flat(rec: dict, prefix: str = "") -> list:
    rows = []
    for k, v in rec.items():
        if isinstance(v, dict):
            rows += _flat(v, f"{prefix}{k}.")
        elif isinstance(v, list):
            rows.append((prefix + k, json.dumps(v)))
        else:
            rows.append((prefix + k, v))
    return rows


def line(out_md: str, title: str, files: list, command: str) -> None:
    out = [f"# {title}", "", f"Command: `{command}`", ""]
    for f in files:
        rec = json.loads(open(f).read().strip().splitlines()[-1])
        out += [f"## {rec.get('config', {}).get('workload', rec.get('metric', f))}", "",
                "| field | value |", "|---|---|"]
        out += [f"| {k} | {v} |" for k, v in _flat(rec)]
        out.append("")
    open(out_md, "w").write("\n".join(out))
    print(f"wrote {out_md}")


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "stats":
        stats(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]))
    elif mode == "traffic":
        traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], " ".join(sys.argv[6:]))
    elif mode == "line":
        sep = sys.argv.index("--")
        line(sys.argv[2], sys.argv[3], sys.argv[4:sep], " ".join(sys.argv[sep + 1:]))
    else:
        raise SystemExit(__doc__)
