"""Turn rocprofv3 CSV output into the short summaries kept under profiles/.

    python3 -m lsh_sparse_attention_hash_amd.rocprof_summary trace \
        --stats <dir>/<name>_kernel_stats.csv --workload long --command "..."
    python3 -m lsh_sparse_attention_hash_amd.rocprof_summary traffic \
        --fetch <fetch>_counter_collection.csv --write <write>_counter_collection.csv \
        --workload long --command "..."

`traffic` scales the FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch) by
what the same counters read for the plain device copies of known size that
`bench.py --copy-calibration` runs after its timed steps (512 MiB read and
512 MiB written per copy).  Each row carries a digest of the kernel's source
files; bench.py reports the traffic only while that digest is current.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = "lsh_sparse_attention_hash_amd/csrc"
KERNEL_SOURCES = {
    "hash": [f"{CSRC}/hash.hip", f"{CSRC}/lsh_device.h"],
    "sort": [f"{CSRC}/sort.hip", f"{CSRC}/lsh_device.h"],
    "attend": [f"{CSRC}/attend.hip", f"{CSRC}/lsh_device.h"],
    "combine": [f"{CSRC}/combine.hip", f"{CSRC}/lsh_device.h"],
    "local": [f"{CSRC}/local.hip", f"{CSRC}/lsh_device.h"],
    "gemm": [f"{CSRC}/gemm.hip", f"{CSRC}/lsh_device.h"],
}
# kernel name prefix (as rocprofv3 prints it) -> step
STEP_OF = [("lsh::hash", "hash"), ("lsh::sort", "sort"), ("lsh::attend", "attend"),
           ("lsh::union_keys", "attend"), ("lsh::combine", "combine"), ("lsh::local", "local"),
           ("lsh::gemm", "gemm")]
COPY_BYTES = 512 << 20


def source_digest(step: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[step]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:12]


def _short(name: str) -> str:
    name = name.replace("void ", "")
    return name.split("(")[0]


def _step(name: str):
    for prefix, step in STEP_OF:
        if name.startswith(prefix):
            return step
    return None


def _counters(path: str, counter: str):
    per = collections.defaultdict(list)
    copies = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        k = _short(r["Kernel_Name"])
        v = float(r["Counter_Value"]) * 1024.0
        if "copyBuffer" in k and int(r["Grid_Size"]) >= 65536:
            copies.append(v)
        per[k].append(v)
    return per, copies


def traffic(args):
    fetch, fcopy = _counters(args.fetch, "FETCH_SIZE")
    write, wcopy = _counters(args.write, "WRITE_SIZE")
    if not fcopy or not wcopy:
        raise SystemExit("no calibration copies found (run bench.py with --copy-calibration)")
    fscale = COPY_BYTES / (sum(fcopy) / len(fcopy))
    wscale = COPY_BYTES / (sum(wcopy) / len(wcopy))
    steps = collections.defaultdict(lambda: [0.0, 0.0])
    lines = []
    for k in sorted(fetch, key=lambda n: (_step(n) or "~", n)):
        st = _step(k)
        if st is None:
            continue
        fb = sum(fetch[k]) / len(fetch[k]) * fscale
        wb = sum(write.get(k, [0.0])) / max(1, len(write.get(k, []))) * wscale
        steps[st][0] += fb
        steps[st][1] += wb
        lines.append(f"| {k} | {fb / 1e6:.1f} | {wb / 1e6:.1f} |")
    out = [f"# HBM traffic per launch — {args.workload} workload", "",
           "Commands (one MI355X, repository root):", ""]
    out += ["    " + c for c in args.command]
    out += ["", f"Scale factors from the 512 MiB device copies in the same runs: read x{fscale:.4f}, "
            f"write x{wscale:.4f} (counter KiB x 1024 x factor = bytes).", "",
            "| kernel | read MB | written MB |", "|---|---|---|"] + lines
    out += ["", "Per step (bytes per launch, all kernels of the step; digest of the step's sources):",
            "", "| step | workload | digest | bytes | read MB | written MB |", "|---|---|---|---|---|---|"]
    for st in ("hash", "sort", "attend", "combine", "local", "gemm"):
        if st in steps:
            fb, wb = steps[st]
            out.append(f"| {st} | {args.workload} | {source_digest(st)} | {fb + wb:.0f} | "
                       f"{fb / 1e6:.1f} | {wb / 1e6:.1f} |")
    print("\n".join(out))


def trace(args):
    rows = list(csv.DictReader(open(args.stats)))
    out = [f"# Kernel trace — {args.workload} workload", "", "Commands (one MI355X, repository root):", ""]
    out += ["    " + c for c in args.command]
    out += ["", "| kernel | calls | avg (us) | min (us) | max (us) | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = _short(r["Name"])
        if _step(name) is None:
            continue
        out.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{float(r['Percentage']):.1f} |")
    print("\n".join(out))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--command", action="append", default=[])
    k = sub.add_parser("trace")
    k.add_argument("--stats", required=True)
    k.add_argument("--workload", required=True)
    k.add_argument("--command", action="append", default=[])
    args = ap.parse_args()
    {"traffic": traffic, "trace": trace}[args.what](args)


if __name__ == "__main__":
    main()
