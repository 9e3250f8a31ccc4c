"""Turn rocprofv3 CSV output into the short summaries kept under profiles/.

    python3 -m lsh_sparse_attention_hash_amd.rocprof_summary trace \
        --stats <dir>/<name>_kernel_stats.csv --workload long --command "..."
    python3 -m lsh_sparse_attention_hash_amd.rocprof_summary traffic \
        --fetch <fetch>_counter_collection.csv --write <write>_counter_collection.csv \
        --workload long --command "..."
    python3 -m lsh_sparse_attention_hash_amd.rocprof_summary busy \
        --counters <busy>_counter_collection.csv --workload long --command "..."

`traffic` scales the FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch) by
what the same counters read for the plain device copies of known size that
`bench.py --copy-calibration` runs after its timed steps (512 MiB read and
512 MiB written per copy).  Each row carries a digest of the kernel's source
files; bench.py reports the traffic only while that digest is current.

`busy` turns one pass of SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_MFMA,
SQ_INSTS_VALU and GRBM_GUI_ACTIVE into the matrix cores' busy fraction per
kernel: busy SIMD-cycles / (SIMDs x cycles of the dispatch), the cycles being
GRBM_GUI_ACTIVE divided by the number of XCDs it is summed over.
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
           ("lsh::union_keys", "attend"), ("lsh::vmax", "attend"), ("lsh::combine", "combine"),
           ("lsh::local", "local"),
           ("lsh::gemm", "gemm")]
COPY_BYTES = 512 << 20
SIMDS = 256 * 4   # 256 CUs of 4 SIMDs
XCDS = 8          # GRBM_GUI_ACTIVE is summed over the XCDs


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


def busy(args):
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(list)
    for r in csv.DictReader(open(args.counters)):
        k = _short(r["Kernel_Name"])
        if _step(k) is None:
            continue
        per[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
            dur[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    out = [f"# Matrix-core busy fraction per launch — {args.workload} workload", "",
           "Commands (one MI355X, repository root):", ""]
    out += ["    " + c for c in args.command]
    out += ["", f"busy = SQ_VALU_MFMA_BUSY_CYCLES / ({SIMDS} SIMDs x GRBM_GUI_ACTIVE / {XCDS}); "
            "clock = GRBM_GUI_ACTIVE / {XCDS} / dispatch time (the profiled dispatch, counters "
            "on; shown for dispatches of 50 us or more). Instruction counts are wave instructions per launch; SQ_INSTS_VALU includes "
            "the MFMA instructions.".replace("{XCDS}", str(XCDS)), "",
            "| kernel | launches | dispatch us | clock GHz | MFMA instructions | VALU instructions "
            "| MFMA busy SIMD-cycles | MFMA busy |", "|---|---|---|---|---|---|---|---|"]
    steps = {}
    mean = lambda xs: sum(xs) / len(xs)
    for k in sorted(per, key=lambda n: (_step(n) or "~", n)):
        c = per[k]
        if not all(n in c for n in ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
                                    "GRBM_GUI_ACTIVE")):
            continue
        cyc = mean(c["GRBM_GUI_ACTIVE"]) / XCDS
        mb = mean(c["SQ_VALU_MFMA_BUSY_CYCLES"])
        frac = mb / (SIMDS * cyc) if cyc > 0 else 0.0
        t = mean(dur[k])
        # a short dispatch's GRBM count is dominated by the counters' own set-up
        clock = f"{cyc / t / 1e9:.2f}" if t >= 50e-6 else "-"
        out.append(f"| {k} | {len(c['GRBM_GUI_ACTIVE'])} | {t * 1e6:.1f} | {clock} | "
                   f"{mean(c['SQ_INSTS_MFMA']):.0f} | {mean(c['SQ_INSTS_VALU']):.0f} | {mb:.0f} | "
                   f"{frac:.3f} |")
        st = _step(k)
        if mb > 0 and (st not in steps or mb > steps[st][1]):
            steps[st] = (k, mb, frac)
    out += ["", "Per step (the step's kernel with the most matrix-core work; digest of the step's "
            "sources):", "", "| step | workload | digest | kernel | MFMA busy |", "|---|---|---|---|---|"]
    for st in ("hash", "sort", "attend", "combine", "local", "gemm"):
        if st in steps:
            k, _, frac = steps[st]
            out.append(f"| {st} | {args.workload} | {source_digest(st)} | {k} | {frac:.3f} |")
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
    b = sub.add_parser("busy")
    b.add_argument("--counters", required=True)
    b.add_argument("--workload", required=True)
    b.add_argument("--command", action="append", default=[])
    args = ap.parse_args()
    {"traffic": traffic, "trace": trace, "busy": busy}[args.what](args)


if __name__ == "__main__":
    main()
