"""Turn rocprofv3 CSV output into the short text summaries kept under
profiles/ and the per-kernel HBM traffic record that bench.py reports.

    python -m layer_lstm_amd.profile_summary stats DIR OUT.txt --command "..."
    python -m layer_lstm_amd.profile_summary traffic --workload NAME \
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \
        --copy-bytes N --out-json profiles/traffic.json --out-txt OUT.txt \
        [--stats DIR] --command "..." [--command "..."]
    python -m layer_lstm_amd.profile_summary mfma DIR OUT.txt --workload NAME \
        --command "..."
    python -m layer_lstm_amd.profile_summary stalls DIR [DIR ...] --out OUT.txt \
        --workload NAME --command "..."

`stats` reads <DIR>/*kernel_stats.csv (rocprofv3 --kernel-trace --stats
--output-format csv) and writes the per-kernel table with the command that
produced it.  `traffic` reads the counter_collection.csv of four
rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, each for the LSTM step and
for a plain copy of --copy-bytes bytes), scales each counter by what it reads
for the copy (known bytes / counted bytes), and records HBM bytes per
launch for each kernel kind of the path, with the hash of the kernel's
source so that a record goes stale when the kernel changes; with --stats
(a rocprofv3 --kernel-trace --stats run of the same workload) it also
reports the achieved HBM GB/s of each kind (bytes per launch / average
launch duration).  `mfma` reads
one --pmc run of SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE and reports
the MFMA utilisation of each kernel kind.  `stalls` reads --pmc runs that
each include SQ_WAVE_CYCLES and reports every other SQ counter of them as a
share of the wave-cycles of each kernel kind (median over launches).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "layer_lstm_amd", "csrc")

# kernel kind -> (source files the kernel is built from, predicate on the
# demangled kernel name)
_REC = ("recurrent.hip", "recurrent_vec.hip", "recurrent_bwd.hip", "recurrent_common.hpp", "device_common.hpp",
        "internal.hpp")
_GEMM = ("gemm.hip", "device_common.hpp", "internal.hpp")
KINDS = {
    "input_projection": (_GEMM, lambda n: "gemm" in n and "EpiP" in n),
    "forward_recurrence": (_REC, lambda n: "fwd_rec_kernel" in n or "fwd_vec_kernel" in n),
    "backward_recurrence": (_REC, lambda n: "bwd_col_kernel" in n or "bwd_vec_kernel" in n),
    "dW_product": (_GEMM, lambda n: "EpiDW" in n and "splitk" not in n),
    "dx_product": (_GEMM, lambda n: "EpiStore" in n and "splitk" not in n),
}


def source_sha(fnames) -> str:
    h = hashlib.sha256()
    for f in fnames:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def kind_of(name: str):
    for k, (_, pred) in KINDS.items():
        if pred(name):
            return k
    return None


def find_csv(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[0]


def cmd_stats(a):
    rows = list(csv.DictReader(open(find_csv(a.dir, "kernel_stats.csv"))))
    lines = [f"# rocprofv3 kernel statistics", "", "command:", ""]
    lines += [f"    {c}" for c in a.command] + [""]
    lines.append(f"{'kernel':96s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}")
    for r in rows:
        name = r["Name"]
        if len(name) > 96:
            name = name[:93] + "..."
        lines.append(f"{name:96s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):6.2f}")
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counter_rows(d: str, counter: str):
    """Per-dispatch (kernel name, value) of one counter."""
    out = []
    for r in csv.DictReader(open(find_csv(d, "counter_collection.csv"))):
        if r.get("Counter_Name") == counter:
            out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    if not out:
        raise SystemExit(f"counter {counter} not found under {d}")
    return out


def copy_factor(d: str, counter: str, nbytes: int):
    """Known bytes / counted bytes for the largest dispatch of the copy run
    (the copy itself; torch's small set-up kernels are smaller)."""
    rows = counter_rows(d, counter)
    name, kib = max(rows, key=lambda r: r[1])
    return nbytes / (kib * 1024.0), name, kib


def kind_durations(d: str):
    """Average launch duration (ns) of each kernel kind from a kernel_stats.csv."""
    tot = {}
    for r in csv.DictReader(open(find_csv(d, "kernel_stats.csv"))):
        k = kind_of(r["Name"])
        if k is None:
            continue
        ns, n = tot.get(k, (0.0, 0))
        tot[k] = (ns + float(r["TotalDurationNs"]), n + int(r["Calls"]))
    return {k: ns / n for k, (ns, n) in tot.items() if n}


def cmd_traffic(a):
    ff, fname, fkib = copy_factor(a.copy_fetch, "FETCH_SIZE", a.copy_bytes)
    wf, wname, wkib = copy_factor(a.copy_write, "WRITE_SIZE", a.copy_bytes)
    per = {}
    for counter, d, fac in (("FETCH_SIZE", a.fetch, ff), ("WRITE_SIZE", a.write, wf)):
        for name, kib in counter_rows(d, counter):
            k = kind_of(name)
            if k is None:
                continue
            per.setdefault(k, {}).setdefault(counter, []).append(kib * 1024.0 * fac)
    try:
        rec = json.load(open(a.out_json))
    except (OSError, ValueError):
        rec = {}
    wrec = rec.setdefault(a.workload, {})
    lines = ["# HBM traffic per launch from rocprofv3 counters", "", "commands:", ""]
    lines += [f"    {c}" for c in a.command] + [""]
    lines.append(f"copy calibration: {a.copy_bytes} bytes copied; FETCH_SIZE read {fkib:.0f} KiB "
                 f"(factor {ff:.4f}), WRITE_SIZE read {wkib:.0f} KiB (factor {wf:.4f})")
    lines.append(f"workload {a.workload}")
    dur = kind_durations(a.stats) if a.stats else {}
    lines.append(f"{'kernel kind':22s} {'launches':>8s} {'fetch MB':>10s} {'write MB':>10s} {'total MB':>10s}"
                 + (f" {'avg us':>9s} {'GB/s':>8s}" if dur else ""))
    for k, v in per.items():
        fetch = statistics.median(v.get("FETCH_SIZE", [0.0]))
        write = statistics.median(v.get("WRITE_SIZE", [0.0]))
        n = len(v.get("FETCH_SIZE", []))
        wrec[k] = {"bytes_per_launch": round(fetch + write), "fetch_bytes": round(fetch), "write_bytes": round(write),
                   "source_sha": source_sha(KINDS[k][0]), "copy_factor_fetch": round(ff, 5),
                   "copy_factor_write": round(wf, 5)}
        row = f"{k:22s} {n:8d} {fetch / 1e6:10.3f} {write / 1e6:10.3f} {(fetch + write) / 1e6:10.3f}"
        if k in dur:
            row += f" {dur[k] / 1e3:9.1f} {(fetch + write) / dur[k]:8.0f}"
        lines.append(row)
    json.dump(rec, open(a.out_json, "w"), indent=1, sort_keys=True)
    open(a.out_txt, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_mfma(a):
    """MFMA utilisation per kernel kind from one rocprofv3 --pmc run with
    SQ_VALU_MFMA_BUSY_CYCLES (busy cycles summed over SIMDs) and
    GRBM_GUI_ACTIVE (active cycles summed over the XCDs):
    utilisation = busy / (active / xcds * simds)."""
    rows = list(csv.DictReader(open(find_csv(a.dir, "counter_collection.csv"))))
    per = {}
    for r in rows:
        k = kind_of(r["Kernel_Name"])
        if k is None:
            continue
        key = (k, r["Dispatch_Id"])
        per.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
    agg = {}
    for (k, _), d in per.items():
        if "SQ_VALU_MFMA_BUSY_CYCLES" in d and "GRBM_GUI_ACTIVE" in d and d["GRBM_GUI_ACTIVE"] > 0:
            u = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (d["GRBM_GUI_ACTIVE"] / a.xcds * a.simds)
            agg.setdefault(k, []).append(u)
    lines = ["# MFMA utilisation per kernel from rocprofv3 counters", "", "command:", ""]
    lines += [f"    {c}" for c in a.command] + [""]
    lines.append(f"utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {a.xcds} XCDs x {a.simds} SIMDs)")
    lines.append(f"workload {a.workload}")
    lines.append(f"{'kernel kind':22s} {'launches':>8s} {'MFMA busy':>10s}")
    for k, v in agg.items():
        lines.append(f"{k:22s} {len(v):8d} {100 * statistics.median(v):9.1f}%")
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


# per-wave SQ counters that `stalls` reports against SQ_WAVE_CYCLES (the
# others of a run, counted per SIMD or per CU, are left out)
WAVE_COUNTERS = ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
                 "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_ANY")


def cmd_stalls(a):
    """Each per-wave SQ counter of the runs as a share of SQ_WAVE_CYCLES
    (both summed over the device for one dispatch), median over the
    dispatches of a kernel kind."""
    shares = {}
    names = []
    for d in a.dirs:
        per = {}
        for r in csv.DictReader(open(find_csv(d, "counter_collection.csv"))):
            k = kind_of(r["Kernel_Name"])
            if k is None:
                continue
            per.setdefault((k, r["Dispatch_Id"]), {})[r["Counter_Name"]] = float(r["Counter_Value"])
        for (k, _), c in per.items():
            wc = c.get("SQ_WAVE_CYCLES", 0.0)
            if wc <= 0:
                continue
            for n, v in c.items():
                if n not in WAVE_COUNTERS:
                    continue
                if n not in names:
                    names.append(n)
                shares.setdefault(k, {}).setdefault(n, []).append(v / wc)
    lines = ["# Wave-cycle shares per kernel from rocprofv3 counters", "", "commands:", ""]
    lines += [f"    {c}" for c in a.command] + [""]
    lines.append("share = counter / SQ_WAVE_CYCLES of the same launch (median over launches).  WAIT_ANY: waves")
    lines.append("waiting on s_waitcnt or a barrier; WAIT_INST_ANY: waves ready but not issuing (dependencies, a")
    lines.append("busy unit such as the other wave's MFMAs); ACTIVE_INST_*: issuing that kind (VALU includes MFMA)")
    lines.append(f"workload {a.workload}")
    short = [n[3:] for n in names]
    lines.append(f"{'kernel kind':22s} " + " ".join(f"{n:>14s}" for n in short))
    for k in KINDS:
        if k not in shares:
            continue
        row = f"{k:22s} "
        row += " ".join(f"{100 * statistics.median(shares[k][n]):13.1f}%" if n in shares[k] else f"{'-':>14s}"
                        for n in names)
        lines.append(row)
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    mm = sub.add_parser("mfma")
    mm.add_argument("dir")
    mm.add_argument("out")
    mm.add_argument("--workload", required=True)
    mm.add_argument("--xcds", type=int, default=8)
    mm.add_argument("--simds", type=int, default=1024)
    mm.add_argument("--command", action="append", default=[])
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("out")
    s.add_argument("--command", action="append", default=[])
    t = sub.add_parser("traffic")
    t.add_argument("--workload", required=True)
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--out-json", required=True)
    t.add_argument("--out-txt", required=True)
    t.add_argument("--stats", default=None)
    t.add_argument("--command", action="append", default=[])
    st = sub.add_parser("stalls")
    st.add_argument("dirs", nargs="+")
    st.add_argument("--out", required=True)
    st.add_argument("--workload", required=True)
    st.add_argument("--command", action="append", default=[])
    a = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "mfma": cmd_mfma, "stalls": cmd_stalls}[a.cmd](a)


if __name__ == "__main__":
    main()
