"""Summarise rocprofv3 CSV output into the short text summaries kept under profiles/.

    # kernel durations (rocprofv3 --kernel-trace --stats -f csv ... -o NAME)
    python -m attention_forward_amd.profsum stats DIR NAME --cmd "<command>" [--skip-first N | --last N] > profiles/X.md

    # HBM bytes per dispatch from two --pmc runs (FETCH_SIZE, WRITE_SIZE), each scaled by
    # what the same counter reads for a plain copy of --copy-mib MiB run in the same process
    python -m attention_forward_amd.profsum traffic DIR FETCH_NAME WRITE_NAME --copy-mib 1024 \
        --cmd-fetch "<command>" --cmd-write "<command>" --out profiles/traffic.json > profiles/Y.md

    # several workloads at once: comma-separated FETCH and WRITE runs, one pair per workload
    python -m attention_forward_amd.profsum traffic DIR F1,F2 W1,W2 --copy-mib 1024 ...

    # one table over workloads profiled one per process (attention_forward_amd/profile_run.py):
    # DIR/trace_W.json (stats --last N --json) and the passes mfma_W issue_W l2_W fetch_W write_W
    python -m attention_forward_amd.profsum workloads DIR W1 W2 ... --copy-mib 1024

    # per-kernel means of any counters, one --pmc run per NAME
    python -m attention_forward_amd.profsum counters DIR NAME[@SUBSTR] ... --cmd "<c1>" --cmd "<c2>"

Only parses files; it runs nothing on the GPU.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace runs collapsed (string
    literals in these sources hold no comment markers)."""
    import re

    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_sources_hash() -> str:
    """sha256 over the code (comments and layout ignored) of the HIP sources and
    headers the kernels are built from."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(HERE, "csrc", "*.h")) +
                   glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    for f in files:
        h.update(os.path.basename(f).encode())
        h.update(_code_only(open(f, encoding="utf-8").read()).encode())
    return h.hexdigest()


def short(name: str) -> str:
    name = name.replace("void ", "")
    i = name.find("(")
    return name if i < 0 else name[:i]


def stats(d, name, cmd, skip_first=0, last=0, json_out=None):
    """The --stats table, and (with skip_first) the same averages over each kernel's
    dispatches after its first skip_first, from the kernel trace: the untimed
    warmup steps of a benchmark run drop out, so the figures compare with the
    benchmark's own timed-step averages."""
    path = os.path.join(d, name + "_kernel_stats.csv")
    rows = list(csv.DictReader(open(path)))
    out = ["# Kernel durations", "", "Command:", "", "```", cmd, "```", "",
           "All dispatches (rocprofv3 --stats):", "",
           "| kernel | calls | average µs | min µs | max µs | share |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        out.append("| `%s` | %s | %.1f | %.1f | %.1f | %.1f%% |" % (
            short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    if skip_first > 0 or last > 0:
        trace = os.path.join(d, name + "_kernel_trace.csv")
        per = collections.defaultdict(list)
        for r in csv.DictReader(open(trace)):
            per[short(r["Kernel_Name"])].append(
                (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        what = ("each kernel's last %d dispatches (the measured launches, after the warmup)" % last
                if last > 0 else
                "dispatches after each kernel's first %d (the untimed warmup steps)" % skip_first)
        out += ["", what[0].upper() + what[1:] + ":", "",
                "| kernel | calls | average µs | median µs | min µs | max µs |",
                "|---|---|---|---|---|---|"]
        summary = {}
        for k, v in per.items():
            v = sorted(v)
            dur = sorted(x[1] for x in (v[-last:] if last > 0 else v[skip_first:]))
            if not dur:
                continue
            summary[k] = {"calls": len(dur), "avg_us": sum(dur) / len(dur) / 1e3,
                          "median_us": dur[len(dur) // 2] / 1e3, "min_us": dur[0] / 1e3,
                          "max_us": dur[-1] / 1e3}
            out.append("| `%s` | %d | %.1f | %.1f | %.1f | %.1f |" % (
                k, len(dur), sum(dur) / len(dur) / 1e3, dur[len(dur) // 2] / 1e3, dur[0] / 1e3,
                dur[-1] / 1e3))
        if json_out:
            with open(json_out, "w") as fh:
                json.dump({"cmd": cmd, "kernels": summary}, fh, indent=1, sort_keys=True)
    return "\n".join(out) + "\n"


def _open_csv(path):
    """A counter CSV, or its gzip-compressed copy (PATH.gz)."""
    import gzip

    if os.path.exists(path):
        return open(path)
    return gzip.open(path + ".gz", "rt")


def _counters(path):
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(_open_csv(path)):
        agg[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return agg


def traffic(d, fetch_name, write_name, copy_mib, cmd_fetch, cmd_write, out_json):
    """fetch_name / write_name: one run each, or comma-separated lists of runs
    (one workload per pair), each pair scaled by its own copy kernel."""
    copy_kib = copy_mib * 1024.0

    def find_copy(agg, counter):
        for k, v in agg.items():
            if COPY_KERNEL in k and counter in v:
                return max(v[counter])
        raise SystemExit("no %s dispatch with %s in the counter file" % (COPY_KERNEL, counter))

    result = {"kernel_sources_sha256": kernel_sources_hash(), "copy_mib": copy_mib,
              "kernels": {}}
    lines = ["# HBM traffic per dispatch", "",
             "FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by the factor that makes the",
             "same counter read %d MiB for a plain %d MiB device copy in the same process." % (copy_mib, copy_mib),
             "", "Commands:", "", "```", cmd_fetch, cmd_write, "```", "",
             "| run | kernel | dispatches | FETCH KiB (raw) | WRITE KiB (raw) | FETCH scale | "
             "WRITE scale | read MB | written MB |",
             "|---|---|---|---|---|---|---|---|---|"]
    fnames, wnames = fetch_name.split(","), write_name.split(",")
    if len(fnames) != len(wnames):
        raise SystemExit("as many FETCH_SIZE runs as WRITE_SIZE runs")
    for fn, wn in zip(fnames, wnames):
        f = _counters(os.path.join(d, fn + "_counter_collection.csv"))
        w = _counters(os.path.join(d, wn + "_counter_collection.csv"))
        f_scale = copy_kib / find_copy(f, "FETCH_SIZE")
        w_scale = copy_kib / find_copy(w, "WRITE_SIZE")
        for k in f:
            if "attn::" not in k:
                continue
            fv = f[k].get("FETCH_SIZE", [])
            wv = w.get(k, {}).get("WRITE_SIZE", [])
            if not fv or not wv:
                continue
            fk = sum(fv) / len(fv)
            wk = sum(wv) / len(wv)
            rd = fk * 1024 * f_scale
            wr = wk * 1024 * w_scale
            result["kernels"][short(k)] = {"read_bytes": rd, "write_bytes": wr,
                                           "dispatches": len(fv), "fetch_scale": f_scale,
                                           "write_scale": w_scale}
            lines.append("| %s | `%s` | %d | %.0f | %.0f | %.4f | %.4f | %.1f | %.1f |" % (
                fn, short(k), len(fv), fk, wk, f_scale, w_scale, rd / 1e6, wr / 1e6))
    if out_json:
        with open(out_json, "w") as fh:
            json.dump(result, fh, indent=1, sort_keys=True)
    return "\n".join(lines) + "\n"


def counters(d, names, cmds, match=("attn::",), xcc=8, simds=1024):
    """Per-kernel mean over dispatches of every counter in one or more --pmc runs
    (one run per name, each within the hardware's per-block counter limits).

    GRBM_GUI_ACTIVE is summed over the XCDs in the CSV, so its per-XCD value over
    the dispatch's duration is the effective shader clock (slightly high for short
    dispatches, whose counter window includes the launch); MFMA busy is
    SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs) over SIMDs x per-XCD cycles."""
    out = ["# Hardware counters per dispatch", "", "Commands (one counter pass each):", "", "```"]
    out += list(cmds) + ["```", ""]
    for name in names:
        name, _, only = name.partition("@")  # NAME@SUBSTR: this pass's kernels must hold SUBSTR
        pass_match = (only,) if only else match
        path = os.path.join(d, name + "_counter_collection.csv")
        agg = _counters(path)
        dur = collections.defaultdict(dict)
        for r in csv.DictReader(_open_csv(path)):
            dur[r["Kernel_Name"]][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) -
                                                       int(r["Start_Timestamp"]))
        out += ["Pass `%s`:" % name, ""]
        kernels = [k for k in agg if any(m in k for m in pass_match)]
        cols = sorted({c for k in kernels for c in agg[k]})
        derived = []
        if "GRBM_GUI_ACTIVE" in cols:
            derived.append("clock GHz")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in cols:
                derived.append("MFMA busy")
        out.append("| kernel | dispatches | mean µs | " + " | ".join(cols + derived) + " |")
        out.append("|---|---|---|" + "---|" * (len(cols) + len(derived)))
        for k in kernels:
            n = max(len(v) for v in agg[k].values())
            mean = {c: sum(v) / len(v) for c, v in agg[k].items() if v}
            ns = sum(dur[k].values()) / len(dur[k])
            cells = ["%.4g" % mean[c] if c in mean else "" for c in cols]
            if derived:
                cyc = mean["GRBM_GUI_ACTIVE"] / xcc
                cells.append("%.2f" % (cyc / ns))
                if len(derived) > 1:
                    cells.append("%.1f%%" % (100.0 * mean["SQ_VALU_MFMA_BUSY_CYCLES"] /
                                             (simds * cyc)))
            out.append("| `%s` | %d | %.1f | %s |" % (short(k)[:70], n, ns / 1e3, " | ".join(cells)))
        out.append("")
    return "\n".join(out)


def workloads(d, names, copy_mib, xcc=8, simds=1024):
    """One table over workloads, each profiled in a process of its own (see
    profile_run.py): for workload W the directory holds trace_W.json (profsum
    stats --json of its kernel trace) and the counter passes mfma_W, issue_W,
    l2_W, fetch_W and write_W.  Per kernel: mean duration of the measured
    launches, the rate they give (TFLOP/s by the metric's FLOP count for a
    prefill, GB/s of algorithmic bytes for a decode step's split kernel), the
    shader clock and MFMA busy fraction over the dispatch, instructions per
    MFMA, the L2 hit rate and the HBM bytes per dispatch (FETCH_SIZE and
    WRITE_SIZE scaled by a plain copy of copy_mib MiB in the same process)."""
    from attention_forward_amd.synthetic import ALL_WORKLOADS, FP8_WORKLOADS

    rows = ["| workload | kernel | µs | rate | clock GHz | MFMA busy | VALU / MFMA | "
            "LDS / MFMA | co-exec / MFMA busy | L2 hit | read MB | written MB |",
            "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    copy_kib = copy_mib * 1024.0
    for wn in names:
        w = FP8_WORKLOADS.get(wn) or ALL_WORKLOADS[wn]
        tr = json.load(open(os.path.join(d, "trace_%s.json" % wn)))["kernels"]
        agg = {}
        for pas in ("mfma", "issue", "l2", "fetch", "write"):
            agg[pas] = _counters(os.path.join(d, "%s_%s_counter_collection.csv" % (pas, wn)))

        def copy_scale(pas, counter):
            for k, v in agg[pas].items():
                if COPY_KERNEL in k and counter in v:
                    return copy_kib / max(v[counter])
            return None

        fs, ws = copy_scale("fetch", "FETCH_SIZE"), copy_scale("write", "WRITE_SIZE")
        for full in agg["mfma"]:
            if "attn::" not in full:
                continue
            k = short(full)
            mean = {}
            for pas in ("mfma", "issue", "l2", "fetch", "write"):
                for c, v in agg[pas].get(full, {}).items():
                    mean[c] = sum(v) / len(v)
            t = tr.get(k)
            us = t["avg_us"] if t else float("nan")
            if "fa_fwd_kernel" in k:
                rate = "%.0f TFLOP/s" % (w.flops / (us * 1e-6) / 1e12)
            elif "decode_split" in k:
                kv = 2 * w.B * w.Hkv * w.Sk * w.d * 2
                rate = "%.0f GB/s (K, V)" % (kv / (us * 1e-6) / 1e9)
            else:
                rate = ""
            cyc = mean.get("GRBM_GUI_ACTIVE", 0.0) / xcc
            # the clock over the dispatch as the mfma pass timed it
            dur_ns = None
            for r in csv.DictReader(_open_csv(os.path.join(
                    d, "mfma_%s_counter_collection.csv" % wn))):
                if r["Kernel_Name"] == full:
                    dur_ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            clock = cyc / dur_ns if dur_ns else float("nan")
            busy = mean.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (simds * cyc) if cyc else 0.0
            mf = mean.get("SQ_INSTS_MFMA", 0.0)
            valu = (mean.get("SQ_INSTS_VALU", 0.0) - mf) / mf if mf else float("nan")
            lds = mean.get("SQ_INSTS_LDS", 0.0) / mf if mf else float("nan")
            coex = (mean.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) /
                    mean.get("SQ_VALU_MFMA_BUSY_CYCLES", 1.0)) if mf else float("nan")
            hit = mean.get("TCC_HIT_sum", 0.0)
            miss = mean.get("TCC_MISS_sum", 0.0)
            rd = mean.get("FETCH_SIZE", 0.0) * 1024 * fs / 1e6 if fs else float("nan")
            wr = mean.get("WRITE_SIZE", 0.0) * 1024 * ws / 1e6 if ws else float("nan")
            rows.append("| %s | `%s` | %.1f | %s | %.2f | %.1f%% | %.1f | %.2f | %.2f | %.1f%% | "
                        "%.1f | %.1f |" % (
                            wn, k, us, rate, clock, 100 * busy, valu, lds, coex,
                            100 * hit / max(hit + miss, 1.0), rd, wr))
    return "\n".join(rows) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("names", nargs="+")
    c.add_argument("--cmd", action="append", required=True)
    c.add_argument("--match", action="append", default=None,
                   help="substring a kernel name must hold (repeatable; default attn::)")
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("name")
    s.add_argument("--cmd", required=True)
    s.add_argument("--skip-first", type=int, default=0,
                   help="also average each kernel's dispatches after its first N")
    s.add_argument("--last", type=int, default=0,
                   help="also average each kernel's last N dispatches")
    s.add_argument("--json", default=None,
                   help="also write those averages (with --last/--skip-first) as JSON")
    wl = sub.add_parser("workloads")
    wl.add_argument("dir")
    wl.add_argument("names", nargs="+")
    wl.add_argument("--copy-mib", type=int, required=True)
    t = sub.add_parser("traffic")
    t.add_argument("dir")
    t.add_argument("fetch_name")
    t.add_argument("write_name")
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    t.add_argument("--out", default=None)
    a = ap.parse_args()
    if a.what == "stats":
        sys.stdout.write(stats(a.dir, a.name, a.cmd, a.skip_first, a.last, a.json))
    elif a.what == "workloads":
        sys.stdout.write(workloads(a.dir, a.names, a.copy_mib))
    elif a.what == "counters":
        sys.stdout.write(counters(a.dir, a.names, a.cmd, tuple(a.match or ["attn::"])))
    else:
        sys.stdout.write(traffic(a.dir, a.fetch_name, a.write_name, a.copy_mib, a.cmd_fetch,
                                 a.cmd_write, a.out))


if __name__ == "__main__":
    main()
