"""Summaries of rocprofv3 output for the decode kernels.

    python -m compressed_cache_decode_jolt_amd.profiling stats CSV --command CMD --out FILE
    python -m compressed_cache_decode_jolt_amd.profiling traffic --workload NAME --kernel SUBSTR \\
        --fetch CSV --write CSV --calib-fetch CSV --calib-write CSV --copy-bytes N --out JSON \\
        [--md FILE --command CMD --title T --alg-bytes B]
    python -m compressed_cache_decode_jolt_amd.profiling counters CSV --kernel SUBSTR \\
        --command CMD --out FILE

`stats` turns a `rocprofv3 --kernel-trace --stats -f csv` kernel_stats.csv
into a short markdown table.  `traffic` turns two `--pmc` runs (FETCH_SIZE,
then WRITE_SIZE, KiB per dispatch) into HBM bytes per launch of one kernel,
each counter scaled by what it reads for a plain device copy of known size
(the calibration runs), and records the hash of the kernel sources so a
stale figure is never reported for a changed kernel.  `counters` turns one
`--pmc` run of busy / activity counters into a per-kernel table of means per
dispatch with the derived utilisation ratios.
"""
import argparse
import csv
import hashlib
import json
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))


def _code_only(text):
    """C/C++ source without comments and with whitespace runs collapsed, so
    that an edit of a comment does not change the hash of the code."""
    text = re.sub(r"//[^\n]*", " ", text)
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    return " ".join(text.split())


def kernel_hash():
    """Hash of the HIP sources (kernels, headers, includes), comments and
    whitespace aside."""
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".inc")):
            h.update(f.encode() + b"\0")
            h.update(_code_only(open(os.path.join(csrc, f)).read()).encode())
    return h.hexdigest()[:16]


def short_name(name):
    name = name.strip('"')
    return name if len(name) <= 90 else name[:87] + "..."


def stats_table(path, top=8):
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = ["| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows[:top]:
        out.append("| `%s` | %s | %.2f | %.2f | %.2f | %.1f |" % (
            short_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return "\n".join(out)


def window_mean(trace, match, start, count):
    """Mean duration (us) of dispatches start .. start+count-1, in start-time
    order, of the kernels whose name contains ``match`` (a --kernel-trace CSV)."""
    rows = [r for r in csv.DictReader(open(trace)) if match in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    sel = rows[start:start + count]
    assert len(sel) == count, f"only {len(rows)} dispatches of {match!r}"
    return sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in sel) / count / 1e3


def call_window_mean(trace, start, count, first="decode_mfma", last="value_finish",
                     kernels=("decode_mfma", "merge_outputs", "value_gemm", "value_finish"),
                     per_call=None):
    """Mean span (us) of layer calls start .. start+count-1 of a --kernel-trace
    CSV: a call is a run of ``first`` dispatches and the kernels after it up
    to the next ``first``; its span runs from its first dispatch's start to
    the end of its ``last`` dispatch if it has one, else of its last
    ``first`` dispatch -- what the library's timing events bracket.  A call
    launches each of its classes (kernel names) once, so a ``first``
    dispatch whose name the current run already holds starts a new call
    (single-split calls without a value pass have no kernel in between).
    per_call: the calls' number of ``first`` dispatches where it is fixed
    (a call of one class, e.g.), so that calls of different classes that
    follow each other with nothing in between are told apart too."""
    rows = [r for r in csv.DictReader(open(trace)) if any(k in r["Kernel_Name"] for k in kernels)]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    calls, cur, prev_first, seen = [], None, False, set()
    for r in rows:
        is_first = first in r["Kernel_Name"]
        if is_first and (not prev_first or r["Kernel_Name"] in seen or
                         (per_call and len(seen) >= per_call)):
            cur = {"start": int(r["Start_Timestamp"]), "end_first": 0, "end_last": None}
            calls.append(cur)
            seen = set()
        if is_first:
            seen.add(r["Kernel_Name"])
        if cur is None:
            continue
        if is_first:
            cur["end_first"] = max(cur["end_first"], int(r["End_Timestamp"]))
        elif last in r["Kernel_Name"]:
            cur["end_last"] = int(r["End_Timestamp"])
        prev_first = is_first
    sel = calls[start:start + count]
    assert len(sel) == count, f"only {len(calls)} calls"
    return sum(((c["end_last"] or c["end_first"]) - c["start"]) for c in sel) / count / 1e3


def counter_per_dispatch(path, counter, match=None):
    """{kernel name: [value per dispatch]} for one counter of a --pmc CSV."""
    acc = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        if match and not any(m in r["Kernel_Name"] for m in match.split("|")):
            continue
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    per = {}
    for (name, _), v in acc.items():
        per.setdefault(name, []).append(v)
    return per


def copy_factor(path, counter, copy_bytes):
    """Bytes per counter unit: the copy kernel is the dispatch with the
    largest reading; it moved copy_bytes in each direction."""
    per = counter_per_dispatch(path, counter)
    best = max(max(v) for v in per.values())
    return copy_bytes / best, best


def traffic(args):
    ff, fraw = copy_factor(args.calib_fetch, "FETCH_SIZE", args.copy_bytes)
    wf, wraw = copy_factor(args.calib_write, "WRITE_SIZE", args.copy_bytes)
    fetch = counter_per_dispatch(args.fetch, "FETCH_SIZE", args.kernel)
    write = counter_per_dispatch(args.write, "WRITE_SIZE", args.kernel)
    assert fetch and write, f"no dispatch of a kernel matching {args.kernel!r}"
    fv = [x for v in fetch.values() for x in v]
    wv = [x for v in write.values() for x in v]
    # a launch (one layer call) may run several launch classes, i.e.
    # dispatches of the anchor kernel (the first of --kernel's alternatives),
    # and other kernels (a second value pass): bytes per launch = all
    # matching dispatches' bytes / launches, launches = anchor dispatches /
    # dispatches per launch
    per = getattr(args, "dispatches_per_launch", 1.0) or 1.0
    anchor = args.kernel.split("|")[0]
    nf = sum(len(v) for k, v in fetch.items() if anchor in k) / per
    nw = sum(len(v) for k, v in write.items() if anchor in k) / per
    fb, wb = ff * sum(fv) / nf, wf * sum(wv) / nw
    rec = {"kernel_hash": kernel_hash(), "bytes_per_launch": fb + wb,
           "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
           "dispatches": [len(fv), len(wv)], "dispatches_per_launch": per,
           "calibration": {"copy_bytes": args.copy_bytes, "fetch_counter": fraw,
                           "write_counter": wraw, "fetch_bytes_per_unit": ff,
                           "write_bytes_per_unit": wf},
           "kernels": sorted(fetch)}
    data = json.load(open(args.out)) if os.path.exists(args.out) else {}
    data[f"{args.workload}/{args.name or args.kernel}"] = rec
    json.dump(data, open(args.out, "w"), indent=1, sort_keys=True)
    print(json.dumps(rec, indent=1))
    if getattr(args, "md", None):
        lines = [f"# {args.title}", "", "Commands (from the repository root on one MI355X):", "",
                 "```", args.command, "```", "",
                 "| quantity | value |", "|---|---|",
                 "| copy of %s B: FETCH_SIZE | %s (=> %.1f B per unit) |" % (
                     f"{args.copy_bytes:,}", f"{fraw:,.0f}", ff),
                 "| copy of %s B: WRITE_SIZE | %s (=> %.1f B per unit) |" % (
                     f"{args.copy_bytes:,}", f"{wraw:,.0f}", wf),
                 "| `%s` FETCH_SIZE x factor | %s B per launch (%d dispatches, %.3g of `%s` per launch) |" % (
                     args.kernel, f"{fb:,.0f}", len(fv), per, anchor),
                 "| `%s` WRITE_SIZE x factor | %s B per launch (%d dispatches, %.3g of `%s` per launch) |" % (
                     args.kernel, f"{wb:,.0f}", len(wv), per, anchor),
                 "| HBM traffic per launch | %s B |" % f"{fb + wb:,.0f}"]
        if args.alg_bytes:
            lines += ["| algorithmic bytes per launch | %s B |" % f"{args.alg_bytes:,.0f}",
                      "| traffic / algorithmic | %.2f |" % ((fb + wb) / args.alg_bytes)]
        lines += ["", "Per kernel instantiation (mean per dispatch):", "",
                  "| kernel | dispatches | fetch B | write B |", "|---|---|---|---|"]
        for name in sorted(fetch):
            f_ = fetch[name]
            w_ = write.get(name, [0.0])
            lines.append("| `%s` | %d | %s | %s |" % (short_name(name), len(f_),
                                                    f"{ff * sum(f_) / len(f_):,.0f}",
                                                    f"{wf * sum(w_) / len(w_):,.0f}"))
        lines += ["", "Kernel sources hash: `%s`" % rec["kernel_hash"], ""]
        open(args.md, "w").write("\n".join(lines))


# derived ratios of the busy counters: (name, numerator, denominator)
RATIOS = [("MFMA busy / CU busy", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES"),
          ("VALU active / wave cycles", "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES"),
          ("LDS active / wave cycles", "SQ_ACTIVE_INST_LDS", "SQ_WAVE_CYCLES"),
          ("waiting / wave cycles", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
          ("waiting on LDS / wave cycles", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES")]


def counters_table(path, match):
    """Markdown table: per kernel whose name contains ``match``, the mean per
    dispatch of every counter in a --pmc CSV, then the ratios of RATIOS whose
    counters are present."""
    names = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] not in names:
            names.append(r["Counter_Name"])
    per = {c: counter_per_dispatch(path, c, match) for c in names}
    kernels = sorted({k for c in names for k in per[c]})
    mean = {k: {c: sum(per[c][k]) / len(per[c][k]) for c in names if k in per[c]} for k in kernels}
    ratios = [r for r in RATIOS if r[1] in names and r[2] in names]
    head = ["kernel", "dispatches"] + names + [r[0] for r in ratios]
    out = ["| " + " | ".join(head) + " |", "|" + "---|" * len(head)]
    for k in kernels:
        m = mean[k]
        cells = ["`%s`" % short_name(k), str(len(per[names[0]].get(k, [])))]
        cells += ["%.4g" % m[c] if c in m else "" for c in names]
        cells += ["%.3f" % (m[n] / m[d]) if m.get(d) else "" for _, n, d in ratios]
        out.append("| " + " | ".join(cells) + " |")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="rocprofv3 kernel statistics")
    s.add_argument("--note", default="")
    s.add_argument("--out", required=True)
    s.add_argument("--top", type=int, default=8, help="rows of the table")
    s.add_argument("--trace", default=None, help="kernel-trace CSV for --window")
    s.add_argument("--window", nargs=3, metavar=("KERNEL", "START", "COUNT"), default=None,
                   help="also report the mean duration of these dispatches of KERNEL")
    s.add_argument("--call-window", nargs=2, type=int, metavar=("START", "COUNT"), default=None,
                   help="also report the mean span of these layer calls (split kernels to "
                        "the end of the second value pass)")
    s.add_argument("--call-dispatches", type=int, default=None,
                   help="split-kernel dispatches per layer call, where it is fixed")
    t = sub.add_parser("traffic")
    for k in ("workload", "kernel", "fetch", "write", "calib_fetch", "calib_write", "out"):
        t.add_argument("--" + k.replace("_", "-"), required=True)
    t.add_argument("--name", default=None)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--md", default=None, help="also write a markdown summary here")
    t.add_argument("--command", default="")
    t.add_argument("--title", default="HBM traffic")
    t.add_argument("--alg-bytes", type=float, default=0.0)
    t.add_argument("--dispatches-per-launch", type=float, default=1.0,
                   help="kernel dispatches per launch of the bench's roofline (a layer call)")
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("--kernel", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--title", default="rocprofv3 counters")
    c.add_argument("--note", default="")
    c.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.cmd == "stats":
        text = f"# {a.title}\n\nCommand (from the repository root on one MI355X):\n\n```\n{a.command}\n```\n\n"
        if a.note:
            text += a.note + "\n\n"
        text += stats_table(a.csv, a.top) + "\n"
        if a.window:
            k, st, n = a.window[0], int(a.window[1]), int(a.window[2])
            text += ("\nMean duration of `%s` dispatches %d-%d (in start order): %.2f us\n"
                     % (k, st, st + n - 1, window_mean(a.trace, k, st, n)))
        if a.call_window:
            st, n = a.call_window
            text += ("\nMean span of layer calls %d-%d (first split-kernel start to the end of the "
                     "call's last split kernel, or of its second value pass): %.2f us\n"
                     % (st, st + n - 1, call_window_mean(a.trace, st, n, per_call=a.call_dispatches)))
        text += "\nKernel sources hash: `%s`\n" % kernel_hash()
        open(a.out, "w").write(text)
        print(text)
    elif a.cmd == "counters":
        text = f"# {a.title}\n\nCommand (from the repository root on one MI355X):\n\n```\n{a.command}\n```\n\n"
        if a.note:
            text += a.note + "\n\n"
        text += counters_table(a.csv, a.kernel) + "\n"
        text += "\nKernel sources hash: `%s`\n" % kernel_hash()
        open(a.out, "w").write(text)
        print(text)
    else:
        traffic(a)


if __name__ == "__main__":
    main()
