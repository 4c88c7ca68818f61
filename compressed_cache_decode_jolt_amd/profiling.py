"""Summaries of rocprofv3 output for the decode kernels.

    python -m compressed_cache_decode_jolt_amd.profiling stats CSV --command CMD --out FILE
    python -m compressed_cache_decode_jolt_amd.profiling traffic --workload NAME --kernel SUBSTR \\
        --fetch CSV --write CSV --calib-fetch CSV --calib-write CSV --copy-bytes N --out JSON

`stats` turns a `rocprofv3 --kernel-trace --stats -f csv` kernel_stats.csv
into a short markdown table.  `traffic` turns two `--pmc` runs (FETCH_SIZE,
then WRITE_SIZE, KiB per dispatch) into HBM bytes per launch of one kernel,
each counter scaled by what it reads for a plain device copy of known size
(the calibration runs), and records the hash of the kernel sources so a
stale figure is never reported for a changed kernel.
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


def counter_per_dispatch(path, counter, match=None):
    """{kernel name: [value per dispatch]} for one counter of a --pmc CSV."""
    acc = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        if match and match not in r["Kernel_Name"]:
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
    fb, wb = ff * sum(fv) / len(fv), wf * sum(wv) / len(wv)
    rec = {"kernel_hash": kernel_hash(), "bytes_per_launch": fb + wb,
           "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
           "dispatches": [len(fv), len(wv)],
           "calibration": {"copy_bytes": args.copy_bytes, "fetch_counter": fraw,
                           "write_counter": wraw, "fetch_bytes_per_unit": ff,
                           "write_bytes_per_unit": wf},
           "kernels": sorted(fetch)}
    data = json.load(open(args.out)) if os.path.exists(args.out) else {}
    data[f"{args.workload}/{args.name or args.kernel}"] = rec
    json.dump(data, open(args.out, "w"), indent=1, sort_keys=True)
    print(json.dumps(rec, indent=1))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="rocprofv3 kernel statistics")
    s.add_argument("--note", default="")
    s.add_argument("--out", required=True)
    s.add_argument("--trace", default=None, help="kernel-trace CSV for --window")
    s.add_argument("--window", nargs=3, metavar=("KERNEL", "START", "COUNT"), default=None,
                   help="also report the mean duration of these dispatches of KERNEL")
    t = sub.add_parser("traffic")
    for k in ("workload", "kernel", "fetch", "write", "calib_fetch", "calib_write", "out"):
        t.add_argument("--" + k.replace("_", "-"), required=True)
    t.add_argument("--name", default=None)
    t.add_argument("--copy-bytes", type=int, required=True)
    a = ap.parse_args()
    if a.cmd == "stats":
        text = f"# {a.title}\n\nCommand (from the repository root on one MI355X):\n\n```\n{a.command}\n```\n\n"
        if a.note:
            text += a.note + "\n\n"
        text += stats_table(a.csv) + "\n"
        if a.window:
            k, st, n = a.window[0], int(a.window[1]), int(a.window[2])
            text += ("\nMean duration of `%s` dispatches %d-%d (in start order): %.2f us\n"
                     % (k, st, st + n - 1, window_mean(a.trace, k, st, n)))
        text += "\nKernel sources hash: `%s`\n" % kernel_hash()
        open(a.out, "w").write(text)
        print(text)
    else:
        traffic(a)


if __name__ == "__main__":
    main()
