"""Summaries of rocprofv3 output for the drafter's kernels.

  python -m block_diffusion_draft_tap_amd.prof_report stats <kernel_stats.csv> [--per N] [--command CMD]
      Markdown table of a `rocprofv3 --kernel-trace --stats --output-format csv`
      run: calls, average / min / max duration and share of GPU time per kernel;
      --per divides the call counts by N, --per-kernel NAME by the call count of
      a kernel that runs once per step.

  python -m block_diffusion_draft_tap_amd.prof_report traffic --fetch <counter_collection.csv>
      --write <counter_collection.csv> --kernel <name substring> --copy-bytes N
      --algorithmic-bytes A [--command CMD ...]
      Memory traffic per launch of one kernel from two counter passes
      (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`, values in KiB per dispatch).
      Each counter is scaled by what it reads for a calibration kernel that
      reads and writes N bytes: the last PyTorch multiply kernel of the run
      (bench.py's calibration copy); the measured kernel's dispatches after it count.

  python -m block_diffusion_draft_tap_amd.prof_report counters <counter_collection.csv>...
      --kernel <name substring> [--command CMD ...]
      Per-dispatch averages of the counters of one kernel over one or more
      `--pmc` passes, with the share of LDS-active cycles lost to bank
      conflicts when both SQ_LDS_BANK_CONFLICT and SQ_LDS_IDX_ACTIVE are there.

The traffic summary records a hash of the sources that decide the measured
kernel (kernel_sources_hash: its own .hip file, the headers and the host launch
code, not the files of other kernels); a reader of the summary compares it with
the current sources and ignores the figure once they differ.
"""

import argparse
import csv
import hashlib
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
def _kernel_files():
    """{kernel function name: the .hip file that defines it}"""
    d = os.path.join(HERE, "csrc")
    out = {}
    for f in sorted(os.listdir(d)):
        if f.endswith(".hip"):
            with open(os.path.join(d, f)) as fh:
                for name in re.findall(r"\bvoid\s+([A-Za-z0-9_]+_kernel)\b", fh.read()):
                    out.setdefault(name, os.path.join("csrc", f))
    return out


def kernel_sources(kernel=None):
    """The sources that decide a kernel's code and launch shapes: the .hip file that defines
    it and every source that defines no other kernel (headers, the host code that sizes the
    launches). Without a kernel, or for one not found: every source."""
    d = os.path.join(HERE, "csrc")
    every = sorted(os.path.join("csrc", f) for f in os.listdir(d) if f.endswith((".hip", ".hpp", ".cpp")))
    if not kernel:
        return every
    files = _kernel_files()
    own = {f for n, f in files.items() if re.search(r"\b" + n + r"\b", kernel)}
    if not own:
        return every
    others = set(files.values()) - own
    return [rel for rel in every if rel not in others]


def kernel_sources_hash(kernel=None):
    h = hashlib.sha256()
    for rel in kernel_sources(kernel):
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def read_summary(path):
    """'- key: value' lines of a summary file as a dict."""
    out = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                out[k.strip()] = v.strip()
    return out


def stats_table(path, per=1.0, top=40, per_kernel=None):
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    if per_kernel:
        per = float(sum(int(r["Calls"]) for r in rows if per_kernel in r["Name"]))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = ["| kernel | calls | calls/step | avg us | min us | max us | share |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows[:top]:
        name = r["Name"].replace("|", "/")
        if len(name) > 160:  # template-heavy library kernels: the head of the name says which
            name = name[:157] + "..."
        calls = int(r["Calls"])
        lines.append(f"| `{name}` | {calls} | {calls / per:.2f} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{100.0 * float(r['TotalDurationNs']) / total:.1f}% |")
    lines.append(f"\nTotal GPU kernel time: {total / 1e6:.3f} ms over {sum(int(r['Calls']) for r in rows)} launches.")
    return "\n".join(lines)


def _dispatches(path):
    d = {}
    for r in csv.DictReader(open(path)):
        i = int(r["Dispatch_Id"])
        d.setdefault(i, {"name": r["Kernel_Name"], "vals": {}})
        d[i]["vals"][r["Counter_Name"]] = float(r["Counter_Value"])
    return d


def _split(path, counter, kernel):
    """The measured kernel's dispatches after the calibration copy (bench.py's scalar
    multiply, a MulFunctor elementwise kernel: the last one in the run), and the copy."""
    disp = _dispatches(path)
    ids = sorted(disp)
    calib = [i for i in ids if disp[i]["name"].startswith("void at::native") and "MulFunctor" in disp[i]["name"]]
    if not calib:
        raise SystemExit(f"{path}: no calibration dispatch (a PyTorch multiply kernel)")
    c = calib[-1]
    targets = [i for i in ids if i > c and kernel in disp[i]["name"]]
    if not targets:
        raise SystemExit(f"{path}: no dispatch of a kernel containing {kernel!r} after the calibration copy")
    vals = [disp[i]["vals"][counter] for i in targets]
    return disp[targets[0]]["name"], vals, disp[c]["name"], disp[c]["vals"][counter]


def traffic_summary(fetch_csv, write_csv, kernel, copy_bytes, algorithmic_bytes):
    name, fetch, cname, cfetch = _split(fetch_csv, "FETCH_SIZE", kernel)
    _, write, _, cwrite = _split(write_csv, "WRITE_SIZE", kernel)
    f_scale = copy_bytes / (cfetch * 1024.0)
    w_scale = copy_bytes / (cwrite * 1024.0)
    fetch_kib = sum(fetch) / len(fetch)
    write_kib = sum(write) / len(write)
    bytes_per = (fetch_kib * f_scale + write_kib * w_scale) * 1024.0
    return {
        "kernel": name,
        "launches": f"{len(fetch)} (fetch pass), {len(write)} (write pass)",
        "FETCH_SIZE per launch, KiB raw": f"{fetch_kib:.2f}",
        "WRITE_SIZE per launch, KiB raw": f"{write_kib:.2f}",
        "calibration kernel": cname[:80],
        "calibration bytes read and written": f"{copy_bytes}",
        "calibration FETCH_SIZE, KiB": f"{cfetch:.2f}",
        "calibration WRITE_SIZE, KiB": f"{cwrite:.2f}",
        "fetch scale": f"{f_scale:.5f}",
        "write scale": f"{w_scale:.5f}",
        "bytes per launch": f"{bytes_per:.0f}",
        "algorithmic bytes per launch": f"{algorithmic_bytes}",
        "traffic / algorithmic": f"{bytes_per / algorithmic_bytes:.4f}",
        "kernel sources sha256[:16]": kernel_sources_hash(name),
        "kernel sources hashed": " ".join(kernel_sources(name)),
    }


def counter_summary(paths, kernel):
    vals, name, n = {}, None, 0
    for path in paths:
        disp = _dispatches(path)
        ids = [i for i in sorted(disp) if kernel in disp[i]["name"]]
        if not ids:
            raise SystemExit(f"{path}: no dispatch of a kernel containing {kernel!r}")
        name = disp[ids[0]]["name"]
        n = max(n, len(ids))
        for c in disp[ids[0]]["vals"]:
            vals[c] = sum(disp[i]["vals"][c] for i in ids) / len(ids)
    out = {"kernel": name[:120], "dispatches per pass": str(n)}
    out.update({f"{c} per dispatch": f"{v:.6g}" for c, v in sorted(vals.items())})
    if vals.get("SQ_LDS_IDX_ACTIVE"):
        if "SQ_LDS_BANK_CONFLICT" in vals:
            out["bank-conflict cycles / LDS-active cycles"] = f"{vals['SQ_LDS_BANK_CONFLICT'] / vals['SQ_LDS_IDX_ACTIVE']:.4f}"
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--per", type=float, default=1.0)
    s.add_argument("--per-kernel", default=None, help="divide call counts by this kernel's call count")
    s.add_argument("--title", default="Kernel statistics")
    s.add_argument("--command", action="append", default=[])
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--algorithmic-bytes", type=int, required=True)
    t.add_argument("--title", default="Memory traffic per launch")
    t.add_argument("--command", action="append", default=[])
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--title", default="Hardware counters per dispatch")
    c.add_argument("--command", action="append", default=[])
    a = ap.parse_args(argv)
    out = [f"# {a.title}", ""]
    if a.command:
        out += ["Made with:", "", "```"] + a.command + ["```", ""]
    if a.cmd == "stats":
        out.append(stats_table(a.csv, a.per, per_kernel=a.per_kernel))
    elif a.cmd == "counters":
        out += [f"- {k}: {v}" for k, v in counter_summary(a.csv, a.kernel).items()]
    else:
        vals = traffic_summary(a.fetch, a.write, a.kernel, a.copy_bytes, a.algorithmic_bytes)
        out += [f"- {k}: {v}" for k, v in vals.items()]
    sys.stdout.write("\n".join(out) + "\n")


if __name__ == "__main__":
    main()
