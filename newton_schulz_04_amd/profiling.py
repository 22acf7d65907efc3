"""Turn rocprofv3 output of bench.py runs into the short summaries kept in
profiles/ (host-side parsing only; nothing here touches the GPU).

    python -m newton_schulz_04_amd.profiling stats KERNEL_STATS_CSV OUT_MD --command "..."
    python -m newton_schulz_04_amd.profiling traffic FETCH_CSV WRITE_CSV OUT_JSON --command "..."

`stats` reads the kernel statistics that `rocprofv3 --kernel-trace --stats`
writes and tabulates the per-kernel average durations.

`traffic` reads two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of
`bench.py --copy-probe` (counter values in KiB per dispatch). The copy probe
is one plain device-to-device copy of COPY_PROBE_BYTES; the ratio of its known
size to what each counter reads for it is the scale applied to every other
kernel's reading. The result is keyed by a hash of the library sources so
that bench.py can tell when the counters no longer describe the kernels.
"""
import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re

COPY_PROBE_BYTES = 1 << 30
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
# GEMM stage template argument -> the name bench.py reports it under
GEMM_KINDS = {"0": "syrk", "1": "poly", "2": "update"}


def source_hash():
    """sha256 over the library's sources (kernels, planner, launch code)."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if os.path.splitext(path)[1] in (".hip", ".cpp", ".h"):
            h.update(os.path.basename(path).encode())
            with open(path, "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def kernel_kind(name):
    """Short name of a kernel from its (demangled or mangled) name."""
    m = (re.search(r"k_gemm<\s*\d+\s*,\s*(\d+)\s*>", name) or
         re.search(r"k_gemmI(?:Li\d+E|DF16b|f)Li(\d+)E", name))
    if m:
        return GEMM_KINDS.get(m.group(1), "gemm" + m.group(1))
    for short in ("k_norm_partial", "k_norm_final", "k_prep", "k_small", "k_scale_out"):
        if short in name:
            return short[2:]
    if "copy" in name.lower():
        return "copy_probe"
    return None


def _per_dispatch(path, counter):
    vals = collections.defaultdict(list)
    with open(path) as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            kind = kernel_kind(row["Kernel_Name"])
            if kind is None:
                continue
            if kind == "copy_probe" and "copy" not in row["Kernel_Name"].lower():
                continue
            vals[kind].append(float(row["Counter_Value"]))
    return vals


def traffic(fetch_csv, write_csv, command):
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    # the probe is the largest copy dispatch in each run
    kib = COPY_PROBE_BYTES / 1024
    probe_f = max(fetch.pop("copy_probe", [0.0]))
    probe_w = max(write.pop("copy_probe", [0.0]))
    if probe_f <= 0 or probe_w <= 0:
        raise SystemExit("no copy-probe dispatch found: run bench.py with --copy-probe")
    sf, sw = kib / probe_f, kib / probe_w
    kernels = {}
    for kind in sorted(set(fetch) | set(write)):
        f = fetch.get(kind, [])
        w = write.get(kind, [])
        fb = sum(f) / len(f) * 1024 * sf if f else None
        wb = sum(w) / len(w) * 1024 * sw if w else None
        kernels[kind] = {"dispatches": max(len(f), len(w)),
                         "fetch_bytes": round(fb) if fb is not None else None,
                         "write_bytes": round(wb) if wb is not None else None,
                         "bytes": round(fb + wb) if fb is not None and wb is not None else None}
    return {"source_sha256": source_hash(), "command": command,
            "copy_probe": {"bytes": COPY_PROBE_BYTES, "fetch_kib": probe_f, "write_kib": probe_w,
                           "fetch_scale": round(sf, 4), "write_scale": round(sw, 4)},
            "kernels": kernels}


def stats_md(stats_csv, command):
    rows = []
    with open(stats_csv) as f:
        for row in csv.DictReader(f):
            rows.append(row)
    def col(row, *names):
        for n in names:
            if n in row:
                return row[n]
        raise KeyError(f"none of {names} in {sorted(row)}")
    lines = ["| kernel | calls | avg (ms) | min (ms) | max (ms) | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = col(r, "Name", "KERNEL_NAME", "Kernel_Name")
        kind = kernel_kind(name) or name[:40]
        avg = float(col(r, "AverageNs", "AVERAGE (nsec)")) / 1e6
        lo = float(col(r, "MinNs", "MIN (nsec)")) / 1e6
        hi = float(col(r, "MaxNs", "MAX (nsec)")) / 1e6
        share = float(col(r, "Percentage", "PERCENT (INC)"))
        lines.append(f"| {kind} | {col(r, 'Calls', 'CALLS')} | {avg:.4f} | {lo:.4f} | {hi:.4f} | {share:.1f}% |")
    return "\n".join(["Command:", "", "    " + command, ""] + lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("out")
    t.add_argument("--command", required=True)
    a = ap.parse_args()
    if a.what == "stats":
        with open(a.out, "w") as f:
            f.write(stats_md(a.csv, a.command))
    else:
        with open(a.out, "w") as f:
            json.dump(traffic(a.fetch_csv, a.write_csv, a.command), f, indent=1)
            f.write("\n")


if __name__ == "__main__":
    main()
