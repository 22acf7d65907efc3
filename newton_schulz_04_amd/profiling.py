"""Turn rocprofv3 output of bench.py runs into the short summaries kept in
profiles/ (host-side parsing only; nothing here touches the GPU).

    python -m newton_schulz_04_amd.profiling stats KERNEL_STATS_CSV OUT_MD --command "..."
    python -m newton_schulz_04_amd.profiling traffic FETCH_CSV WRITE_CSV OUT_JSON --command "..."
    python -m newton_schulz_04_amd.profiling summary KERNEL_STATS_CSV TRAFFIC_JSON BENCH_JSON OUT_MD --title ... --command "..."
        [--mfma-csv MFMA_COUNTERS_CSV --mfma-command "..."]

`stats` reads the kernel statistics that `rocprofv3 --kernel-trace --stats`
writes and tabulates the per-kernel average durations.

The optional MFMA counter run (`rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES
SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE`) gives each GEMM's MFMA utilisation (busy
cycles of the 4 matrix units per compute unit over the compute units' busy
cycles) and its average shader clock (GRBM_GUI_ACTIVE counts per XCD).

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
XCDS = 8
SIMDS_PER_CU = 4


# The sources whose changes can change what the counters measure: the
# kernels, and the planner that orders their tiles and lays out the workspace.
TRAFFIC_SOURCES = ("ns_kernels.hip", "ns_internal.h", "ns_plan.cpp", "ns_plan.h")


def code_only(text):
    """C/C++ source without its comments and with whitespace runs collapsed:
    what the compiler sees, so that an edit to a comment does not count as a
    change of the kernels. (The hashed sources hold no comment markers inside
    string literals.)"""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash():
    """sha256 over the code (comments excluded) of the kernel and planner
    sources (TRAFFIC_SOURCES)."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if os.path.basename(path) in TRAFFIC_SOURCES:
            h.update(os.path.basename(path).encode())
            with open(path, encoding="utf-8") as f:
                h.update(code_only(f.read()).encode())
    return h.hexdigest()


def kernel_kind(name):
    """Short name of a kernel from its (demangled or mangled) name."""
    # k_gemm<dtype, stage, last, split>: a split launch (whole tiles, then
    # the half tiles of the last round) is the whole stage, the same kind
    m = (re.search(r"k_gemm<\s*\d+\s*,\s*(\d+)\s*(?:,\s*\d+\s*)?(?:,\s*(\d+)\s*)?>", name) or
         re.search(r"k_gemmI(?:Li\d+E|DF16b|f)Li(\d+)E(?:Li\d+E)?(?:Li(\d+)E)?", name))
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
    return {"source_sha256": source_hash(),
            "source_hash_of": "the code of " + ", ".join(TRAFFIC_SOURCES) + " without comments (code_only)",
            "command": command,
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


def algorithmic_bytes(shapes, elt=2):
    """Bytes each kernel must move per launch over a batch of large bf16
    matrices (m = min dim, n = max dim): what the definition reads and
    writes, with no re-reads. X moves as X_hi + X_lo (2 + 2 bytes)."""
    out = collections.Counter()
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        out["syrk read"] += 2 * n * m            # X_hi
        out["syrk write"] += 2 * m * m           # A
        out["poly read"] += 2 * m * m            # A
        out["poly write"] += 2 * m * m           # B
        out["update read"] += 2 * m * m + 4 * n * m   # B, X_hi, X_lo
        out["update write"] += 4 * n * m         # X_hi, X_lo (next step)
        out["prep read"] += elt * n * m
        out["prep write"] += 4 * n * m
        out["norm_partial read"] += elt * n * m
    return out


def mfma_table(mfma_csv):
    """Per GEMM kind: MFMA utilisation and shader clock, averaged over its
    dispatches in the counter run."""
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    span = {}
    with open(mfma_csv) as f:
        for row in csv.DictReader(f):
            kind = kernel_kind(row["Kernel_Name"])
            if kind not in ("syrk", "poly", "update"):
                continue
            key = (kind, row["Dispatch_Id"])
            acc[key][row["Counter_Name"]].append(float(row["Counter_Value"]))
            span[key] = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-9
    per_kind = collections.defaultdict(list)
    for (kind, _), c in acc.items():
        busy = sum(c["SQ_BUSY_CU_CYCLES"])
        mfma = sum(c["SQ_VALU_MFMA_BUSY_CYCLES"])
        grbm = sum(c["GRBM_GUI_ACTIVE"])
        if busy <= 0 or span[(kind, _)] <= 0:
            continue
        per_kind[kind].append((mfma / (SIMDS_PER_CU * busy), grbm / XCDS / span[(kind, _)] / 1e9))
    rows = ["| kernel | dispatches | MFMA busy | shader clock (GHz) |", "|---|---|---|---|"]
    for kind in ("syrk", "poly", "update"):
        v = per_kind.get(kind)
        if v:
            u = sum(x[0] for x in v) / len(v)
            g = sum(x[1] for x in v) / len(v)
            rows.append(f"| {kind} | {len(v)} | {100 * u:.1f}% | {g:.2f} |")
    return "\n".join(rows)


def summary_md(stats_csv, traffic_json, bench_json, title, shapes, kt_command, mfma_csv=None, mfma_command=None):
    with open(traffic_json) as f:
        t = json.load(f)
    with open(bench_json) as f:
        b = json.loads(f.read().strip().splitlines()[-1])
    alg = algorithmic_bytes(shapes)
    ks = {k: v["ms_avg"] for k, v in b["kernels"].items()}
    rows = ["| kernel | fetch (GB/launch) | write (GB/launch) | algorithmic read / write (GB) | fetch + write per launch time |",
            "|---|---|---|---|---|"]
    for k in ("update", "syrk", "poly", "prep", "norm_partial"):
        e = t["kernels"].get(k)
        if not e:
            continue
        rate = ""
        if ks.get(k):
            rate = f"{(e['fetch_bytes'] + e['write_bytes']) / (ks[k] * 1e-3) / 1e12:.2f} TB/s"
        rows.append(f"| {k} | {e['fetch_bytes'] / 1e9:.2f} | {e['write_bytes'] / 1e9:.2f} | "
                    f"{alg[k + ' read'] / 1e9:.2f} / {alg[k + ' write'] / 1e9:.2f} | {rate} |")
    mfma = ""
    if mfma_csv:
        mfma = f"""
## MFMA utilisation (rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE)

    {mfma_command}

{mfma_table(mfma_csv)}

The bf16 MFMA peak assumes 2.4 GHz; the shader clock under this load is what
the power limit leaves. syrk and poly compute only the upper-triangle tiles
(300 of 576 per 6144 x 6144 output), so their metric TFLOP/s count about
twice the MFMA work they do; bench.py reports `tflops_tiles` (what the MFMAs
execute) beside it.
"""
    cp = t["copy_probe"]
    gc = b.get("gpu_clock") or {}
    clock = ""
    if gc.get("gfxclk_mhz"):
        clock = (f" Under the profiler the AMD SMI library read the XCD clocks at "
                 f"{gc['gfxclk_mhz']:.0f} MHz (per XCD {gc.get('gfxclk_mhz_per_xcd')}) and the socket at "
                 f"{gc.get('socket_power_w')} W against a {gc.get('power_cap_w')} W cap over the timed pass.")
    return f"""# {title}

One bench step = one `ns_orthogonalize_batched` call over the batch: norm_partial,
norm_final, prep, then 5 x (syrk = `k_gemm<0, 0, 0, s>` X X^T, poly = `k_gemm<0, 1, 0, s>`
bA + cA^2, update = `k_gemm<0, 2, 0, 0>` aX + BX; the fifth update is `k_gemm<0, 2, 1, 0>`,
which writes the caller's buffer; s = 1 when the stage's last round is split,
its half tiles running after the whole tiles in the same launch). `copy_probe` rows are the runtime's
device copies (bench restores its inputs from a pristine copy before the timed
pass and before the profiling pass, outside both).
Run from the repository root with `export TMPDIR=/tmp` and the library built
in-tree (`python -c "import __graft_entry__ as g; g.build()"`).

## Kernel trace (rocprofv3 --kernel-trace --stats)

{stats_md(stats_csv, kt_command)}
The same run's bench line: value {b['value']} matrices/s (timed pass, no events),
{b['tflops']} TFLOP/s ({b['pct_bf16_peak']}% of 2.5 PFLOP/s, the metric's 4m^2n + 2m^3
convention; executed by the kernels: {b.get('executed', {}).get('tiles_tflops')} TFLOP/s); per-launch ms from
HIP events on the launch stream in bench.py's separate profiling pass:
{", ".join(f"{k} {v}" for k, v in ks.items())}.{clock}

## HBM-side traffic (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)

    {t['command']}

The 1 GiB copy probe reads FETCH_SIZE = {cp['fetch_kib']:.0f} KiB and WRITE_SIZE =
{cp['write_kib']:.0f} KiB, so fetch readings are scaled by {cp['fetch_scale']} and write readings by
{cp['write_scale']}. FETCH_SIZE counts L2 misses, whether the Infinity Cache or HBM serves
them. Per launch, averaged over a step's dispatches (the last update writes the
caller's buffer instead of X_hi and X_lo):

{chr(10).join(rows)}

The record, keyed by a hash of the code of the kernel and planner sources
(comments excluded), is `{os.path.basename(traffic_json)}`; bench.py reports
the dominant kernel's bytes as `roofline.traffic` only while the hash matches. prep and norm_partial are the HBM-bound passes (peak 8 TB/s).
{mfma}"""


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    m = sub.add_parser("summary")
    m.add_argument("stats_csv")
    m.add_argument("traffic_json")
    m.add_argument("bench_json")
    m.add_argument("out")
    m.add_argument("--title", required=True)
    m.add_argument("--shape", default="8192x6144")
    m.add_argument("--count", type=int, default=8)
    m.add_argument("--command", required=True)
    m.add_argument("--mfma-csv")
    m.add_argument("--mfma-command")
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
    if a.what == "summary":
        r, c = (int(v) for v in a.shape.split("x"))
        with open(a.out, "w") as f:
            f.write(summary_md(a.stats_csv, a.traffic_json, a.bench_json, a.title, [(r, c)] * a.count,
                               a.command, a.mfma_csv, a.mfma_command))
    elif a.what == "stats":
        with open(a.out, "w") as f:
            f.write(stats_md(a.csv, a.command))
    else:
        with open(a.out, "w") as f:
            json.dump(traffic(a.fetch_csv, a.write_csv, a.command), f, indent=1)
            f.write("\n")


if __name__ == "__main__":
    main()
