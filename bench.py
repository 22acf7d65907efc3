"""Throughput of batched Newton-Schulz orthogonalization on one MI355X.

Default workload: 8 bf16 matrices of 8192x6144, each rank-64 plus 1e-3 noise
(seeded), 5 quintic steps per matrix. One "step" of this benchmark is one
ns_orthogonalize_batched call over the whole 8-matrix batch: norm,
normalize/transpose, 5 x (X X^T, bA + cA^2, aX + BX), write-back.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Workloads: dense_lowrank (default), ragged_remainder_R (R of the remainder
pool's 8192x6144 matrices, the last one passed through 64 row shards),
dense_lowrank_fp32 (the default's matrices through the fp32 path, fp32 MFMA),
moe_mixed (130 matrices of four shapes), attn_gate (32 x 18x2304 passed as 8
padded row shards each) and tiny_fp32 (4 x 64x32 fp32). The last two run in
the small-matrix kernel, which evaluates the iteration through the m x m Gram
matrix in fp64 (vector FMAs for the Gram matrix and the final product, fp64
MFMAs for the m x m steps); its roofline is taken against the 78.6 TFLOP/s
fp64 peak.

Prints one JSON line. `value` is matrices per second with the inputs already
resident in HBM. Every timed step works on its own resident copy of the batch
(all restored from a pristine copy before the timed region), so no step
reuses an output. The timed pass runs without the library's profiling events;
per-kernel times (`kernels`, `roofline`) come from a separate pass of
min(steps, 5) calls on fresh copies.

`gpu_clock`: the graphics clock of each XCD and the socket power as the AMD
SMI library reports them (the firmware's gpu_metrics table, refreshed every
few hundred ms), sampled by a host thread through the warm-up and timed
passes; the medians over the samples taken in the timed pass, the power cap,
and the dominant kernel's roofline fraction against the peak scaled to that
clock. Null where the library or the device is not available.

FLOP conventions, reported side by side:
  tflops / pct_bf16_peak        the metric's convention, 5 (4 m^2 n + 2 m^3)
                                per matrix, m = min dim: X X^T and A^2 counted
                                as full products
  executed.algorithmic          5 (3 m^2 n + m^3): the symmetric products at
                                half cost, as the kernels compute them
  executed.tiles                what the MFMAs execute: 2 * 256^2 * K per
                                output tile (upper tiles for the symmetric
                                stages), padding included
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NS-orthogonalized matrices/s + TFLOP/s (% bf16 MFMA peak), 8192x6144 bf16"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 MFMA (the fp32 tiled path)
PEAK_FP64_TFLOPS = 78.6   # MI355X fp64, vector and MFMA alike (the small-matrix path)
PEAK_CLOCK_MHZ = 2400.0   # the clock the peaks above assume
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def make_workload(name):
    import torch
    from newton_schulz_04_amd import workloads as wl
    if name == "dense_lowrank":
        mats = [wl.dense_lowrank_matrix(i) for i in range(wl.DENSE_COUNT)]
        desc = {"workload": "dense_lowrank", "matrices": 8, "shape": [8192, 6144],
                "dtype": "bf16", "input": "rank-64 L@R + 1e-3*N(0,1), seed 2", "ns_steps": 5}
    elif name == "dense_lowrank_fp32":
        # the same matrices (their bf16 values, exactly) through the fp32 path
        mats = [wl.dense_lowrank_matrix(i).float() for i in range(wl.DENSE_COUNT)]
        desc = {"workload": "dense_lowrank_fp32", "matrices": 8, "shape": [8192, 6144],
                "dtype": "fp32", "input": "rank-64 L@R + 1e-3*N(0,1), seed 2, as fp32", "ns_steps": 5}
    elif name.startswith("ragged_remainder_"):
        r = int(name.rsplit("_", 1)[1])
        mats = [c.mat for c in wl.ragged_remainder(r, world=64, padded=True)]
        desc = {"workload": name, "matrices": r, "shape": [8192, 6144], "dtype": "bf16",
                "input": "N(0,1), seed 3", "ns_steps": 5}
    elif name == "attn_gate":
        # the 32 attention-gate matrices of 18 x 2304, each passed as its 8
        # row shards padded to 3 rows (24 x 2304, rows 18..23 zero)
        cases = wl.attn_gate()
        mats = [c.mat for c in cases]
        desc = {"workload": "attn_gate", "matrices": len(mats), "shape": [24, 2304], "real_shape": [18, 2304],
                "dtype": "bf16", "input": "0.02*N(0,1), seed 1, 8 row shards (3,3,3,3,3,3,0,0) padded to 3 rows",
                "ns_steps": 5}
    elif name == "tiny_fp32":
        mats = [c.mat for c in wl.tiny_fp32()]
        desc = {"workload": "tiny_fp32", "matrices": len(mats), "shape": [64, 32], "dtype": "fp32",
                "input": "N(0,1), seed 0, matrix 3 rows 56..63 zero", "ns_steps": 5}
    elif name == "moe_mixed":
        g = torch.Generator(device="cuda").manual_seed(4)
        mats = [torch.randn(s, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
                for s in wl.moe_mixed_shapes()]
        desc = {"workload": "moe_mixed", "matrices": len(mats), "dtype": "bf16",
                "input": "N(0,1) drawn on the GPU (timing only)", "ns_steps": 5}
    else:
        raise SystemExit(f"unknown workload {name}")
    return mats, desc


def cpu_baseline(sample_rows=6144, sample_cols=4608):
    """The fp64 oracle, as it stands, on a bounded sample of the workload: one
    Newton-Schulz step on the top-left sample_rows x sample_cols block of
    matrix 0. Scaled to matrices/s by metric FLOPs (an optimistic scaling for
    the CPU: the oracle gets slower, not faster, at the full size)."""
    import numpy as np
    from newton_schulz_04_amd import workloads as wl
    from oracle import oracle
    g = wl.dense_lowrank_matrix(0)[:sample_rows, :sample_cols].float().numpy()
    m, n = min(g.shape), max(g.shape)
    flops = 4 * m * m * n + 2 * m ** 3
    t0 = time.time()
    oracle.newton_schulz(g, steps=1, coeffs=oracle.QUINTIC)
    dt = time.time() - t0
    per_matrix = wl.flops_per_matrix(*wl.DENSE_SHAPE)
    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    return {"value": round(flops / dt / per_matrix, 6), "unit": "matrices/s", "cores": cores,
            "kind": "oracle", "gflops_fp64": round(flops / dt / 1e9, 3), "seconds": round(dt, 2),
            "sample": f"1 NS step of the top-left {sample_rows}x{sample_cols} block of matrix 0 "
                      f"(fp64, plain loops + OpenMP), scaled by metric FLOPs to 8192x6144 x 5 steps"}


def cpu_baseline_small(mats, real_shape=None):
    """The fp64 oracle, as it stands, on the whole batch of a small-matrix
    workload (milliseconds of CPU work per matrix)."""
    from newton_schulz_04_amd import workloads as wl
    from oracle import oracle
    t0 = time.time()
    for g in mats:
        oracle.newton_schulz(g.float().numpy(), steps=5, coeffs=oracle.QUINTIC)
    dt = time.time() - t0
    flops = sum(wl.flops_per_matrix(*(real_shape or tuple(g.shape))) for g in mats)
    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    return {"value": round(len(mats) / dt, 3), "unit": "matrices/s", "cores": cores, "kind": "oracle",
            "gflops_fp64": round(flops / dt / 1e9, 3), "seconds": round(dt, 3),
            "sample": f"the whole batch ({len(mats)} matrices, 5 steps each)"}


class GpuClockSampler:
    """Graphics clock per XCD and socket power of the GPU that torch calls
    cuda:0, from the AMD SMI library's gpu_metrics table, sampled every
    `period` seconds by a host thread (reads only: no GPU work, no HIP calls).
    The firmware refreshes the table every few hundred ms, so a sample is the
    latest snapshot. `mark()` opens the window the summary covers."""

    def __init__(self, period=0.02):
        import threading
        self.period = period
        self.samples = []
        self.t_mark = None
        self.error = None
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            import torch
            self._smi = amdsmi
            amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
            props = torch.cuda.get_device_properties(0)
            want = (int(getattr(props, "pci_domain_id", 0)), int(props.pci_bus_id), int(props.pci_device_id))
            self._handle = None
            for h in amdsmi.amdsmi_get_processor_handles():
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)   # "dddd:bb:dd.f"
                dom, bus, rest = bdf.split(":")
                if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    self._handle = h
            if self._handle is None:
                raise RuntimeError(f"no SMI device at PCI {want}")
            cap = amdsmi.amdsmi_get_power_cap_info(self._handle).get("power_cap")
            self.power_cap_w = cap / 1e6 if isinstance(cap, (int, float)) else None
        except Exception as e:  # the figure is optional: report why it is missing
            self.error = f"{type(e).__name__}: {e}"

    def _run(self):
        import time as _t
        while not self._stop.is_set():
            t = _t.perf_counter()
            try:
                m = self._smi.amdsmi_get_gpu_metrics_info(self._handle)
                clks = [v for v in (m.get("current_gfxclks") or []) if isinstance(v, (int, float))]
                pw = m.get("current_socket_power")
                self.samples.append((t, clks, pw if isinstance(pw, (int, float)) else None))
            except Exception as e:
                self.error = f"{type(e).__name__}: {e}"
                return
            self._stop.wait(self.period)

    def start(self):
        import threading
        if self.error is None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def mark(self):
        self.t_mark = time.perf_counter()

    def stop(self, t_end):
        if self._thread is not None:
            self._stop.set()
            self._thread.join(timeout=5)
        try:
            self._smi.amdsmi_shut_down()
        except Exception:
            pass
        win = [x for x in self.samples if self.t_mark is not None and self.t_mark <= x[0] <= t_end]
        note = None
        if not win and self.t_mark is not None:
            # a pass shorter than the sampling period: the snapshot in effect
            # when it began
            before = [x for x in self.samples if x[0] < self.t_mark]
            win = before[-1:]
            note = "timed pass shorter than the sampling period: the last sample before it"
        if self.error is not None or not win:
            return {"error": self.error or "no sample before the end of the timed pass"}
        import statistics
        mean_clk = [statistics.fmean(c) for _, c, _ in win if c]
        per_xcd = [statistics.median(v) for v in zip(*[c for _, c, _ in win if c])]
        power = [p for _, _, p in win if p is not None]
        return {
            "source": "AMD SMI gpu_metrics (current_gfxclks, current_socket_power)",
            "samples": len(win),
            "gfxclk_mhz": round(statistics.median(mean_clk), 1) if mean_clk else None,
            "gfxclk_mhz_per_xcd": [round(v) for v in per_xcd],
            "socket_power_w": round(statistics.median(power), 1) if power else None,
            "power_cap_w": self.power_cap_w,
            **({"note": note} if note else {}),
        }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def tile_flops_per_kind(shapes, dtype):
    """MFMA FLOPs one launch of each GEMM stage executes over the batch, from
    the library's own tile lists (2 * 256^2 * K per tile)."""
    import newton_schulz_04_amd as ns
    f = {}
    for kind, stage in (("syrk", 0), ("poly", 1), ("update", 2)):
        tiles, edge = ns.plan_tiles(shapes, dtype, stage)
        f[kind] = int(sum(2 * edge * edge * int(t[3]) for t in tiles))
    return f


def small_executed_flops(shapes, steps=5):
    """fp64 FLOPs the small-matrix kernel executes per call: per matrix (m =
    min dim rounded up to 8 rows, n columns) the norm's m n FMAs, the Gram
    matrix's m^2 n, the final product's m^2 n, and in every 512-column slice
    the steps' 32 x 32 products (4 steps - 3 of them, 32^3 FMAs each; every
    slice runs them, for n <= 131072)."""
    total = 0
    nprod = 4 * steps - 3 if steps > 0 else 0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        if m == 0:
            continue
        mr = -(-m // 8) * 8
        slices = -(-n // 512)
        total += 2 * (mr * n + 2 * mr * mr * n + slices * nprod * 32 ** 3)
    return total


def pass_bytes(shapes, elt):
    """Algorithmic HBM bytes of one launch of the norm and normalize passes:
    the norm reads G; normalize reads G and writes the padded X^T (bf16: X_hi
    and X_lo, 2 x 2 bytes; fp32: X^T and X, 2 x 4 bytes per element)."""
    norm = prep = 0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        if m <= 32:
            continue
        mp, np_ = -(-m // 256) * 256, -(-n // 256) * 256
        norm += r * c * elt
        prep += r * c * elt + mp * np_ * 2 * elt
    return {"norm_partial": norm, "prep": prep}


def metric_flops_per_kind(shapes):
    """Metric FLOPs of one launch of each GEMM stage over the batch (each
    product counted in full: X X^T 2m^2n, A A 2m^3, B X 2m^2n), and the
    symmetric-aware algorithmic FLOPs (X X^T m^2 n, A A m^3, B X 2 m^2 n)."""
    f = {"syrk": 0, "poly": 0, "update": 0}
    a = {"syrk": 0, "poly": 0, "update": 0}
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        if m <= 32 or m == 0:
            continue
        f["syrk"] += 2 * m * m * n
        f["poly"] += 2 * m ** 3
        f["update"] += 2 * m * m * n
        a["syrk"] += m * m * n
        a["poly"] += m ** 3
        a["update"] += 2 * m * m * n
    return f, a


def accuracy_vs_stored_oracle(workload, mats_cpu, outputs):
    """Relative error of this run's results against the stored fp64 oracle
    samples of the workload (tests/golden/oracle_<workload>_<i>.npz, written
    by tests/golden/make_oracle_golden.py): per sampled matrix, over its
    stored rows and columns. Only the data files are read; None when the
    workload has no stored sample or an input's hash differs."""
    import numpy as np
    from newton_schulz_04_amd import workloads as wl
    base = {"dense_lowrank": "dense_lowrank"}.get(workload)
    if workload.startswith("ragged_remainder_"):
        base = "ragged_remainder"
    if base is None or mats_cpu is None:
        return None
    out = {}
    for i, (g, y) in enumerate(zip(mats_cpu, outputs)):
        path = os.path.join(ROOT, "tests", "golden", f"oracle_{base}_{i}.npz")
        if not os.path.exists(path):
            continue
        with np.load(path, allow_pickle=False) as z:
            if str(z["input_sha256"]) != wl.sha256(g):
                continue
            yf = y.float().cpu().numpy().astype(np.float64)
            rows, ref = z["rows_idx"], z["rows"].astype(np.float64)
            num, den = np.linalg.norm(yf[rows] - ref) ** 2, np.linalg.norm(ref) ** 2
            if "cols_idx" in z.files:
                cols, refc = z["cols_idx"], z["cols"].astype(np.float64)
                num += np.linalg.norm(yf[:, cols] - refc) ** 2
                den += np.linalg.norm(refc) ** 2
            out[f"matrix_{i}"] = float(np.sqrt(num / den))
    if not out:
        return None
    return {"max_rel_err": max(out.values()), "per_matrix": out,
            "against": "stored fp64 oracle rows and columns (tests/golden)", "tolerance": 2e-2}


def measured_traffic(workload, kind):
    """HBM bytes per launch of `kind` from the committed PMC summary of this
    workload, or None when there is none or the library sources changed since
    the counters were taken."""
    from newton_schulz_04_amd.profiling import source_hash
    path = os.path.join(ROOT, "profiles", f"k_gemm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != source_hash():
        log("traffic: PMC summary predates the current sources; reporting null")
        return None
    entry = rec.get("kernels", {}).get(kind)
    return entry.get("bytes") if entry else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dense_lowrank")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one plain 1 GiB device copy first (calibrates PMC byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        log("only --gpus 1 is supported: the batched Newton-Schulz path runs on one GPU")
        sys.exit(2)

    import torch
    import newton_schulz_04_amd as ns
    from newton_schulz_04_amd import workloads as wl

    torch.cuda.set_device(0)
    if args.copy_probe:
        from newton_schulz_04_amd.profiling import COPY_PROBE_BYTES
        src = torch.ones(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy probe: {COPY_PROBE_BYTES} bytes device to device")
    log(f"library {ns.version()}; generating workload {args.workload}")
    mats, desc = make_workload(args.workload)
    shapes = [tuple(m.shape) for m in mats]
    # metric FLOPs on the real shape (the attention gate's 18 x 2304, not
    # its padded 24 x 2304)
    real = tuple(desc.get("real_shape", ())) or None
    flops_batch = sum(wl.flops_per_matrix(*(real or (r, c))) for r, c in shapes)
    small_batch = all(min(r, c) <= 32 for r, c in shapes)
    fp32 = all(m.dtype == torch.float32 for m in mats)
    elt = 4 if fp32 else 2
    cpu_mats = [m.clone() for m in mats] if small_batch else None
    # CPU copies of the inputs the stored oracle samples cover
    ref_inputs = [m.clone() for m in mats] if (args.workload == "dense_lowrank" or
                                               args.workload.startswith("ragged_remainder_")) else None
    h = hashlib.sha256()
    for m in mats:
        h.update(m.cpu().contiguous().view(torch.uint8).numpy().tobytes())
    input_sha = h.hexdigest()
    pristine = [m.cuda() for m in mats]
    del mats
    nbatch = max(1, args.steps)
    batches = [[p.clone() for p in pristine] for _ in range(nbatch)]
    torch.cuda.synchronize()
    log(f"{len(shapes)} matrices, {flops_batch / 1e12:.3f} TFLOP per step, {nbatch} resident copies")

    def restore(bs):
        for b in bs:
            for dst, src in zip(b, pristine):
                dst.copy_(src)
        torch.cuda.synchronize()

    sampler = GpuClockSampler()
    sampler.start()
    for w in range(args.warmup):
        ns.orthogonalize(batches[w % nbatch])
        torch.cuda.synchronize()
        log(f"warmup {w + 1}/{args.warmup} done")
    restore(batches)

    # timed pass: K calls, each on its own pristine copy, no profiling events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    sampler.mark()
    for k in range(args.steps):
        ns.orthogonalize(batches[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    gpu_clock = sampler.stop(t1)
    log(f"timed {args.steps} steps in {elapsed:.3f} s")

    # profiling pass: per-kernel HIP events on the call's stream
    nprof = min(args.steps, 5)
    restore(batches[:nprof])
    ns.profile_enable(True)
    for k in range(nprof):
        ns.orthogonalize(batches[k])
    torch.cuda.synchronize()
    ns.profile_enable(False)
    prof = ns.profile_read()
    log(f"profiling pass: {nprof} calls")

    per_kind, algo_kind = metric_flops_per_kind(shapes)
    tile_kind = tile_flops_per_kind(shapes, 1 if fp32 else 0)
    bytes_kind = pass_bytes(shapes, elt)
    kernels = {}
    for kind, (ms, n) in prof.items():
        if n == 0:
            continue
        avg = ms / n
        entry = {"ms_avg": round(avg, 4), "launches": n, "ms_total": round(ms, 3)}
        if kind in per_kind and per_kind[kind]:
            entry["tflops_metric"] = round(per_kind[kind] / (avg * 1e-3) / 1e12, 1)
            entry["tflops_algorithmic"] = round(algo_kind[kind] / (avg * 1e-3) / 1e12, 1)
            entry["tflops_tiles"] = round(tile_kind[kind] / (avg * 1e-3) / 1e12, 1)
        if kind in bytes_kind and bytes_kind[kind]:
            entry["gbs"] = round(bytes_kind[kind] / (avg * 1e-3) / 1e9, 1)
            entry["pct_hbm_peak"] = round(100 * bytes_kind[kind] / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 1)
        kernels[kind] = entry
    if small_batch:
        # the small-path kernel evaluates the iteration in fp64, in one launch
        # per phase: the metric FLOPs of the batch as passed per call over the
        # kernel time of a call, against the fp64 peak; beside it the fp64
        # FLOPs the kernel executes
        dom = "small"
        kernels[dom]["ms_per_call"] = round(kernels[dom]["ms_total"] / nprof, 4)
        call_s = kernels[dom]["ms_per_call"] * 1e-3
        achieved = sum(wl.flops_per_matrix(r, c) for r, c in shapes) / call_s / 1e12
        kernels[dom]["executed_fp64_tflops"] = round(small_executed_flops(shapes) / call_s / 1e12, 3)
        roofline = {"bound": "alu", "kernel": dom, "achieved": round(achieved, 3),
                    "peak": PEAK_FP64_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_FP64_TFLOPS, 5), "traffic": None}
    else:
        dom = max((k for k in kernels if k in per_kind), key=lambda k: kernels[k]["ms_total"])
        # the dominant kernel's algorithmic FLOPs per launch (for the update,
        # a full product, the same under every convention)
        achieved = algo_kind[dom] / (kernels[dom]["ms_avg"] * 1e-3) / 1e12
        peak = PEAK_FP32_MFMA_TFLOPS if fp32 else PEAK_BF16_TFLOPS
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                    "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4),
                    "traffic": measured_traffic(args.workload, dom)}
    ms_per_step = elapsed / args.steps * 1e3
    tflops = flops_batch / (elapsed / args.steps) / 1e12
    value = len(shapes) * args.steps / elapsed
    peak_main = PEAK_FP32_MFMA_TFLOPS if fp32 else PEAK_BF16_TFLOPS
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64" if small_batch else "f32" if fp32 else "bf16",
        "data": "synthetic",
        "config": desc,
        "tflops": round(tflops, 1),
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "flop_convention": "tflops and pct_bf16_peak count 5(4m^2n+2m^3) per matrix (the symmetric "
                           "products X X^T and A^2 as full GEMMs); executed.* give what the kernels compute",
        "roofline": roofline,
        "kernels": kernels,
        "input_sha256": input_sha,
        "host_cpu": cpu_model(),
    }
    if not small_batch:
        step_s = elapsed / args.steps
        algo = sum(5 * (3 * min(r, c) ** 2 * max(r, c) + min(r, c) ** 3) for r, c in shapes)
        tiles_all = sum(5 * v for v in tile_kind.values())
        out["executed"] = {
            "algorithmic_tflops": round(algo / step_s / 1e12, 1),
            "algorithmic_pct_peak": round(100 * algo / step_s / 1e12 / peak_main, 2),
            "tiles_tflops": round(tiles_all / step_s / 1e12, 1),
            "tiles_pct_peak": round(100 * tiles_all / step_s / 1e12 / peak_main, 2),
        }
    if gpu_clock.get("gfxclk_mhz"):
        # the roofline's peak scaled to the clock the chip sustained
        scaled = roofline["peak"] * gpu_clock["gfxclk_mhz"] / PEAK_CLOCK_MHZ
        gpu_clock["roofline_peak_at_this_clock"] = round(scaled, 1)
        gpu_clock["roofline_frac_at_this_clock"] = round(roofline["achieved"] / scaled, 4)
    out["gpu_clock"] = gpu_clock
    acc = accuracy_vs_stored_oracle(args.workload, ref_inputs, batches[args.steps - 1])
    if acc is not None:
        out["accuracy"] = acc
    if not args.no_cpu_baseline:
        try:
            log("timing the CPU oracle on a bounded sample")
            out["cpu_baseline"] = cpu_baseline_small(cpu_mats, real) if small_batch else cpu_baseline()
            out["cpu_baseline"]["cpu_model"] = cpu_model()
        except Exception as e:  # the oracle is optional for the GPU figure
            out["cpu_baseline"] = {"error": str(e)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
