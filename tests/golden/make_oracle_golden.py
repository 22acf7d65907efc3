"""Write stored oracle results for full-size workload matrices.

The fp64 oracle needs minutes per 8192x6144 matrix, too slow to run inside a
GPU test, so this script runs it once on a seeded sample of each large
workload's matrices and stores, per matrix:

  rows_idx, rows   one seeded output row from every 256-row band, plus the
                   first and the last row (fp32 values)
  cols_idx, cols   one seeded output column from every 256-column band, plus
                   the first and the last column (fp32 values)
  sketch           Y @ Omega, Omega a seeded (cols x 4) matrix of +-1 (fp64)
  fro              ||Y||_F (fp64)
  input_sha256     hash of the input bytes the oracle saw

A band of 256 is one output tile edge of the GPU library's GEMMs, so every
output tile of a sampled matrix has at least one stored row and one stored
column running through it.

Everything stored comes from oracle/ (the fp64 CPU oracle) applied to inputs
from newton_schulz_04_amd/workloads.py; nothing comes from the GPU library.

usage: python tests/golden/make_oracle_golden.py [name ...]
       (matrices whose file already holds the band samples are skipped)
"""
import os
import sys
import time
import zlib

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from newton_schulz_04_amd import workloads  # noqa: E402
from oracle import oracle  # noqa: E402

SKETCH_K = 4
BAND = 256


def omega(cols: int, seed: int) -> np.ndarray:
    return np.random.default_rng(seed).choice([-1.0, 1.0], size=(cols, SKETCH_K))


def band_sample(size: int, seed: int) -> np.ndarray:
    """One index drawn uniformly from every band of BAND indices (the last
    band may be short), plus 0 and size - 1, sorted and unique."""
    rng = np.random.default_rng(seed)
    pick = [lo + int(rng.integers(min(BAND, size - lo))) for lo in range(0, size, BAND)]
    return np.unique(np.concatenate([[0, size - 1], pick])).astype(np.int64)


def sampled_indices():
    """(name, generator, index) of every stored matrix; the sample of each
    workload is drawn with numpy default_rng(1000 + seed)."""
    out = []
    dense = np.random.default_rng(1002).choice(workloads.DENSE_COUNT, size=2, replace=False)
    for i in sorted(int(v) for v in dense):
        out.append((f"dense_lowrank_{i}", workloads.dense_lowrank_matrix, i))
    for i in (0, workloads.REMAINDER_POOL - 1):
        out.append((f"ragged_remainder_{i}", workloads.ragged_remainder_matrix, i))
    rng = np.random.default_rng(1004)
    start = 0
    for shape, count in workloads.MOE_GROUPS:
        i = start + int(rng.integers(count))
        out.append((f"moe_mixed_{i}", workloads.moe_mixed_matrix, i))
        start += count
    return out


def write_one(name, make, index):
    path = os.path.join(HERE, f"oracle_{name}.npz")
    if os.path.exists(path):
        with np.load(path, allow_pickle=False) as old:
            if "cols_idx" in old.files:
                print(f"{name}: exists with band samples, skipped", flush=True)
                return
    g = make(index)
    sha = workloads.sha256(g)
    t0 = time.time()
    y = oracle.newton_schulz(g.float().numpy(), steps=5, coeffs=oracle.QUINTIC)
    dt = time.time() - t0
    seed = zlib.crc32(name.encode())
    ridx = band_sample(y.shape[0], seed)
    cidx = band_sample(y.shape[1], seed + 2)
    om = omega(y.shape[1], seed + 1)
    np.savez_compressed(
        path + ".tmp.npz", name=name, index=index, shape=np.array(y.shape),
        steps=5, coeffs=np.array(oracle.QUINTIC), eps=oracle.EPS,
        input_sha256=sha, rows_idx=ridx, rows=y[ridx].astype(np.float32),
        cols_idx=cidx, cols=np.ascontiguousarray(y[:, cidx]).astype(np.float32),
        omega=om.astype(np.int8), sketch=y @ om, fro=np.linalg.norm(y),
        oracle_seconds=dt)
    os.replace(path + ".tmp.npz", path)
    print(f"{name}: {y.shape} in {dt:.0f} s", flush=True)


if __name__ == "__main__":
    want = set(sys.argv[1:])
    todo = [t for t in sampled_indices() if not want or t[0] in want]
    # cheapest first, so that an interrupted run still leaves finished files
    shape = {workloads.dense_lowrank_matrix: lambda i: workloads.DENSE_SHAPE,
             workloads.ragged_remainder_matrix: lambda i: workloads.REMAINDER_SHAPE,
             workloads.moe_mixed_matrix: lambda i: workloads.moe_mixed_shapes()[i]}
    todo.sort(key=lambda t: workloads.flops_per_matrix(*shape[t[1]](t[2])))
    for name, make, index in todo:
        write_one(name, make, index)
