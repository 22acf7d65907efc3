"""Write stored oracle results for full-size workload matrices.

The fp64 oracle needs minutes per 8192x6144 matrix, too slow to run inside a
GPU test, so this script runs it once on a seeded sample of each large
workload's matrices and stores, per matrix:

  rows_idx, rows   a seeded sample of whole output rows (fp32)
  sketch           Y @ Omega, Omega a seeded (cols x 4) matrix of +-1 (fp64)
  fro              ||Y||_F (fp64)
  input_sha256     hash of the input bytes the oracle saw

Everything stored comes from oracle/ (the fp64 CPU oracle) applied to inputs
from newton_schulz_04_amd/workloads.py; nothing comes from the GPU library.

usage: python tests/golden/make_oracle_golden.py [name ...]
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
SAMPLE_ROWS = 8


def omega(cols: int, seed: int) -> np.ndarray:
    return np.random.default_rng(seed).choice([-1.0, 1.0], size=(cols, SKETCH_K))


def row_sample(rows: int, seed: int) -> np.ndarray:
    pick = np.random.default_rng(seed).choice(rows, size=SAMPLE_ROWS - 2, replace=False)
    return np.unique(np.concatenate([[0, rows - 1], pick])).astype(np.int64)


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
        print(f"{name}: exists, skipped", flush=True)
        return
    g = make(index)
    sha = workloads.sha256(g)
    t0 = time.time()
    y = oracle.newton_schulz(g.float().numpy(), steps=5, coeffs=oracle.QUINTIC)
    dt = time.time() - t0
    seed = zlib.crc32(name.encode())
    ridx = row_sample(y.shape[0], seed)
    om = omega(y.shape[1], seed + 1)
    np.savez_compressed(
        path + ".tmp.npz", name=name, index=index, shape=np.array(y.shape),
        steps=5, coeffs=np.array(oracle.QUINTIC), eps=oracle.EPS,
        input_sha256=sha, rows_idx=ridx, rows=y[ridx].astype(np.float32),
        omega=om.astype(np.int8), sketch=y @ om, fro=np.linalg.norm(y),
        oracle_seconds=dt)
    os.replace(path + ".tmp.npz", path)
    print(f"{name}: {y.shape} in {dt:.0f} s", flush=True)


if __name__ == "__main__":
    want = set(sys.argv[1:])
    for name, make, index in sampled_indices():
        if not want or name in want:
            write_one(name, make, index)
