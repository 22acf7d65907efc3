"""Seeded synthetic inputs for the Newton-Schulz workloads.

This module only draws and lays out input matrices. It holds none of the
orthogonalization's arithmetic and imports nothing from the GPU binding or the
oracle, so both sides can be fed the same bytes from it.

Random numbers: matrix `index` of a workload with seed `seed` is drawn from its
own CPU generator, ``torch.Generator().manual_seed(seed * 2**20 + index)``,
with ``torch.randn`` in float32, then scaled and rounded to the workload's
dtype with round-to-nearest-even (``Tensor.to``). One generator per matrix lets
a test regenerate any single matrix of a large batch on its own.

Shard layouts follow the pages:
  * torch.chunk / DTensor split of a dimension over W ranks: chunk =
    ceil(size / W), trailing ranks short or empty (microsoft/dion PR #74,
    Concrete repro: 18 rows over 8 ranks give six (3, 2304) chunks and two
    (0, 2304) ones; InternLM/xtuner PR #2069, commit "ragged remainder ...
    uneven shards").
  * padded assembly: every chunk zero-padded to the largest local size, then
    stacked (dion PR #74, Fix: pad to max(local_sizes)).
  * ragged assembly: only the real rows, concatenated (xtuner PR #2069,
    ragged all-to-all with split sizes).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import torch

BF16 = torch.bfloat16
FP32 = torch.float32


def generator(seed: int, index: int) -> torch.Generator:
    return torch.Generator().manual_seed(seed * (1 << 20) + index)


def shard_sizes(size: int, world: int) -> List[int]:
    """Rows each of `world` ranks holds when `size` rows are split the
    torch.chunk / DTensor way: ceil(size/world) per rank, the tail short or
    empty."""
    if size < 0 or world <= 0:
        raise ValueError("size must be >= 0 and world > 0")
    chunk = -(-size // world) if size else 0
    return [max(0, min(chunk, size - r * chunk)) for r in range(world)]


def pad_assemble(mat: torch.Tensor, world: int):
    """Split `mat` by rows into `world` shards, zero-pad each shard to the
    largest shard and stack them. Returns (assembled, real_row_mask)."""
    sizes = shard_sizes(mat.shape[0], world)
    width = max(sizes) if sizes else 0
    out = torch.zeros((world * width, mat.shape[1]), dtype=mat.dtype)
    mask = torch.zeros(world * width, dtype=torch.bool)
    start = 0
    for r, sz in enumerate(sizes):
        out[r * width: r * width + sz] = mat[start: start + sz]
        mask[r * width: r * width + sz] = True
        start += sz
    return out, mask


def ragged_assemble(mat: torch.Tensor, world: int) -> torch.Tensor:
    """Concatenate only the real rows of each shard (no padding)."""
    sizes = shard_sizes(mat.shape[0], world)
    parts, start = [], 0
    for sz in sizes:
        parts.append(mat[start: start + sz])
        start += sz
    return torch.cat(parts, 0)


def sha256(t: torch.Tensor) -> str:
    t = t.contiguous()
    if t.dtype == BF16:
        t = t.view(torch.int16)
    return hashlib.sha256(t.numpy().tobytes()).hexdigest()


@dataclass
class Case:
    """One NS input: `mat` (CPU, the bytes handed to the library) and, when
    the matrix was assembled from padded shards, which rows are real."""
    mat: torch.Tensor
    real_rows: Optional[torch.Tensor] = None      # bool mask over rows
    zero_rows: Optional[torch.Tensor] = None      # rows that are exactly zero
    tags: dict = field(default_factory=dict)


# ---------------------------------------------------------------------------
# tiny_fp32: 4 fp32 matrices 64x32, N(0,1), seed 0; matrix 3 has its last 8
# rows zeroed.
def tiny_fp32() -> List[Case]:
    cases = []
    for i in range(4):
        g = torch.randn((64, 32), generator=generator(0, i), dtype=FP32)
        zero = torch.zeros(64, dtype=torch.bool)
        if i == 3:
            g[56:] = 0.0
            zero[56:] = True
        cases.append(Case(g, zero_rows=zero))
    return cases


# attn_gate: 32 bf16 matrices 18x2304, N(0, 0.02), seed 1, each split into 8
# row shards (3,3,3,3,3,3,0,0), padded to 3 rows -> 24x2304 with rows 18..23 zero.
ATTN_ROWS, ATTN_COLS, ATTN_WORLD, ATTN_COUNT = 18, 2304, 8, 32


def attn_gate_raw(i: int) -> torch.Tensor:
    g = torch.randn((ATTN_ROWS, ATTN_COLS), generator=generator(1, i), dtype=FP32)
    return (0.02 * g).to(BF16)


def attn_gate() -> List[Case]:
    cases = []
    for i in range(ATTN_COUNT):
        raw = attn_gate_raw(i)
        mat, mask = pad_assemble(raw, ATTN_WORLD)
        cases.append(Case(mat, real_rows=mask, zero_rows=~mask,
                          tags={"raw": raw}))
    return cases


# dense_lowrank: 8 bf16 matrices 8192x6144; per matrix L=randn(8192,64),
# R=randn(64,6144), E=randn(8192,6144) drawn in that order, G = L@R + 1e-3 E
# formed in fp64, rounded to bf16. Seed 2.
DENSE_SHAPE, DENSE_RANK, DENSE_COUNT = (8192, 6144), 64, 8


def dense_lowrank_matrix(i: int) -> torch.Tensor:
    gen = generator(2, i)
    rows, cols = DENSE_SHAPE
    left = torch.randn((rows, DENSE_RANK), generator=gen, dtype=FP32)
    right = torch.randn((DENSE_RANK, cols), generator=gen, dtype=FP32)
    noise = torch.randn((rows, cols), generator=gen, dtype=FP32)
    g = left.double() @ right.double()
    g += 1e-3 * noise.double()
    return g.to(BF16)


def dense_lowrank(indices: Optional[Sequence[int]] = None) -> List[Case]:
    idx = range(DENSE_COUNT) if indices is None else indices
    return [Case(dense_lowrank_matrix(i)) for i in idx]


# ragged_remainder: 12 bf16 matrices 8192x6144, N(0,1), seed 3. A batch of R
# uses the first R; its last matrix is sharded along dim 0 over W ranks and
# re-assembled (W=64: 64 chunks of 128, no short chunk; W=65: 64 chunks of 127
# and one of 64, padded -> 8255 rows with 63 trailing zero rows).
REMAINDER_SHAPE, REMAINDER_POOL = (8192, 6144), 12
REMAINDER_BATCHES = (1, 3, 5, 7, 12)


def ragged_remainder_matrix(i: int) -> torch.Tensor:
    g = torch.randn(REMAINDER_SHAPE, generator=generator(3, i), dtype=FP32)
    return g.to(BF16)


def ragged_remainder(r: int, world: int = 64, padded: bool = True) -> List[Case]:
    if r not in range(1, REMAINDER_POOL + 1):
        raise ValueError("R must be in 1..12")
    cases = [Case(ragged_remainder_matrix(i)) for i in range(r - 1)]
    last = ragged_remainder_matrix(r - 1)
    if padded:
        mat, mask = pad_assemble(last, world)
        cases.append(Case(mat, real_rows=mask, zero_rows=~mask,
                          tags={"world": world, "index": r - 1}))
    else:
        cases.append(Case(ragged_assemble(last, world),
                          tags={"world": world, "index": r - 1}))
    return cases


# moe_mixed: 64 x (2048,6144), 48 x (512,10240), 16 x (6144,6144),
# 2 x (10240,10240), bf16 N(0,1), seed 4; matrix index runs over the list in
# that order.
MOE_GROUPS = (((2048, 6144), 64), ((512, 10240), 48),
              ((6144, 6144), 16), ((10240, 10240), 2))


def moe_mixed_shapes() -> List[tuple]:
    return [shape for shape, count in MOE_GROUPS for _ in range(count)]


def moe_mixed_matrix(i: int) -> torch.Tensor:
    shape = moe_mixed_shapes()[i]
    return torch.randn(shape, generator=generator(4, i), dtype=FP32).to(BF16)


def moe_mixed(indices: Optional[Sequence[int]] = None) -> List[Case]:
    n = len(moe_mixed_shapes())
    idx = range(n) if indices is None else indices
    return [Case(moe_mixed_matrix(i)) for i in idx]


def moe_group_first_indices() -> List[int]:
    """Index of the first matrix of each shape class."""
    out, start = [], 0
    for _, count in MOE_GROUPS:
        out.append(start)
        start += count
    return out


# Generic helper for tests: a seeded Gaussian matrix of any shape and dtype.
def gaussian(shape, seed: int, index: int = 0, dtype=BF16, scale: float = 1.0):
    g = torch.randn(tuple(shape), generator=generator(seed, index), dtype=FP32)
    return (scale * g).to(dtype)


def flops_per_matrix(rows: int, cols: int, steps: int = 5) -> int:
    """Metric work of one matrix: steps * (4 m^2 n + 2 m^3), m = min dim,
    n = max dim."""
    m, n = min(rows, cols), max(rows, cols)
    return steps * (4 * m * m * n + 2 * m * m * m)
