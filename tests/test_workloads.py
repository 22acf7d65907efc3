"""Input generators: the shard layouts the pages print and the workload recipes."""
import json
import os

import pytest
import torch

from newton_schulz_04_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_shard_layouts.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["shard_sizes"], ids=lambda c: f"{c['size']}/{c['world']}")
def test_shard_sizes_match_pages(case):
    assert workloads.shard_sizes(case["size"], case["world"]) == case["sizes"]


def test_shard_sizes_match_torch_chunk():
    for size in range(0, 40):
        for world in range(1, 10):
            chunks = [c.shape[0] for c in torch.chunk(torch.zeros(size), world)] if size else []
            chunks += [0] * (world - len(chunks))
            assert workloads.shard_sizes(size, world) == chunks


def test_watchdog_numel_matches_attn_gate_layout():
    # per_rank = 4 of 32 same-shape params on W = 8; a real shard is (3, 2304)
    g = _golden()["watchdog_numel"][0]
    sizes = workloads.shard_sizes(workloads.ATTN_ROWS, g["world"])
    assert max(sizes) == g["rows"]
    assert g["world"] * g["per_rank"] * max(sizes) * workloads.ATTN_COLS == g["numel"]
    assert workloads.ATTN_COUNT // g["world"] == g["per_rank"]


def test_matrix_bytes():
    g = _golden()["matrix_bytes"][0]
    assert g["rows"] * g["cols"] * g["dtype_bytes"] == g["mib"] * 2 ** 20
    assert workloads.DENSE_SHAPE == (g["rows"], g["cols"])


def test_pad_and_ragged_assemble():
    g = torch.arange(5 * 3, dtype=torch.float32).reshape(5, 3) + 1
    padded, mask = workloads.pad_assemble(g, 4)          # sizes 2,2,1,0 -> 8 rows
    assert padded.shape == (8, 3)
    assert mask.tolist() == [True, True, True, True, True, False, False, False]
    assert torch.equal(padded[mask], g)
    assert not padded[~mask].any()
    assert torch.equal(workloads.ragged_assemble(g, 4), g)


def test_remainder_w65_layout():
    sizes = workloads.shard_sizes(8192, 65)
    assert sizes[:64] == [127] * 64 and sizes[64] == 64
    assert workloads.shard_sizes(8192, 64) == [128] * 64


def test_tiny_fp32_recipe():
    cases = workloads.tiny_fp32()
    assert len(cases) == 4
    for i, c in enumerate(cases):
        assert c.mat.shape == (64, 32) and c.mat.dtype == torch.float32
    assert not cases[3].mat[56:].any() and cases[3].mat[:56].abs().min() > 0
    again = workloads.tiny_fp32()
    assert all(torch.equal(a.mat, b.mat) for a, b in zip(cases, again))


def test_attn_gate_recipe():
    cases = workloads.attn_gate()
    assert len(cases) == 32
    for c in cases:
        assert c.mat.shape == (24, 2304) and c.mat.dtype == torch.bfloat16
        assert c.real_rows.sum() == 18 and c.real_rows[:18].all()
        assert not c.mat[18:].float().any()
    std = torch.stack([c.tags["raw"].float() for c in cases]).std().item()
    assert 0.019 < std < 0.021


def test_moe_shapes_and_costs():
    shapes = workloads.moe_mixed_shapes()
    assert len(shapes) == 130
    assert shapes[0] == (2048, 6144) and shapes[64] == (512, 10240)
    assert shapes[112] == (6144, 6144) and shapes[128] == (10240, 10240)
    assert workloads.moe_group_first_indices() == [0, 64, 112, 128]


def test_flops_convention():
    # 5 * (4 m^2 n + 2 m^3), m = 6144, n = 8192: 8.504 TFLOP per matrix
    assert workloads.flops_per_matrix(8192, 6144) == 5 * (4 * 6144**2 * 8192 + 2 * 6144**3)
    assert workloads.flops_per_matrix(6144, 8192) == workloads.flops_per_matrix(8192, 6144)
