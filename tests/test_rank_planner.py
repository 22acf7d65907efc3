"""ns_plan_ranks: placement of whole matrices onto data-parallel ranks
(NVIDIA/Megatron-LM PR #6379, Problem, Changes 1-3, Tests and Notes). Host
only; no GPU."""
import json
import os
import random

import pytest

import newton_schulz_04_amd as ns

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_shard_layouts.json")


def test_absorbing_counterexample_from_the_pages():
    g = json.load(open(GOLDEN))["megatron_absorb_counterexample"]
    numel = g["numel_backprop_order"]
    for by_cost in (False, True):   # 1-D parameters: cost is the element count
        a = ns.plan_ranks(numel, numel, g["dp_size"], g["bucket_size"], by_cost=by_cost, absorb=True)
        t = ns.plan_ranks(numel, numel, g["dp_size"], g["bucket_size"], by_cost=by_cost, absorb=False)
        assert a["bucket_elems"] == g["absorbing_buckets"] and sum(a["bucket_elems"]) == g["absorbing_emits"]
        assert t["bucket_elems"] == g["threshold_buckets"] and sum(t["bucket_elems"]) == g["threshold_emits"]


def _gtp_case(dense=3):
    # three GTP-sharded matrices, full shape 1024 x 512 split 64 ways along
    # dim 0 (local 16 x 512), next to dense 256 x 256 matrices: the GTP cost is
    # 16x the largest dense matrix's while their numel is the smallest
    gtp = [(16 * 512, ns.compute_cost(1024, 512))] * 3
    dns = [(256 * 256, ns.compute_cost(256, 256))] * dense
    params = dns + gtp
    assert gtp[0][1] == 16 * dns[0][1] and gtp[0][0] < dns[0][0]
    return [p[0] for p in params], [p[1] for p in params]


def test_cost_order_spreads_gtp_matrices_numel_order_piles_them():
    numel, cost = _gtp_case()
    world, big = 4, 1 << 40            # one bucket
    by_numel = ns.plan_ranks(numel, cost, world, big, by_cost=False)
    by_cost = ns.plan_ranks(numel, cost, world, big, by_cost=True)
    gtp_ranks_numel = set(by_numel["rank"][-3:])
    gtp_ranks_cost = set(by_cost["rank"][-3:])
    assert len(gtp_ranks_numel) == 1 and len(gtp_ranks_cost) == 3

    def imbalance(rc):
        return max(rc) / (sum(rc) / len(rc))
    # max over mean rank cost. The page prints 3.77x and 1.33x for shapes it
    # does not give; this construction gives 48 / 12.75 = 3.765x and
    # 17 / 12.75 = 1.333x (in units of the dense cost)
    assert abs(imbalance(by_numel["rank_cost"]) - 48 / 12.75) < 1e-12
    assert abs(imbalance(by_cost["rank_cost"]) - 4 / 3) < 1e-12


def test_loads_persist_across_buckets():
    # each bucket: one GTP matrix and two dense ones; with loads kept across
    # buckets the GTP matrices of successive buckets go to different ranks
    # (reset per bucket, every bucket would put its GTP matrix on rank 0)
    g = (16 * 512, ns.compute_cost(1024, 512))
    d = (256 * 256, ns.compute_cost(256, 256))
    params = [g, d, d] * 4
    numel = [p[0] for p in params]
    cost = [p[1] for p in params]
    r = ns.plan_ranks(numel, cost, 4, 2 * 65536 + 8192, by_cost=True, absorb=False)
    assert len(r["bucket_elems"]) == 4
    gtp = [r["rank"][i] for i in range(0, 12, 3)]
    assert sorted(gtp) == [0, 1, 2, 3]


def test_equal_costs_only_rotate_the_starting_rank():
    # the review: with equal costs the persistent loads only rotate which rank
    # starts a bucket, so the multiset of shard sizes, hence every bucket's
    # size, matches the least-numel rule
    rnd = random.Random(1)
    for _ in range(100):
        world = rnd.choice([2, 3, 4, 8])
        n = rnd.randint(1, 40)
        numel = [rnd.choice([1024, 2048])] * n
        cost = [7] * n
        bs = rnd.randint(1, 8) * 1024
        a = ns.plan_ranks(numel, cost, world, bs, by_cost=True)
        b = ns.plan_ranks(numel, cost, world, bs, by_cost=False)
        assert a["bucket_elems"] == b["bucket_elems"]


def test_numel_cap_bounds_padding():
    rnd = random.Random(2)
    for _ in range(200):
        world = rnd.choice([2, 3, 4, 8, 16])
        n = rnd.randint(1, 30)
        shapes = [(rnd.randint(1, 64) * 16, rnd.randint(1, 64) * 16) for _ in range(n)]
        gtp = [rnd.choice([1, 1, 8]) for _ in range(n)]
        numel = [r * c // g for (r, c), g in zip(shapes, gtp)]
        cost = [ns.compute_cost(r, c) for r, c in shapes]
        res = ns.plan_ranks(numel, cost, world, rnd.randint(1, 20) * 4096, by_cost=True)
        for b, elems in enumerate(res["bucket_elems"]):
            members = [i for i in range(n) if res["bucket"][i] == b]
            total = sum(numel[i] for i in members)
            ideal = -(-total // world)
            bound = max(1.3 * ideal, ideal + max(numel[i] for i in members))
            assert elems / world <= bound + 1e-9
            # shards never overlap: offsets are disjoint per rank
            for rk in range(world):
                spans = sorted((res["offset"][i], res["offset"][i] + numel[i])
                               for i in members if res["rank"][i] == rk)
                assert all(spans[k][1] <= spans[k + 1][0] for k in range(len(spans) - 1))


def test_cost_order_never_worse_on_moe_shapes():
    # the page's claim for its model (cost balancing never worse than numel
    # balancing) checked on the mixed MoE shapes, whole matrices, one bucket
    from newton_schulz_04_amd import workloads
    shapes = workloads.moe_mixed_shapes()
    numel = [r * c for r, c in shapes]
    cost = [ns.compute_cost(r, c) for r, c in shapes]
    for world in (2, 4, 8, 16, 32, 64):
        a = ns.plan_ranks(numel, cost, world, 1 << 40, by_cost=True)
        b = ns.plan_ranks(numel, cost, world, 1 << 40, by_cost=False)
        assert max(a["rank_cost"]) <= max(b["rank_cost"])


def test_alignment_and_validation():
    r = ns.plan_ranks([3, 5, 7], [3, 5, 7], 1, 1 << 20, align=4, by_cost=False)
    assert r["offset"] == [16, 8, 0] and r["bucket_elems"] == [19]   # 7 at 0, 5 at 8, 3 at 16
    with pytest.raises(ns.NSError):
        ns.plan_ranks([1], [1], 0, 10)
    with pytest.raises(ns.NSError):
        ns.plan_ranks([-1], [1], 2, 10)
    with pytest.raises(ns.NSError):
        ns.plan_ranks([1], [1], 2, 10, align=0)
    assert ns.plan_ranks([], [], 4, 10)["bucket_elems"] == []
