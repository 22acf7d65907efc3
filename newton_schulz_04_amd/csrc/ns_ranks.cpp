// ns_ranks.cpp -- placement of whole matrices onto data-parallel ranks (host
// only, no HIP calls): which rank orthogonalizes which matrix, and where each
// matrix sits in the rank's shard of a bucket buffer.
//
// NVIDIA/Megatron-LM PR #6379, "Balance LayerWise optimizer shards by
// Newton-Schulz cost, not parameter size":
//   Problem: matrices are packed largest first onto the least-loaded shard.
//   Changes 1-2: order and assign by the Newton-Schulz cost
//     max(M,N) * min(M,N)^2 of the full (all-gathered) shape.
//   Changes 3: the per-shard compute loads persist across buckets, the shard
//     cursors restart in every bucket, a per-bucket numel cap
//     (epsilon = 0.3) limits the padding, and a matrix that fits under the cap
//     on no shard goes to the shard with the least numel (the earlier rule).
//   Notes: buckets are cut in backprop order with bucket_size as a soft
//     minimum (once reached, a matrix is still taken if the estimate, a
//     least-loaded placement in backprop order, says it fills padding);
//     emitting a bucket sorts it first, so the two can disagree (the page's
//     counterexample: 1408 emitted elements where closing at the threshold
//     emits 1280).
#include <algorithm>
#include <cstdint>
#include <numeric>
#include <string>
#include <vector>

#include "ns.h"

namespace {

int64_t align_up(int64_t v, int64_t a) { return a <= 1 ? v : (v + a - 1) / a * a; }

// Least-loaded index of `load`; ties go to the lowest index.
int argmin(const std::vector<int64_t>& load)
{
    return (int)(std::min_element(load.begin(), load.end()) - load.begin());
}

// Bucket boundaries over params in backprop order: bucket b is
// [cut[b], cut[b+1]).
std::vector<int32_t> cut_buckets(const int64_t* numel, int32_t count, int32_t world,
                                 int64_t bucket_size, int64_t align, bool absorb)
{
    std::vector<int32_t> cut{0};
    int64_t total = 0;
    std::vector<int64_t> est(world, 0);   // incremental placement estimate
    for (int32_t i = 0; i < count; ++i) {
        if (total >= bucket_size && cut.back() < i) {
            // at the threshold: take param i only if it fills padding
            bool fits = false;
            if (absorb) {
                const int64_t top = *std::max_element(est.begin(), est.end());
                const int s = argmin(est);
                fits = align_up(est[s], align) + numel[i] <= top;
            }
            if (!fits) {
                cut.push_back(i);
                total = 0;
                std::fill(est.begin(), est.end(), 0);
            }
        }
        const int s = argmin(est);
        est[s] = align_up(est[s], align) + numel[i];
        total += numel[i];
    }
    if (cut.back() < count)
        cut.push_back(count);
    return cut;
}

}  // namespace

extern "C" {

ns_status ns_plan_ranks(const int64_t* numel, const int64_t* cost, int32_t count, int32_t world,
                        int64_t bucket_size, int64_t align, int32_t by_cost, int32_t absorb,
                        int32_t* rank, int64_t* offset, int32_t* bucket, int64_t* bucket_elems,
                        int32_t* nbuckets, int64_t* rank_cost)
{
    if (count < 0 || world <= 0 || bucket_size < 0 || align < 1)
        return NS_EINVAL;
    if (count > 0 && (!numel || !cost || !rank || !offset || !bucket || !bucket_elems))
        return NS_EINVAL;
    if (!nbuckets)
        return NS_EINVAL;
    for (int32_t i = 0; i < count; ++i)
        if (numel[i] < 0 || cost[i] < 0)
            return NS_EINVAL;

    constexpr double kNumelEpsilon = 0.3;
    const std::vector<int32_t> cut = cut_buckets(numel, count, world, bucket_size, align, absorb != 0);
    std::vector<int64_t> load(world, 0);   // persists across buckets (cost rule)
    int32_t nb = 0;
    for (size_t b = 0; b + 1 < cut.size(); ++b, ++nb) {
        const int32_t lo = cut[b], hi = cut[b + 1];
        std::vector<int32_t> order(hi - lo);
        std::iota(order.begin(), order.end(), lo);
        // largest first by the rule's measure; ties keep backprop order
        std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
            return by_cost ? cost[x] > cost[y] : numel[x] > numel[y];
        });
        int64_t sum = 0;
        for (int32_t i = lo; i < hi; ++i)
            sum += numel[i];
        const double cap = (1.0 + kNumelEpsilon) * (double)((sum + world - 1) / world);
        std::vector<int64_t> cursor(world, 0);
        for (int32_t i : order) {
            int s = -1;
            if (by_cost) {
                for (int r = 0; r < world; ++r)
                    if ((double)(align_up(cursor[r], align) + numel[i]) <= cap &&
                        (s < 0 || load[r] < load[s]))
                        s = r;
            }
            if (s < 0)
                s = argmin(cursor);   // the least-numel rule
            offset[i] = align_up(cursor[s], align);
            cursor[s] = offset[i] + numel[i];
            load[s] += cost[i];
            rank[i] = s;
            bucket[i] = (int32_t)b;
        }
        bucket_elems[b] = (int64_t)world * *std::max_element(cursor.begin(), cursor.end());
    }
    // per-rank total cost over all buckets (both rules)
    if (rank_cost) {
        std::fill(rank_cost, rank_cost + world, 0);
        for (int32_t i = 0; i < count; ++i)
            rank_cost[rank[i]] += cost[i];
    }
    *nbuckets = nb;
    return NS_OK;
}

}  // extern "C"
