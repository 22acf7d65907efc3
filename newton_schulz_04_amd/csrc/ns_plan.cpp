// ns_plan.cpp -- batch planner for libns.so (host only, no HIP calls).
//
// Each matrix is classified (empty / small / large), large matrices are
// ordered by the Newton-Schulz cost max(M,N)*min(M,N)^2 (NVIDIA/Megatron-LM
// PR #6379, "Balance LayerWise optimizer shards by Newton-Schulz cost, not
// parameter size", Changes items 1-2: order and assign by that cost, largest
// first), and every grouped GEMM stage gets one tile list for the whole
// batch. Tiles are sorted by their own work (K depth x 256^2) largest first,
// ties keeping the cost order of their matrices, so the hardware dispatcher,
// which hands out workgroups in index order as compute units free up, runs a
// longest-processing-time-first list schedule over all compute units.
#include "ns_plan.h"

#include <algorithm>
#include <limits>

namespace ns {

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 24;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int32_t pad_to(int64_t v, int64_t q) { return (int32_t)((v + q - 1) / q * q); }

}  // namespace

int64_t ns_cost(int64_t rows, int64_t cols)
{
    if (rows < 0 || cols < 0)
        return -1;
    const unsigned __int128 hi = (unsigned __int128)(rows > cols ? rows : cols);
    const unsigned __int128 lo = (unsigned __int128)(rows > cols ? cols : rows);
    const unsigned __int128 c = hi * lo * lo;
    const unsigned __int128 cap = (unsigned __int128)std::numeric_limits<int64_t>::max();
    return c > cap ? std::numeric_limits<int64_t>::max() : (int64_t)c;
}

int make_plan(const int64_t* shapes, int32_t count, int32_t dtype, Plan* plan, std::string* err)
{
    if (count < 0) {
        *err = "count must be >= 0";
        return 1;
    }
    if (count > 0 && !shapes) {
        *err = "shapes is NULL";
        return 1;
    }
    if (dtype != 0 && dtype != 1) {
        *err = "unknown dtype " + std::to_string(dtype);
        return 2;
    }
    Plan& p = *plan;
    p = Plan();
    p.dtype = dtype;
    p.elt = dtype == 0 ? 2 : 4;
    p.mats.resize(count);
    for (int32_t i = 0; i < count; ++i) {
        const int64_t rows = shapes[2 * i], cols = shapes[2 * i + 1];
        if (rows < 0 || cols < 0) {
            *err = "matrix " + std::to_string(i) + " has a negative dimension";
            return 1;
        }
        if (rows > kMaxDim || cols > kMaxDim) {
            *err = "matrix " + std::to_string(i) + " has a dimension above 2^24";
            return 1;
        }
        PlanMat& pm = p.mats[i];
        pm.index = i;
        pm.rows = rows;
        pm.cols = cols;
        pm.trans = rows > cols;
        pm.m = (int32_t)(pm.trans ? cols : rows);
        pm.n = (int32_t)(pm.trans ? rows : cols);
        pm.cost = ns_cost(rows, cols);
        if (rows == 0 || cols == 0) {
            pm.cls = kEmpty;
        } else if (pm.m <= kSmallMax) {
            pm.cls = kSmall;
        } else {
            pm.cls = kLarge;
            pm.mp = pad_to(pm.m, kTile);
            pm.np = pad_to(pm.n, kTile);
            // Tile coordinates are int16 and a 256-row operand block must fit
            // a 32-bit buffer range.
            if (pm.np / kTile > 32767 || (int64_t)pm.np * (int64_t)p.elt * kTile >= (int64_t(1) << 31)) {
                *err = "matrix " + std::to_string(i) + " is too large for the tiled path";
                return 1;
            }
        }
    }

    // Launch order: largest cost first; ties keep batch order.
    for (const PlanMat& pm : p.mats) {
        if (pm.cls == kLarge) p.large.push_back(pm.index);
        if (pm.cls == kSmall) p.small.push_back(pm.index);
    }
    auto by_cost = [&](int32_t a, int32_t b) { return p.mats[a].cost > p.mats[b].cost; };
    std::stable_sort(p.large.begin(), p.large.end(), by_cost);
    std::stable_sort(p.small.begin(), p.small.end(), by_cost);

    // Tile lists. Within a matrix, tiles run row by row.
    struct Item { Tile t; int64_t depth; };
    std::vector<Item> syrk, poly, upd;
    p.part_prefix.assign(1, 0);
    p.prep_prefix.assign(1, 0);
    for (size_t li = 0; li < p.large.size(); ++li) {
        const PlanMat& pm = p.mats[p.large[li]];
        const int mb = pm.mp / kTile, nb = pm.np / kTile;
        for (int bi = 0; bi < mb; ++bi)
            for (int bj = bi; bj < mb; ++bj) {
                syrk.push_back({Tile{(int32_t)li, (int16_t)bi, (int16_t)bj}, pm.np});
                poly.push_back({Tile{(int32_t)li, (int16_t)bi, (int16_t)bj}, pm.mp});
            }
        for (int bi = 0; bi < mb; ++bi)
            for (int bj = 0; bj < nb; ++bj)
                upd.push_back({Tile{(int32_t)li, (int16_t)bi, (int16_t)bj}, pm.mp});
        const int64_t numel = pm.rows * pm.cols;
        const int64_t parts = (numel + kNormChunk - 1) / kNormChunk;
        const int64_t prep = (int64_t)(pm.mp / kPrepTile) * (pm.np / kPrepTile);
        if (p.part_prefix.back() + parts > std::numeric_limits<int32_t>::max() ||
            p.prep_prefix.back() + prep > std::numeric_limits<int32_t>::max()) {
            *err = "batch too large";
            return 1;
        }
        p.part_prefix.push_back(p.part_prefix.back() + (int32_t)parts);
        p.prep_prefix.push_back(p.prep_prefix.back() + (int32_t)prep);
    }
    auto by_depth = [](const Item& a, const Item& b) { return a.depth > b.depth; };
    std::stable_sort(syrk.begin(), syrk.end(), by_depth);
    std::stable_sort(poly.begin(), poly.end(), by_depth);
    std::stable_sort(upd.begin(), upd.end(), by_depth);
    for (const Item& it : syrk) p.syrk_tiles.push_back(it.t);
    for (const Item& it : poly) p.poly_tiles.push_back(it.t);
    for (const Item& it : upd) p.update_tiles.push_back(it.t);
    p.total_parts = p.part_prefix.back();
    p.total_prep = p.prep_prefix.back();

    // Workspace: data buffers first, then metadata.
    size_t off = 0;
    for (int32_t idx : p.large) {
        const PlanMat& pm = p.mats[idx];
        const size_t mn = (size_t)pm.mp * pm.np, mm = (size_t)pm.mp * pm.mp;
        LargeOffsets lo{};
        if (dtype == 0) {
            lo.xf = off;
            off = align_up(off + 4 * mn);
        } else {
            lo.xf = SIZE_MAX;
        }
        for (int s = 0; s < 2; ++s) {
            lo.xb[s] = off;
            off = align_up(off + p.elt * mn);
            lo.xt[s] = off;
            off = align_up(off + p.elt * mn);
        }
        lo.a = off;
        off = align_up(off + p.elt * mm);
        lo.b = off;
        off = align_up(off + p.elt * mm);
        p.large_off.push_back(lo);
    }
    for (int32_t idx : p.small) {
        const PlanMat& pm = p.mats[idx];
        p.small_off.push_back(off);
        off = align_up(off + 4 * (size_t)pm.m * pm.n);
    }
    p.data_bytes = off;
    // Metadata lives in its own allocation, laid out from 0.
    off = 0;
    p.meta_large = off;
    off = align_up(off + sizeof(LargeMat) * p.large.size());
    p.meta_small = off;
    off = align_up(off + sizeof(SmallMat) * p.small.size());
    p.meta_syrk = off;
    off = align_up(off + sizeof(Tile) * p.syrk_tiles.size());
    p.meta_poly = off;
    off = align_up(off + sizeof(Tile) * p.poly_tiles.size());
    p.meta_update = off;
    off = align_up(off + sizeof(Tile) * p.update_tiles.size());
    p.meta_part_prefix = off;
    off = align_up(off + sizeof(int32_t) * p.part_prefix.size());
    p.meta_prep_prefix = off;
    off = align_up(off + sizeof(int32_t) * p.prep_prefix.size());
    p.meta_inv = off;
    off = align_up(off + sizeof(float) * p.large.size());
    p.meta_partials = off;
    off = align_up(off + sizeof(float) * (size_t)p.total_parts);
    p.meta_end = off;
    return 0;
}

}  // namespace ns
