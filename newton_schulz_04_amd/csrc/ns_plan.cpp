// ns_plan.cpp -- batch planner for libns.so (host only, no HIP calls).
//
// Each matrix is classified (empty / small / large) and large matrices are
// ordered by the Newton-Schulz cost max(M,N)*min(M,N)^2 (NVIDIA/Megatron-LM
// PR #6379, "Balance LayerWise optimizer shards by Newton-Schulz cost, not
// parameter size", Changes items 1-2: order and assign by that cost, largest
// first). Every grouped GEMM stage gets one tile list for the whole batch:
// tiles are grouped per XCD so that the compute units sharing an L2 work on
// neighbouring tiles, and groups go longest first (K depth x 256^2, then the
// cost order of their matrices) to the least-loaded XCD, so the dispatcher,
// which hands out workgroups in index order as compute units free up, runs a
// longest-processing-time-first list schedule.
#include "ns_plan.h"

#include <algorithm>
#include <cstdlib>
#include <limits>

namespace ns {

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 24;
// Dispatch topology: XCDs per device and the tile group one XCD runs at once.
constexpr int kXcds = 8;
constexpr int kGroupRows = 4, kGroupCols = 8;
enum { kStageSyrk = 0, kStagePoly = 1, kStageUpdate = 2 };
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Row pitch (elements) of a GEMM operand array whose rows hold `len`
// elements of `elt` bytes. Rows 4 KB x (odd number) apart stream into LDS
// ~20% slower than other spacings on MI355X (measured: 12 KB and 20 KB
// pitches against 8, 16 KB and padded ones), so such pitches get 128 bytes
// of padding; the padding is never read or written.
int32_t row_pitch(int64_t len, int64_t elt)
{
    const int64_t bytes = len * elt;
    return (int32_t)(bytes % 8192 == 4096 ? len + 128 / elt : len);
}

int32_t pad_to(int64_t v, int64_t q) { return (int32_t)((v + q - 1) / q * q); }

// Tile order of one grouped GEMM stage.
//
// The dispatcher hands workgroup w to XCD w % kXcds, and each XCD's 32 compute
// units share one L2. So the list is built per XCD: every matrix's tile grid
// is cut into groups of kGroupRows x kGroupCols tiles (one group = what an
// XCD's compute units run at once, sharing kGroupRows + kGroupCols operand
// blocks), groups are taken longest first (K depth, then the cost order of
// their matrices), each goes to the XCD with the least work so far, and the
// XCD sequences are interleaved so that position w holds the next tile of XCD
// w % kXcds. An XCD that runs out early takes the next tile of the XCD with
// the most work left.
std::vector<Tile> order_tiles(const Plan& p, int stage)
{
    struct Group { int64_t depth; std::vector<Tile> tiles; };
    std::vector<Group> groups;
    for (size_t li = 0; li < p.large.size(); ++li) {
        const PlanMat& pm = p.mats[p.large[li]];
        const int mb = pm.mp / kTile;
        const int nb = stage == kStageUpdate ? pm.np / kTile : mb;
        const int64_t depth = stage == kStageSyrk ? pm.np : pm.mp;
        for (int gi = 0; gi < mb; gi += kGroupRows)
            for (int gj = 0; gj < nb; gj += kGroupCols) {
                Group g{depth, {}};
                for (int bi = gi; bi < std::min(gi + kGroupRows, mb); ++bi)
                    for (int bj = gj; bj < std::min(gj + kGroupCols, nb); ++bj)
                        if (stage == kStageUpdate || bj >= bi)
                            g.tiles.push_back(Tile{(int32_t)li, (int16_t)bi, (int16_t)bj});
                if (!g.tiles.empty())
                    groups.push_back(std::move(g));
            }
    }
    std::stable_sort(groups.begin(), groups.end(),
                     [](const Group& a, const Group& b) { return a.depth > b.depth; });
    std::vector<std::vector<Tile>> xcd(kXcds);
    std::vector<int64_t> load(kXcds, 0);
    size_t total = 0;
    for (const Group& g : groups) {
        int best = 0;
        for (int x = 1; x < kXcds; ++x)
            if (load[x] < load[best]) best = x;
        load[best] += g.depth * (int64_t)g.tiles.size();
        xcd[best].insert(xcd[best].end(), g.tiles.begin(), g.tiles.end());
        total += g.tiles.size();
    }
    std::vector<Tile> out;
    out.reserve(total);
    std::vector<size_t> next(kXcds, 0);
    for (size_t pos = 0; pos < total; ++pos) {
        int x = (int)(pos % kXcds);
        if (next[x] == xcd[x].size()) {
            int most = -1;
            for (int y = 0; y < kXcds; ++y)
                if (next[y] < xcd[y].size() &&
                    (most < 0 || xcd[y].size() - next[y] > xcd[most].size() - next[most]))
                    most = y;
            x = most;
        }
        out.push_back(xcd[x][next[x]++]);
    }
    return out;
}

// Compute units of the device the tile lists are cut for (MI355X).
constexpr size_t kCus = 256;

// The last r = n mod kCus tiles of a symmetric stage form a partial last
// round. When r <= kCus / 2 (after at least one full round), they run as
// 2r half tiles (each half of a tile's columns, the same bits) on twice as
// many compute units. Diagonal tiles cannot be halved: those in the tail
// trade places with an off-diagonal tile of the same matrix before it
// (same K depth, same XCD position where there is one). Returns r, or 0 when
// nothing is split.
int32_t split_tail(std::vector<Tile>& tl)
{
    const size_t n = tl.size(), r = n % kCus;
    if (n <= kCus || r == 0 || r > kCus / 2)
        return 0;
    const size_t t0 = n - r;
    for (size_t pos = t0; pos < n; ++pos) {
        if (tl[pos].bi != tl[pos].bj)
            continue;
        size_t found = SIZE_MAX;
        for (int pass = 0; pass < 2 && found == SIZE_MAX; ++pass)
            for (size_t q = t0; q-- > 0;)
                if (tl[q].mat == tl[pos].mat && tl[q].bi != tl[q].bj &&
                    (pass == 1 || q % kXcds == pos % kXcds)) {
                    found = q;
                    break;
                }
        if (found == SIZE_MAX)
            return 0;
        std::swap(tl[pos], tl[found]);
    }
    return (int32_t)r;
}

// The uploaded list: tiles [0, n - r), then the halves of the last r, all
// in one launch. Tiles k and k' of a group of 8 sat on XCD k mod 8; their
// halves go to positions 16 g + k mod 8 and 16 g + c + k mod 8 of the half
// part, which starts at n - r, a multiple of kCus and so of 8 (c = the
// group's size), i.e. the same XCD for whole groups, so two halves share
// their operand blocks in one L2.
std::vector<Tile> run_list(const std::vector<Tile>& tl, int32_t split)
{
    const size_t n = tl.size(), r = (size_t)split, t0 = n - r;
    std::vector<Tile> out(tl.begin(), tl.begin() + t0);
    out.resize(n + r);
    for (size_t g = 0; g * kXcds < r; ++g) {
        const size_t c = std::min((size_t)kXcds, r - g * kXcds);
        for (size_t j = 0; j < c; ++j) {
            const Tile t = tl[t0 + g * kXcds + j];
            out[t0 + 2 * g * kXcds + j] = Tile{t.mat, t.bi, t.bj};
            out[t0 + 2 * g * kXcds + c + j] = Tile{(int32_t)((uint32_t)t.mat | (1u << 30)), t.bi, t.bj};
        }
    }
    return out;
}

}  // namespace

int32_t small_threshold()
{
    const char* v = std::getenv("NS_SMALL_M");
    if (!v || !*v)
        return kSmallMax;
    char* end = nullptr;
    const long t = std::strtol(v, &end, 10);
    return (*end == 0 && t >= 0 && t <= kSmallMax) ? (int32_t)t : kSmallMax;
}

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
    p.small_max = small_threshold();
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
        } else if (pm.m <= p.small_max) {
            pm.cls = kSmall;
        } else {
            pm.cls = kLarge;
            pm.mp = pad_to(pm.m, kTile);
            pm.np = pad_to(pm.n, kTile);
            pm.ldx = row_pitch(pm.np, p.elt);
            pm.ldt = row_pitch(pm.mp, p.elt);
            // Tile coordinates are int16 and a 256-row operand block must fit
            // a 32-bit buffer range.
            if (pm.np / kTile > 32767 || (int64_t)pm.np * (int64_t)p.elt * kTile >= (int64_t(1) << 31) ||
                (int64_t)pm.np * pm.ldt * (int64_t)p.elt >= (int64_t(1) << 31)) {
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
    // small matrices: grouped by m rounded up to 8 (one kernel instance per
    // group), largest cost first within a group
    std::stable_sort(p.small.begin(), p.small.end(), [&](int32_t a, int32_t b) {
        const int ra = (p.mats[a].m + 7) / 8, rb = (p.mats[b].m + 7) / 8;
        return ra != rb ? ra < rb : p.mats[a].cost > p.mats[b].cost;
    });

    // Tile lists. Norm and normalize pieces per matrix first.
    p.part_prefix.assign(1, 0);
    p.prep_prefix.assign(1, 0);
    for (size_t li = 0; li < p.large.size(); ++li) {
        const PlanMat& pm = p.mats[p.large[li]];
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
    p.syrk_tiles = order_tiles(p, kStageSyrk);
    p.poly_tiles = order_tiles(p, kStagePoly);
    p.update_tiles = order_tiles(p, kStageUpdate);
    if (dtype == 0) {
        p.syrk_split = split_tail(p.syrk_tiles);
        p.poly_split = split_tail(p.poly_tiles);
    }
    p.syrk_run = run_list(p.syrk_tiles, p.syrk_split);
    p.poly_run = run_list(p.poly_tiles, p.poly_split);
    p.total_parts = p.part_prefix.back();
    p.total_prep = p.prep_prefix.back();

    // Workspace: data buffers first, then metadata.
    size_t off = 0;
    for (int32_t idx : p.large) {
        const PlanMat& pm = p.mats[idx];
        const size_t xb_bytes = p.elt * (size_t)pm.mp * pm.ldx;   // mp rows of np
        const size_t xt_bytes = p.elt * (size_t)pm.np * pm.ldt;   // np rows of mp
        const size_t sq_bytes = p.elt * (size_t)pm.mp * pm.ldt;   // mp rows of mp
        LargeOffsets lo{};
        if (dtype == 0) {
            lo.xlo = off;
            off = align_up(off + xt_bytes);
        } else {
            lo.xlo = SIZE_MAX;
        }
        for (int s = 0; s < 2; ++s) {
            if (dtype == 0) {
                lo.xb[s] = SIZE_MAX;   // bf16: X X^T reads X from X^T
            } else {
                lo.xb[s] = off;
                off = align_up(off + xb_bytes);
            }
            lo.xt[s] = off;
            off = align_up(off + xt_bytes);
        }
        lo.a = off;
        off = align_up(off + sq_bytes);
        lo.b = off;
        off = align_up(off + sq_bytes);
        if (dtype == 0) {
            lo.adiag = off;
            off = align_up(off + 4 * (size_t)pm.mp);
            lo.bdiag = off;
            off = align_up(off + 4 * (size_t)pm.mp);
        } else {
            lo.adiag = lo.bdiag = SIZE_MAX;
        }
        p.large_off.push_back(lo);
    }
    p.small_prefix.assign(1, 0);
    for (int32_t idx : p.small) {
        const PlanMat& pm = p.mats[idx];
        SmallOffsets so{};
        so.mr = (pm.m + 7) / 8 * 8;
        const int64_t chunks = ((int64_t)pm.n + kSmallSlice - 1) / kSmallSlice;
        const int64_t per = (chunks + kSmallMaxSlices - 1) / kSmallMaxSlices;   // chunks per slice
        so.slice_cols = (int32_t)(per * kSmallSlice);
        so.nslices = (int32_t)((pm.n + so.slice_cols - 1) / so.slice_cols);
        if ((int64_t)p.small_prefix.back() + so.nslices > std::numeric_limits<int32_t>::max()) {
            *err = "batch too large";
            return 1;
        }
        p.small_prefix.push_back(p.small_prefix.back() + so.nslices);
        so.gram = off;
        off = align_up(off + 8 * (size_t)so.nslices * so.mr * so.mr);
        so.norm = off;
        off = align_up(off + 8 * (size_t)so.nslices);
        p.small_off.push_back(so);
    }
    p.total_small = p.small_prefix.back();
    p.data_bytes = off;
    // Metadata lives in its own allocation, laid out from 0.
    off = 0;
    p.meta_large = off;
    off = align_up(off + sizeof(LargeMat) * p.large.size());
    p.meta_small = off;
    off = align_up(off + sizeof(SmallMat) * p.small.size());
    p.meta_syrk = off;
    off = align_up(off + sizeof(Tile) * p.syrk_run.size());
    p.meta_poly = off;
    off = align_up(off + sizeof(Tile) * p.poly_run.size());
    p.meta_update = off;
    off = align_up(off + sizeof(Tile) * p.update_tiles.size());
    p.meta_part_prefix = off;
    off = align_up(off + sizeof(int32_t) * p.part_prefix.size());
    p.meta_prep_prefix = off;
    off = align_up(off + sizeof(int32_t) * p.prep_prefix.size());
    p.meta_small_prefix = off;
    off = align_up(off + sizeof(int32_t) * p.small_prefix.size());
    p.meta_inv = off;   // (scale, 2^E) per matrix
    off = align_up(off + 2 * sizeof(float) * p.large.size());
    p.meta_partials = off;   // scaled sums, then exponents, per piece
    off = align_up(off + 2 * sizeof(float) * (size_t)p.total_parts);
    p.meta_end = off;
    return 0;
}

}  // namespace ns
