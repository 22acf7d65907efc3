// Host-side checks run under AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_host_sanitizers.py builds this with g++ together with the host
// sources of libns.so, host-only kernel stand-ins and the fp64 oracle).
//
//  1. argument validation of every entry point: each invalid call returns its
//     status before anything touches a device;
//  2. the batch planner over seeded random batches (empty, small, large,
//     transposed, near the size limits), with its tile lists checked to
//     cover every output block once;
//  3. the rank planner over seeded random parameter lists;
//  4. the oracle on seeded random small matrices (all step counts 0..3, per
//     step schedules, empty shapes).
// Prints "host_check ok" and returns 0 when every expectation holds.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <set>
#include <string>
#include <tuple>
#include <vector>

#include "ns.h"
#include "ns_plan.h"

extern "C" int ns_oracle_f64_sched(const double* in, double* out, int64_t rows, int64_t cols,
                                   int32_t steps, const double* coeffs, int32_t per_step, double eps);

static int g_fail = 0;
#define EXPECT(cond, ...)                                   \
    do {                                                    \
        if (!(cond)) {                                      \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);              \
            std::fprintf(stderr, "\n");                     \
            ++g_fail;                                       \
        }                                                   \
    } while (0)

static void check_validation()
{
    const float q[3] = {NS_QUINTIC_A, NS_QUINTIC_B, NS_QUINTIC_C};
    alignas(16) static char buf[64];
    void* p[2] = {buf, buf + 16};
    int64_t ok[4] = {300, 520, 24, 100};
    int64_t neg[4] = {300, 520, -1, 3};
    int64_t big[2] = {(int64_t(1) << 24) + 1, 4};
    EXPECT(ns_orthogonalize_batched(p, neg, 2, 5, q, NS_BF16, nullptr) == NS_EINVAL, "negative shape");
    EXPECT(ns_orthogonalize_batched(p, big, 1, 5, q, NS_BF16, nullptr) == NS_EINVAL, "dimension above 2^24");
    EXPECT(ns_orthogonalize_batched(p, ok, 2, 5, q, 7, nullptr) == NS_EDTYPE, "dtype");
    EXPECT(ns_orthogonalize_batched(p, ok, 2, -1, q, NS_BF16, nullptr) == NS_EINVAL, "steps");
    EXPECT(ns_orthogonalize_batched(p, ok, 2, 5, nullptr, NS_BF16, nullptr) == NS_EINVAL, "coeffs");
    EXPECT(ns_orthogonalize_batched(p, ok, -1, 5, q, NS_BF16, nullptr) == NS_EINVAL, "count");
    EXPECT(ns_orthogonalize_batched(nullptr, ok, 2, 5, q, NS_BF16, nullptr) == NS_EINVAL, "null ptrs");
    EXPECT(ns_orthogonalize_batched(p, nullptr, 2, 5, q, NS_BF16, nullptr) == NS_EINVAL, "null shapes");
    void* np_[2] = {buf, nullptr};
    EXPECT(ns_orthogonalize_batched(np_, ok, 2, 5, q, NS_BF16, nullptr) == NS_EINVAL, "null matrix ptr");
    void* mis[2] = {buf + 1, buf + 16};
    EXPECT(ns_orthogonalize_batched(mis, ok, 2, 5, q, NS_BF16, nullptr) == NS_EINVAL, "misaligned");
    EXPECT(std::strlen(ns_last_error()) > 0, "message");
    // nothing to do: no device is touched
    int64_t empty[4] = {0, 17, 9, 0};
    void* nul[2] = {nullptr, nullptr};
    EXPECT(ns_orthogonalize_batched(nul, empty, 2, 5, q, NS_FP32, nullptr) == NS_OK, "empty batch");
    EXPECT(ns_orthogonalize_batched(nullptr, nullptr, 0, 5, q, NS_FP32, nullptr) == NS_OK, "count 0");
    std::vector<float> sched(3 * 65, 1.f);
    EXPECT(ns_orthogonalize_batched_sched(p, ok, 2, 65, sched.data(), NS_BF16, nullptr) == NS_EINVAL,
           "schedule too long");
    // chunked
    void* cp[3] = {buf, buf + 16, nullptr};
    int64_t cr[3] = {3, 3, 0};
    int32_t nc[1] = {3};
    int64_t cc[1] = {8};
    int64_t crn[3] = {3, -3, 0};
    EXPECT(ns_orthogonalize_chunked(cp, crn, nc, cc, 1, 5, q, NS_BF16, nullptr) == NS_EINVAL, "negative chunk");
    int32_t ncn[1] = {-1};
    EXPECT(ns_orthogonalize_chunked(cp, cr, ncn, cc, 1, 5, q, NS_BF16, nullptr) == NS_EINVAL, "negative count");
    void* cpn[3] = {buf, nullptr, nullptr};
    EXPECT(ns_orthogonalize_chunked(cpn, cr, nc, cc, 1, 5, q, NS_BF16, nullptr) == NS_EINVAL, "null chunk");
    // workspace sizes, including the tiled-path limit
    size_t bytes = 0;
    int64_t lim[2] = {8192, 131072};
    EXPECT(ns_workspace_bytes(lim, 1, NS_BF16, &bytes) == NS_EINVAL, "too large for the tiled path");
    int64_t fit[2] = {8192, 65536};
    EXPECT(ns_workspace_bytes(fit, 1, NS_BF16, &bytes) == NS_OK && bytes > 0, "fits");
    EXPECT(ns_workspace_bytes(fit, 1, NS_BF16, nullptr) == NS_EINVAL, "null out");
    EXPECT(ns_compute_cost(8192, 6144) == int64_t(8192) * 6144 * 6144, "cost");
    EXPECT(ns_compute_cost(-1, 4) == -1, "cost of a negative dimension");
}

static void check_planner(std::mt19937_64& rng)
{
    const int64_t dims[] = {0, 1, 7, 31, 32, 33, 100, 255, 256, 257, 520, 1000, 2048, 2304, 6144};
    for (int trial = 0; trial < 300; ++trial) {
        const int count = 1 + (int)(rng() % 40);
        const int dtype = (int)(rng() % 2);
        std::vector<int64_t> shapes(2 * count);
        for (int i = 0; i < 2 * count; ++i)
            shapes[i] = dims[rng() % (sizeof(dims) / sizeof(dims[0]))];
        ns::Plan plan;
        std::string err;
        const int rc = ns::make_plan(shapes.data(), count, dtype, &plan, &err);
        EXPECT(rc == 0, "plan failed: %s", err.c_str());
        if (rc != 0)
            continue;
        for (int stage = 0; stage < 3; ++stage) {
            const std::vector<ns::Tile>& tl =
                stage == 0 ? plan.syrk_tiles : stage == 1 ? plan.poly_tiles : plan.update_tiles;
            std::set<std::tuple<int, int, int>> seen;
            size_t expect = 0;
            for (size_t li = 0; li < plan.large.size(); ++li) {
                const ns::PlanMat& pm = plan.mats[plan.large[li]];
                const int mb = pm.mp / ns::kTile, nb = pm.np / ns::kTile;
                expect += stage == 2 ? (size_t)mb * nb : (size_t)mb * (mb + 1) / 2;
            }
            for (const ns::Tile& t : tl) {
                EXPECT(t.mat >= 0 && (size_t)t.mat < plan.large.size(), "tile matrix index");
                EXPECT(seen.insert(std::make_tuple(t.mat, (int)t.bi, (int)t.bj)).second, "tile twice");
            }
            EXPECT(seen.size() == expect, "stage %d: %zu tiles, expected %zu", stage, seen.size(), expect);
        }
        // the uploaded lists hold the whole tiles, then both halves of the split ones
        EXPECT(plan.syrk_run.size() == plan.syrk_tiles.size() + (size_t)plan.syrk_split, "syrk run list");
        EXPECT(plan.poly_run.size() == plan.poly_tiles.size() + (size_t)plan.poly_split, "poly run list");
        size_t w = 0;
        int64_t* sh = shapes.data();
        EXPECT(ns_workspace_bytes(sh, count, dtype, &w) == NS_OK && w == plan.total_bytes(), "workspace bytes");
        std::vector<int32_t> kinds(count);
        EXPECT(ns_plan_classify(sh, count, dtype, kinds.data()) == NS_OK, "classify");
        int64_t nt = 0;
        int32_t edge = 0;
        EXPECT(ns_plan_tiles(sh, count, dtype, 2, nullptr, 0, &nt, &edge) == NS_OK, "tiles count");
        std::vector<int32_t> out(4 * (size_t)(nt > 0 ? nt : 1));
        EXPECT(ns_plan_tiles(sh, count, dtype, 2, out.data(), nt, &nt, &edge) == NS_OK, "tiles");
    }
}

static void check_ranks(std::mt19937_64& rng)
{
    for (int trial = 0; trial < 300; ++trial) {
        const int count = (int)(rng() % 60);
        const int world = 1 + (int)(rng() % 16);
        std::vector<int64_t> numel(count), cost(count), offset(count), belems(count > 0 ? count : 1);
        std::vector<int32_t> rank(count), bucket(count);
        std::vector<int64_t> rcost(world);
        for (int i = 0; i < count; ++i) {
            const int64_t r = 1 + (int64_t)(rng() % 4096), c = 1 + (int64_t)(rng() % 4096);
            numel[i] = r * c;
            cost[i] = ns_compute_cost(r, c);
        }
        int32_t nb = 0;
        const int64_t bucket_size = (int64_t)(rng() % (1 << 24));
        const int64_t align = 1 + (int64_t)(rng() % 128);
        const ns_status st = ns_plan_ranks(numel.data(), cost.data(), count, world, bucket_size, align,
                                           (int)(rng() % 2), (int)(rng() % 2), rank.data(), offset.data(),
                                           bucket.data(), belems.data(), &nb, rcost.data());
        EXPECT(st == NS_OK, "rank plan: %s", ns_last_error());
        for (int i = 0; i < count; ++i)
            EXPECT(rank[i] >= 0 && rank[i] < world && bucket[i] >= 0 && bucket[i] < nb, "rank output");
    }
    int64_t n1 = 4, c1 = 4;
    int32_t r1, b1, nb1;
    int64_t o1, be1;
    EXPECT(ns_plan_ranks(&n1, &c1, 1, 0, 0, 1, 1, 1, &r1, &o1, &b1, &be1, &nb1, nullptr) == NS_EINVAL,
           "world 0");
}

static void check_oracle(std::mt19937_64& rng)
{
    std::normal_distribution<double> nd;
    const double q[3] = {3.4445, -4.775, 2.0315};
    for (int trial = 0; trial < 60; ++trial) {
        const int64_t r = (int64_t)(rng() % 40), c = (int64_t)(rng() % 40);
        const int steps = (int)(rng() % 4);
        std::vector<double> g((size_t)(r * c) + 1), y((size_t)(r * c) + 1);
        for (auto& v : g)
            v = nd(rng);
        std::vector<double> sched(3 * 4);
        for (int s = 0; s < 4; ++s)
            std::memcpy(&sched[3 * s], q, sizeof q);
        EXPECT(ns_oracle_f64_sched(g.data(), y.data(), r, c, steps, q, 0, 1e-7) == 0, "oracle");
        EXPECT(ns_oracle_f64_sched(g.data(), y.data(), r, c, steps, sched.data(), 1, 1e-7) == 0, "oracle sched");
        EXPECT(ns_oracle_f64_sched(g.data(), g.data(), r, c, steps, q, 0, 1e-7) == 0, "oracle in place");
    }
    EXPECT(ns_oracle_f64_sched(nullptr, nullptr, -1, 3, 1, q, 0, 1e-7) == 1, "oracle negative");
    EXPECT(ns_oracle_f64_sched(nullptr, nullptr, 0, 3, 1, q, 0, 1e-7) == 0, "oracle empty");
}

int main()
{
    std::mt19937_64 rng(20240601);
    check_validation();
    check_planner(rng);
    check_ranks(rng);
    check_oracle(rng);
    if (g_fail) {
        std::fprintf(stderr, "host_check: %d failures\n", g_fail);
        return 1;
    }
    std::printf("host_check ok\n");
    return 0;
}
