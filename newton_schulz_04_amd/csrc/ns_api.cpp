// ns_api.cpp -- the C ABI of libns.so (include/ns.h).
//
// A call validates its arguments on the host (no HIP call before the
// arguments are known good), plans the batch, makes sure the (device, stream)
// context holds a large enough workspace, finds or uploads the batch's
// metadata block, and enqueues the kernel sequence on the caller's stream:
//
//   small matrices : k_small per group of matrices with one row count MR:
//                    norm pieces, Gram pieces, the steps and the result (three
//                    launches; one when every matrix of the group is one slice)
//   large matrices : norm pieces, norm fold, normalize/transpose/pad, then per
//                    step the three grouped GEMM stages X X^T, bA + cA^2,
//                    aX + BX (the last one writes the caller's buffers); a
//                    bf16 symmetric stage whose last round is split runs its
//                    half tiles after the whole ones in the same launch.
//
// Nothing here waits for the device. Workspace growth uses stream-ordered
// allocation (hipMallocAsync / hipFreeAsync); metadata goes up from pinned
// host slots that are reused only once their copy has completed (checked with
// hipEventQuery, never waited on; a new slot is taken when none is free).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "ns.h"
#include "ns_enqueue.h"
#include "ns_kernels.h"
#include "ns_plan.h"

namespace {
thread_local std::string g_last_error;
}  // namespace

namespace ns {

ns_status fail(ns_status s, const std::string& msg)
{
    g_last_error = msg;
    return s;
}

ns_status hip_fail(hipError_t e, const char* what)
{
    return fail(NS_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

void clear_error() { g_last_error.clear(); }

}  // namespace ns

namespace {

using ns::Plan;
using ns::fail;
using ns::hip_fail;
using ns::Layout;

// --- profiling --------------------------------------------------------------
struct ProfRec {
    int kind;
    hipEvent_t start, stop;
};

std::atomic<int> g_prof_on{0};
std::mutex g_prof_mu;
std::vector<ProfRec> g_prof_pending;
std::vector<hipEvent_t> g_prof_free;
double g_prof_ms[ns::kNumKinds];
int64_t g_prof_n[ns::kNumKinds];

hipEvent_t prof_event()
{
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_free.empty()) {
        hipEvent_t e = g_prof_free.back();
        g_prof_free.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess)
        return nullptr;
    return e;
}

// --- per (device, stream) context ---------------------------------------------
struct PinnedSlot {
    void* host = nullptr;
    size_t cap = 0;
    hipEvent_t done = nullptr;
    bool used = false;
};

struct CachedPlan {
    std::vector<int64_t> shapes;
    std::vector<uintptr_t> ptrs;          // matrix or chunk pointers
    std::vector<int64_t> chunk_rows;      // chunked calls only
    std::vector<int32_t> nchunks;         // chunked calls only
    int32_t dtype = 0;
    void* ws_base = nullptr;
    void* meta = nullptr;          // device metadata block
    std::shared_ptr<Plan> plan;
    uint64_t last_use = 0;
};

struct Context {
    std::mutex mu;
    int device = 0;
    hipStream_t stream = nullptr;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    std::vector<CachedPlan> plans;
    std::vector<PinnedSlot> slots;
    uint64_t clock = 0;
};

// Batches whose plan and uploaded metadata a context keeps (least recently
// used goes first).
constexpr size_t kMaxCachedPlans = 64;
// Pinned metadata staging per context: slots of at least kSlotMinBytes, at
// most kMaxPinnedBytes in all.
constexpr size_t kSlotMinBytes = size_t(1) << 20;
constexpr size_t kMaxPinnedBytes = size_t(256) << 20;

std::mutex g_ctx_mu;
std::map<std::pair<int, uintptr_t>, std::unique_ptr<Context>> g_ctx;

Context* get_context(int device, hipStream_t stream)
{
    std::lock_guard<std::mutex> lk(g_ctx_mu);
    auto key = std::make_pair(device, reinterpret_cast<uintptr_t>(stream));
    auto it = g_ctx.find(key);
    if (it != g_ctx.end())
        return it->second.get();
    auto c = std::make_unique<Context>();
    c->device = device;
    c->stream = stream;
    Context* raw = c.get();
    g_ctx.emplace(key, std::move(c));
    return raw;
}

void drop_plans(Context* c)
{
    for (CachedPlan& cp : c->plans)
        if (cp.meta)
            (void)hipFreeAsync(cp.meta, c->stream);
    c->plans.clear();
}

ns_status ensure_workspace(Context* c, size_t bytes)
{
    if (bytes <= c->ws_bytes)
        return NS_OK;
    // Grow by at least 1/8 to avoid a reallocation per slightly larger batch.
    size_t want = bytes + bytes / 8;
    drop_plans(c);  // descriptors point into the old workspace
    if (c->ws) {
        hipError_t e = hipFreeAsync(c->ws, c->stream);
        c->ws = nullptr;
        c->ws_bytes = 0;
        if (e != hipSuccess)
            return hip_fail(e, "hipFreeAsync(workspace)");
    }
    hipError_t e = hipMallocAsync(&c->ws, want, c->stream);
    if (e != hipSuccess) {
        c->ws = nullptr;
        (void)hipGetLastError();
        return fail(NS_ENOMEM, "workspace of " + std::to_string(want) + " bytes: " +
                                   hipGetErrorString(e));
    }
    c->ws_bytes = want;
    return NS_OK;
}

// A pinned host slot of at least `bytes` whose previous copy has finished.
// Never waits: a slot still feeding a copy is skipped (hipEventQuery), and
// when none is free a new one is allocated, up to kMaxPinnedBytes per
// context; past that the call fails with NS_ENOMEM rather than block. (Slots
// are only freed by ns_release_workspace: freeing pinned memory can wait for
// the device.) A plan-cache hit uploads nothing, so an optimizer loop over a
// fixed set of batches takes slots only on its first pass.
PinnedSlot* get_slot(Context* c, size_t bytes, std::string* err)
{
    PinnedSlot* best = nullptr;
    size_t held = 0;
    for (PinnedSlot& s : c->slots) {
        held += s.cap;
        if (s.cap < bytes || (best && best->cap <= s.cap))
            continue;
        if (!s.used || hipEventQuery(s.done) == hipSuccess)
            best = &s;   // the smallest free slot that fits
    }
    if (best)
        return best;
    PinnedSlot s;
    s.cap = bytes < kSlotMinBytes ? kSlotMinBytes : bytes;
    if (held + s.cap > kMaxPinnedBytes) {
        *err = "metadata staging: " + std::to_string(c->slots.size()) + " pinned buffers (" +
               std::to_string(held >> 20) + " MiB) all feed pending uploads; a further " +
               std::to_string(s.cap) + " bytes would pass the " + std::to_string(kMaxPinnedBytes >> 20) +
               " MiB cap";
        return nullptr;
    }
    if (hipHostMalloc(&s.host, s.cap, hipHostMallocDefault) != hipSuccess) {
        (void)hipGetLastError();
        *err = "hipHostMalloc failed";
        return nullptr;
    }
    if (hipEventCreateWithFlags(&s.done, hipEventDisableTiming) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipHostFree(s.host);
        *err = "hipEventCreate failed";
        return nullptr;
    }
    c->slots.push_back(s);
    return &c->slots.back();
}

}  // namespace

namespace ns {

// Host image of the metadata block [0, meta_inv).
// Row tables of a chunked call, placed after the plan's metadata: matrix i's
// table (rows pointers) at rowtab_off[i] of the block; returns the bytes.
size_t rowtab_layout(const Plan& p, const Layout& L, int32_t count, std::vector<size_t>* off)
{
    off->assign(count, SIZE_MAX);
    if (!L.chunked())
        return 0;
    size_t at = (p.meta_end + 255) / 256 * 256;
    const size_t start = at;
    for (int32_t i = 0; i < count; ++i) {
        const ns::PlanMat& pm = p.mats[i];
        if (pm.rows == 0 || pm.cols == 0)
            continue;
        (*off)[i] = at;
        at = (at + sizeof(void*) * (size_t)pm.rows + 255) / 256 * 256;
    }
    return at - start;
}

void build_meta(const Plan& p, const Layout& L, int32_t count, char* ws, char* meta,
                std::vector<char>* out)
{
    std::vector<size_t> rt_off;
    const size_t rt_bytes = rowtab_layout(p, L, count, &rt_off);
    // chunked: everything up to the end of the row tables (the device-written
    // norm and scale region in between goes up as zeros)
    out->assign(L.chunked() ? (p.meta_end + 255) / 256 * 256 + rt_bytes : p.meta_inv, 0);
    char* h = out->data();
    std::vector<void*> user(count, nullptr);
    std::vector<void* const*> tab(count, nullptr);
    if (!L.chunked()) {
        for (int32_t i = 0; i < count; ++i)
            user[i] = L.ptrs[i];
    } else {
        const size_t elt = p.elt;
        int32_t k = 0;
        for (int32_t i = 0; i < count; ++i) {
            const ns::PlanMat& pm = p.mats[i];
            void** rows = rt_off[i] == SIZE_MAX ? nullptr : reinterpret_cast<void**>(h + rt_off[i]);
            int64_t r = 0;
            for (int32_t q = 0; q < L.nchunks[i]; ++q, ++k) {
                char* base = static_cast<char*>(L.chunk_ptrs[k]);
                for (int64_t j = 0; j < L.chunk_rows[k]; ++j, ++r)
                    if (rows)
                        rows[r] = base + (size_t)j * pm.cols * elt;
                if (!user[i] && L.chunk_rows[k] > 0)
                    user[i] = base;
            }
            if (rows)
                tab[i] = reinterpret_cast<void* const*>(meta + rt_off[i]);
        }
    }
    auto ws_at = [&](size_t off) -> void* { return off == SIZE_MAX ? nullptr : ws + off; };
    for (size_t li = 0; li < p.large.size(); ++li) {
        const ns::PlanMat& pm = p.mats[p.large[li]];
        const ns::LargeOffsets& lo = p.large_off[li];
        ns::LargeMat d{};
        d.user = user[pm.index];
        d.rows_tab = tab[pm.index];
        d.rows = pm.rows;
        d.cols = pm.cols;
        d.m = pm.m;
        d.n = pm.n;
        d.mp = pm.mp;
        d.np = pm.np;
        d.ldx = pm.ldx;
        d.ldt = pm.ldt;
        d.trans = pm.trans;
        d.batch_index = pm.index;
        d.part_begin = p.part_prefix[li];
        d.nparts = p.part_prefix[li + 1] - p.part_prefix[li];
        d.prep_begin = p.prep_prefix[li];
        d.nprep = p.prep_prefix[li + 1] - p.prep_prefix[li];
        d.xlo = ws_at(lo.xlo);
        for (int s = 0; s < 2; ++s) {
            d.xb[s] = ws_at(lo.xb[s]);
            d.xt[s] = ws_at(lo.xt[s]);
        }
        d.a = ws_at(lo.a);
        d.b = ws_at(lo.b);
        d.adiag = static_cast<float*>(ws_at(lo.adiag));
        d.bdiag = static_cast<float*>(ws_at(lo.bdiag));
        std::memcpy(h + p.meta_large + li * sizeof(ns::LargeMat), &d, sizeof d);
    }
    for (size_t si = 0; si < p.small.size(); ++si) {
        const ns::PlanMat& pm = p.mats[p.small[si]];
        const ns::SmallOffsets& so = p.small_off[si];
        ns::SmallMat d{};
        d.user = user[pm.index];
        d.rows_tab = tab[pm.index];
        d.rows = pm.rows;
        d.cols = pm.cols;
        d.m = pm.m;
        d.n = pm.n;
        d.trans = pm.trans;
        d.batch_index = pm.index;
        d.mr = so.mr;
        d.nslices = so.nslices;
        d.slice_cols = so.slice_cols;
        d.slice_begin = p.small_prefix[si];
        d.gram = reinterpret_cast<double*>(ws + so.gram);
        d.norm = reinterpret_cast<double*>(ws + so.norm);
        std::memcpy(h + p.meta_small + si * sizeof(ns::SmallMat), &d, sizeof d);
    }
    if (!p.syrk_run.empty())
        std::memcpy(h + p.meta_syrk, p.syrk_run.data(), p.syrk_run.size() * sizeof(ns::Tile));
    if (!p.poly_run.empty())
        std::memcpy(h + p.meta_poly, p.poly_run.data(), p.poly_run.size() * sizeof(ns::Tile));
    if (!p.update_tiles.empty())
        std::memcpy(h + p.meta_update, p.update_tiles.data(), p.update_tiles.size() * sizeof(ns::Tile));
    std::memcpy(h + p.meta_part_prefix, p.part_prefix.data(), p.part_prefix.size() * sizeof(int32_t));
    std::memcpy(h + p.meta_prep_prefix, p.prep_prefix.data(), p.prep_prefix.size() * sizeof(int32_t));
    std::memcpy(h + p.meta_small_prefix, p.small_prefix.data(), p.small_prefix.size() * sizeof(int32_t));
}

}  // namespace ns

namespace {

bool same_key(const CachedPlan& cp, const int64_t* shapes, const Layout& L, int32_t count,
              int32_t dtype, void* ws, int32_t small_max)
{
    if (cp.dtype != dtype || cp.ws_base != ws || cp.shapes.size() != (size_t)count * 2 ||
        cp.plan->small_max != small_max)
        return false;
    if (std::memcmp(cp.shapes.data(), shapes, sizeof(int64_t) * 2 * count) != 0)
        return false;
    if (cp.nchunks.empty() == L.chunked())
        return false;
    void* const* ptrs = L.chunked() ? L.chunk_ptrs : L.ptrs;
    const size_t np_ = L.chunked() ? (size_t)L.total_chunks : (size_t)count;
    if (cp.ptrs.size() != np_)
        return false;
    for (size_t i = 0; i < np_; ++i)
        if (cp.ptrs[i] != reinterpret_cast<uintptr_t>(ptrs[i]))
            return false;
    if (L.chunked() &&
        (std::memcmp(cp.chunk_rows.data(), L.chunk_rows, sizeof(int64_t) * np_) != 0 ||
         std::memcmp(cp.nchunks.data(), L.nchunks, sizeof(int32_t) * count) != 0))
        return false;
    return true;
}

// NS_CHECK=1 in the environment (read at every call): a debug mode that
// waits for the stream after every launch and reports the first kernel that
// failed, by kind. The one case in which an entry point waits for the device.
bool check_mode()
{
    const char* v = std::getenv("NS_CHECK");
    return v && v[0] == '1' && v[1] == 0;
}

const char* kind_name(int kind)
{
    static const char* names[ns::kNumKinds] = {"norm partial sums", "norm fold", "normalize", "X X^T",
                                               "bA + cA^2", "aX + BX", "small-matrix", "steps == 0 write-back"};
    return kind >= 0 && kind < ns::kNumKinds ? names[kind] : "unknown";
}

thread_local bool t_check = false;   // check_mode() of the current call
thread_local std::string t_check_msg;

// Launch helper: records profiling events around `fn` when profiling is on;
// in NS_CHECK mode, waits for the stream after the launch.
template <typename F>
hipError_t timed(int kind, hipStream_t stream, F&& fn)
{
    if (t_check) {
        hipError_t e = fn();
        if (e == hipSuccess)
            e = hipStreamSynchronize(stream);
        if (e == hipSuccess)
            e = hipGetLastError();
        if (e != hipSuccess)
            t_check_msg = std::string("NS_CHECK: the ") + kind_name(kind) + " kernel failed";
        return e;
    }
    if (!g_prof_on.load(std::memory_order_relaxed))
        return fn();
    hipEvent_t a = prof_event(), b = prof_event();
    if (!a || !b)
        return fn();
    (void)hipEventRecord(a, stream);
    hipError_t e = fn();
    (void)hipEventRecord(b, stream);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_pending.push_back({kind, a, b});
    return e;
}

ns_status run(Context* c, const int64_t* shapes, const Layout& L, int32_t count, int32_t steps,
              const float* coeffs, int32_t per_step, int32_t dtype)
{
    hipStream_t stream = c->stream;
    // Plan (or reuse) --------------------------------------------------------
    CachedPlan* hit = nullptr;
    const int32_t small_max = ns::small_threshold();
    for (CachedPlan& cp : c->plans)
        if (same_key(cp, shapes, L, count, dtype, c->ws, small_max)) {
            hit = &cp;
            break;
        }
    if (!hit) {
        auto plan = std::make_shared<Plan>();
        std::string err;
        int rc = ns::make_plan(shapes, count, dtype, plan.get(), &err);
        if (rc != 0)
            return fail((ns_status)rc, err);
        ns_status st = ensure_workspace(c, plan->data_bytes);
        if (st != NS_OK)
            return st;
        if (c->plans.size() >= kMaxCachedPlans) {
            size_t lru = 0;
            for (size_t i = 1; i < c->plans.size(); ++i)
                if (c->plans[i].last_use < c->plans[lru].last_use)
                    lru = i;
            (void)hipFreeAsync(c->plans[lru].meta, stream);
            c->plans.erase(c->plans.begin() + lru);
        }
        CachedPlan cp;
        cp.shapes.assign(shapes, shapes + 2 * count);
        void* const* ptrs = L.chunked() ? L.chunk_ptrs : L.ptrs;
        const int32_t np_ = L.chunked() ? L.total_chunks : count;
        cp.ptrs.resize(np_);
        for (int32_t i = 0; i < np_; ++i)
            cp.ptrs[i] = reinterpret_cast<uintptr_t>(ptrs[i]);
        if (L.chunked()) {
            cp.chunk_rows.assign(L.chunk_rows, L.chunk_rows + L.total_chunks);
            cp.nchunks.assign(L.nchunks, L.nchunks + count);
        }
        cp.dtype = dtype;
        cp.ws_base = c->ws;
        cp.plan = plan;
        std::vector<size_t> rt_off;
        const size_t rt_bytes = rowtab_layout(*plan, L, count, &rt_off);
        const size_t meta_bytes = L.chunked() ? (plan->meta_end + 255) / 256 * 256 + rt_bytes : plan->meta_end;
        hipError_t e = hipMallocAsync(&cp.meta, meta_bytes, stream);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(NS_ENOMEM, std::string("metadata block: ") + hipGetErrorString(e));
        }
        std::vector<char> img;
        build_meta(*plan, L, count, static_cast<char*>(c->ws), static_cast<char*>(cp.meta), &img);
        PinnedSlot* slot = get_slot(c, img.size(), &err);
        if (!slot) {
            (void)hipFreeAsync(cp.meta, stream);
            return fail(NS_ENOMEM, err);
        }
        std::memcpy(slot->host, img.data(), img.size());
        e = hipMemcpyAsync(cp.meta, slot->host, img.size(), hipMemcpyHostToDevice, stream);
        if (e == hipSuccess)
            e = hipEventRecord(slot->done, stream);
        slot->used = true;
        if (e != hipSuccess) {
            (void)hipFreeAsync(cp.meta, stream);
            return hip_fail(e, "metadata upload");
        }
        c->plans.push_back(std::move(cp));
        hit = &c->plans.back();
    }
    hit->last_use = ++c->clock;
    return ns::enqueue(*hit->plan, static_cast<char*>(hit->meta), steps, coeffs, per_step, dtype, stream);
}

}  // namespace

namespace ns {

ns_status enqueue(const Plan& p, char* meta, int32_t steps, const float* coeffs, int32_t per_step,
                  int32_t dtype, hipStream_t stream)
{
    t_check = check_mode();
    t_check_msg.clear();
    const ns_status st = enqueue_launches(p, meta, steps, coeffs, per_step, dtype, stream);
    if (st == NS_EHIP && !t_check_msg.empty())
        return fail(NS_EHIP, t_check_msg + " (" + ns_last_error() + ")");
    return st;
}

ns_status enqueue_launches(const Plan& p, char* meta, int32_t steps, const float* coeffs, int32_t per_step,
                           int32_t dtype, hipStream_t stream)
{
    auto* large = reinterpret_cast<const ns::LargeMat*>(meta + p.meta_large);
    auto* small = reinterpret_cast<const ns::SmallMat*>(meta + p.meta_small);
    auto* syrk = reinterpret_cast<const ns::Tile*>(meta + p.meta_syrk);
    auto* poly = reinterpret_cast<const ns::Tile*>(meta + p.meta_poly);
    auto* upd = reinterpret_cast<const ns::Tile*>(meta + p.meta_update);
    auto* part_prefix = reinterpret_cast<const int32_t*>(meta + p.meta_part_prefix);
    auto* prep_prefix = reinterpret_cast<const int32_t*>(meta + p.meta_prep_prefix);
    auto* inv = reinterpret_cast<float*>(meta + p.meta_inv);
    auto* partials = reinterpret_cast<float*>(meta + p.meta_partials);
    // step s uses coeffs[3s .. 3s + 2] when per_step, else coeffs[0 .. 2]
    auto coef = [&](int s, int k) { return coeffs[3 * (per_step ? s : 0) + k]; };
    const int nl = (int)p.large.size();

    hipError_t e = hipSuccess;
    if (!p.small.empty()) {
        // norm pieces, Gram pieces, then the m x m recurrence and the
        // result; a batch of one-slice matrices needs the first only
        auto* small_prefix = reinterpret_cast<const int32_t*>(meta + p.meta_small_prefix);
        const int ns_ = (int)p.small.size();
        ns::SmallCoeffs co{};
        co.per_step = per_step;
        for (int s = 0; s < (per_step ? steps : std::min(steps, 1)); ++s)   // steps <= 64 when per_step
            for (int k = 0; k < 3; ++k)
                co.v[3 * s + k] = coef(s, k);
        // one launch per MR group (the planner orders small matrices by MR)
        // and phase; a group of one-slice matrices needs only phase 0
        hipError_t e2 = hipSuccess;
        const int nphase = steps > 0 ? 3 : 2;
        for (int phase = 0; phase < nphase && e2 == hipSuccess; ++phase) {
            for (int i0 = 0; i0 < ns_ && e2 == hipSuccess;) {
                int i1 = i0, most = 1;
                while (i1 < ns_ && p.small_off[i1].mr == p.small_off[i0].mr)
                    most = std::max(most, p.small_off[i1++].nslices);
                if (phase == 0 || most > 1) {
                    const int mr = p.small_off[i0].mr;
                    const int nsl = p.small_prefix[i1] - p.small_prefix[i0];
                    e2 = timed(ns::kKindSmall, stream, [&] {
                        return ns::launch_small(dtype, mr, small + i0, i1 - i0, small_prefix + i0, nsl, phase,
                                                steps, co, stream);
                    });
                }
                i0 = i1;
            }
        }
        if (e2 != hipSuccess)
            return hip_fail(e2, "small-matrix kernel launch");
    }
    if (nl == 0)
        return NS_OK;
    e = timed(ns::kKindNormPartial, stream, [&] {
        return ns::launch_norm_partial(dtype, large, nl, part_prefix, p.total_parts, partials, stream);
    });
    if (e == hipSuccess)
        e = timed(ns::kKindNormFinal, stream, [&] {
            return ns::launch_norm_final(nl, part_prefix, partials, p.total_parts, inv, stream);
        });
    if (e != hipSuccess)
        return hip_fail(e, "norm kernel launch");
    if (steps == 0) {
        e = timed(ns::kKindScaleOut, stream, [&] {
            return ns::launch_scale_out(dtype, large, nl, part_prefix, p.total_parts, inv, stream);
        });
        return e == hipSuccess ? NS_OK : hip_fail(e, "scale kernel launch");
    }
    e = timed(ns::kKindPrep, stream, [&] {
        return ns::launch_prep(dtype, large, nl, prep_prefix, p.total_prep, inv, stream);
    });
    if (e != hipSuccess)
        return hip_fail(e, "normalize kernel launch");
    const int nu = (int)p.update_tiles.size();
    // a symmetric stage: its whole tiles, then (when its last round is
    // split) the half tiles, in one launch
    auto sym = [&](int stage, const ns::Tile* tl, int n, int split, int cur, int last, float ca, float cb,
                   float cc) {
        return ns::launch_gemm(dtype, stage, large, tl, n + split, n - split, cur, last, ca, cb, cc, stream);
    };
    for (int s = 0; s < steps; ++s) {
        const int cur = s & 1, last = s == steps - 1;
        const float ca = coef(s, 0), cb = coef(s, 1), cc = coef(s, 2);
        e = timed(ns::kKindSyrk, stream, [&] {
            return sym(0, syrk, (int)p.syrk_tiles.size(), p.syrk_split, cur, last, ca, cb, cc);
        });
        if (e == hipSuccess)
            e = timed(ns::kKindPoly, stream, [&] {
                return sym(1, poly, (int)p.poly_tiles.size(), p.poly_split, cur, last, ca, cb, cc);
            });
        if (e == hipSuccess)
            e = timed(ns::kKindUpdate, stream, [&] {
                return ns::launch_gemm(dtype, 2, large, upd, nu, nu, cur, last, ca, cb, cc, stream);
            });
        if (e != hipSuccess)
            return hip_fail(e, "GEMM kernel launch");
    }
    return NS_OK;
}

}  // namespace ns

extern "C" {

// Shared tail of the entry points: shapes and layout are validated.
static ns_status submit(const int64_t* shapes, const Layout& L, int32_t count, int32_t steps,
                        const float* coeffs, int32_t per_step, int32_t dtype, void* stream)
{
    bool any = false;
    for (int32_t i = 0; i < count; ++i)
        any = any || (shapes[2 * i] > 0 && shapes[2 * i + 1] > 0);
    if (!any)
        return NS_OK;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    Context* c = get_context(dev, static_cast<hipStream_t>(stream));
    std::lock_guard<std::mutex> lk(c->mu);
    return run(c, shapes, L, count, steps, coeffs, per_step, dtype);
}

// Checks common to every entry point (before any shape is looked at).
static ns_status check_common(int32_t count, int32_t steps, const float* coeffs, int32_t per_step,
                              int32_t dtype)
{
    if (count < 0)
        return fail(NS_EINVAL, "count must be >= 0");
    if (steps < 0)
        return fail(NS_EINVAL, "steps must be >= 0");
    if (steps > 0 && !coeffs)
        return fail(NS_EINVAL, "coeffs must not be NULL when steps > 0");
    if (per_step && steps > ns::kMaxScheduleSteps)
        return fail(NS_EINVAL, "a coefficient schedule holds at most " +
                                   std::to_string(ns::kMaxScheduleSteps) + " steps");
    if (dtype != NS_BF16 && dtype != NS_FP32)
        return fail(NS_EDTYPE, "unknown dtype " + std::to_string(dtype));
    return NS_OK;
}

static ns_status check_dims(int32_t i, int64_t r, int64_t c)
{
    if (r < 0 || c < 0)
        return fail(NS_EINVAL, "matrix " + std::to_string(i) + " has a negative dimension");
    if (r > (int64_t(1) << 24) || c > (int64_t(1) << 24))
        return fail(NS_EINVAL, "matrix " + std::to_string(i) + " has a dimension above 2^24");
    return NS_OK;
}

}  // extern "C"

ns_status ns::validate_batched(void* const* ptrs, const int64_t* shapes, int32_t count, int32_t steps,
                               const float* coeffs, int32_t per_step, int32_t dtype)
{
    ns_status st = check_common(count, steps, coeffs, per_step, dtype);
    if (st != NS_OK)
        return st;
    if (count > 0 && (!ptrs || !shapes))
        return fail(NS_EINVAL, "ptrs and shapes must not be NULL when count > 0");
    const size_t elt = dtype == NS_BF16 ? 2 : 4;
    for (int32_t i = 0; i < count; ++i) {
        const int64_t r = shapes[2 * i], c = shapes[2 * i + 1];
        if ((st = check_dims(i, r, c)) != NS_OK)
            return st;
        if (r == 0 || c == 0)
            continue;
        if (!ptrs[i])
            return fail(NS_EINVAL, "matrix " + std::to_string(i) + " is non-empty but its pointer is NULL");
        if (reinterpret_cast<uintptr_t>(ptrs[i]) % elt)
            return fail(NS_EINVAL, "matrix " + std::to_string(i) + " is not aligned to its element size");
    }
    return NS_OK;
}

extern "C" {

static ns_status orthogonalize(void* const* ptrs, const int64_t* shapes, int32_t count,
                               int32_t steps, const float* coeffs, int32_t per_step,
                               int32_t dtype, void* stream)
{
    g_last_error.clear();
    ns_status st = ns::validate_batched(ptrs, shapes, count, steps, coeffs, per_step, dtype);
    if (st != NS_OK)
        return st;
    Layout L;
    L.ptrs = ptrs;
    return submit(shapes, L, count, steps, coeffs, per_step, dtype, stream);
}

ns_status ns_orthogonalize_batched(void* const* ptrs, const int64_t* shapes, int32_t count,
                                   int32_t steps, const float* coeffs, int32_t dtype, void* stream)
{
    return orthogonalize(ptrs, shapes, count, steps, coeffs, 0, dtype, stream);
}

ns_status ns_orthogonalize_batched_sched(void* const* ptrs, const int64_t* shapes, int32_t count,
                                         int32_t steps, const float* coeffs, int32_t dtype,
                                         void* stream)
{
    return orthogonalize(ptrs, shapes, count, steps, coeffs, 1, dtype, stream);
}

ns_status ns_orthogonalize_chunked(void* const* chunk_ptrs, const int64_t* chunk_rows,
                                   const int32_t* nchunks, const int64_t* cols, int32_t count,
                                   int32_t steps, const float* coeffs, int32_t dtype, void* stream)
{
    g_last_error.clear();
    ns_status st = check_common(count, steps, coeffs, 0, dtype);
    if (st != NS_OK)
        return st;
    if (count > 0 && (!nchunks || !cols))
        return fail(NS_EINVAL, "nchunks and cols must not be NULL when count > 0");
    const size_t elt = dtype == NS_BF16 ? 2 : 4;
    std::vector<int64_t> shapes(2 * (size_t)count);
    int64_t total = 0;
    for (int32_t i = 0; i < count; ++i) {
        if (nchunks[i] < 0)
            return fail(NS_EINVAL, "matrix " + std::to_string(i) + " has a negative chunk count");
        total += nchunks[i];
        if (total > std::numeric_limits<int32_t>::max())
            return fail(NS_EINVAL, "too many chunks");
    }
    if (total > 0 && (!chunk_ptrs || !chunk_rows))
        return fail(NS_EINVAL, "chunk_ptrs and chunk_rows must not be NULL when there are chunks");
    int64_t k = 0;
    for (int32_t i = 0; i < count; ++i) {
        int64_t rows = 0;
        for (int32_t q = 0; q < nchunks[i]; ++q, ++k) {
            const int64_t r = chunk_rows[k];
            if (r < 0)
                return fail(NS_EINVAL, "chunk " + std::to_string(k) + " has negative rows");
            rows += r;
            if (rows > (int64_t(1) << 24))
                return fail(NS_EINVAL, "matrix " + std::to_string(i) + " has a dimension above 2^24");
            if (r > 0 && cols[i] > 0) {
                if (!chunk_ptrs[k])
                    return fail(NS_EINVAL, "chunk " + std::to_string(k) + " is non-empty but its pointer is NULL");
                if (reinterpret_cast<uintptr_t>(chunk_ptrs[k]) % elt)
                    return fail(NS_EINVAL, "chunk " + std::to_string(k) + " is not aligned to its element size");
            }
        }
        if ((st = check_dims(i, rows, cols[i])) != NS_OK)
            return st;
        shapes[2 * i] = rows;
        shapes[2 * i + 1] = cols[i];
    }
    Layout L;
    L.chunk_ptrs = chunk_ptrs;
    L.chunk_rows = chunk_rows;
    L.nchunks = nchunks;
    L.total_chunks = (int32_t)total;
    return submit(shapes.data(), L, count, steps, coeffs, 0, dtype, stream);
}

ns_status ns_workspace_bytes(const int64_t* shapes, int32_t count, int32_t dtype, size_t* out_bytes)
{
    g_last_error.clear();
    if (!out_bytes)
        return fail(NS_EINVAL, "out_bytes is NULL");
    Plan p;
    std::string err;
    int rc = ns::make_plan(shapes, count, dtype, &p, &err);
    if (rc != 0)
        return fail((ns_status)rc, err);
    *out_bytes = p.total_bytes();
    return NS_OK;
}

ns_status ns_release_workspace(void* stream)
{
    g_last_error.clear();
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    std::unique_ptr<Context> c;
    {
        std::lock_guard<std::mutex> lk(g_ctx_mu);
        auto it = g_ctx.find(std::make_pair(dev, reinterpret_cast<uintptr_t>(stream)));
        if (it == g_ctx.end())
            return NS_OK;
        c = std::move(it->second);
        g_ctx.erase(it);
    }
    std::lock_guard<std::mutex> lk(c->mu);
    drop_plans(c.get());
    if (c->ws)
        (void)hipFreeAsync(c->ws, c->stream);
    for (PinnedSlot& s : c->slots) {
        if (s.used)
            (void)hipEventSynchronize(s.done);
        (void)hipEventDestroy(s.done);
        (void)hipHostFree(s.host);
    }
    return NS_OK;
}

const char* ns_last_error(void) { return g_last_error.c_str(); }

const char* ns_version(void) { return "ns-mi355x 0.1.0 (gfx950)"; }

int64_t ns_compute_cost(int64_t rows, int64_t cols) { return ns::ns_cost(rows, cols); }

ns_status ns_plan_classify(const int64_t* shapes, int32_t count, int32_t dtype, int32_t* kinds)
{
    g_last_error.clear();
    Plan p;
    std::string err;
    int rc = ns::make_plan(shapes, count, dtype, &p, &err);
    if (rc != 0)
        return fail((ns_status)rc, err);
    if (count > 0 && !kinds)
        return fail(NS_EINVAL, "kinds is NULL");
    for (int32_t i = 0; i < count; ++i)
        kinds[i] = p.mats[i].cls;
    return NS_OK;
}

ns_status ns_plan_tiles(const int64_t* shapes, int32_t count, int32_t dtype, int32_t stage,
                        int32_t* out, int64_t capacity, int64_t* n_tiles, int32_t* tile_size)
{
    g_last_error.clear();
    if (stage < 0 || stage > 2)
        return fail(NS_EINVAL, "stage must be 0, 1 or 2");
    if (!n_tiles || (capacity > 0 && !out) || capacity < 0)
        return fail(NS_EINVAL, "bad output arguments");
    Plan p;
    std::string err;
    int rc = ns::make_plan(shapes, count, dtype, &p, &err);
    if (rc != 0)
        return fail((ns_status)rc, err);
    const std::vector<ns::Tile>& tl =
        stage == 2 ? p.update_tiles : stage == 1 ? p.poly_tiles : p.syrk_tiles;
    *n_tiles = (int64_t)tl.size();
    if (tile_size)
        *tile_size = ns::kTile;
    const int64_t nw = capacity < (int64_t)tl.size() ? capacity : (int64_t)tl.size();
    for (int64_t i = 0; i < nw; ++i) {
        const ns::PlanMat& pm = p.mats[p.large[tl[i].mat]];
        out[4 * i + 0] = pm.index;
        out[4 * i + 1] = tl[i].bi;
        out[4 * i + 2] = tl[i].bj;
        out[4 * i + 3] = stage == 0 ? pm.np : pm.mp;
    }
    return NS_OK;
}

ns_status ns_profile_enable(int32_t on)
{
    g_last_error.clear();
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (on) {
        for (ProfRec& r : g_prof_pending) {
            g_prof_free.push_back(r.start);
            g_prof_free.push_back(r.stop);
        }
        g_prof_pending.clear();
        for (int k = 0; k < ns::kNumKinds; ++k) {
            g_prof_ms[k] = 0.0;
            g_prof_n[k] = 0;
        }
    }
    g_prof_on.store(on ? 1 : 0);
    return NS_OK;
}

ns_status ns_profile_read(double* total_ms, int64_t* launches, int32_t n_kinds)
{
    g_last_error.clear();
    if (n_kinds < 0 || (n_kinds > 0 && (!total_ms || !launches)))
        return fail(NS_EINVAL, "bad output arguments");
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (ProfRec& r : g_prof_pending) {
        hipError_t e = hipEventSynchronize(r.stop);
        float ms = 0.f;
        if (e == hipSuccess)
            e = hipEventElapsedTime(&ms, r.start, r.stop);
        if (e != hipSuccess)
            return hip_fail(e, "profiling event");
        g_prof_ms[r.kind] += ms;
        g_prof_n[r.kind] += 1;
        g_prof_free.push_back(r.start);
        g_prof_free.push_back(r.stop);
    }
    g_prof_pending.clear();
    for (int k = 0; k < n_kinds && k < ns::kNumKinds; ++k) {
        total_ms[k] = g_prof_ms[k];
        launches[k] = g_prof_n[k];
    }
    for (int k = ns::kNumKinds; k < n_kinds; ++k) {
        total_ms[k] = 0.0;
        launches[k] = 0;
    }
    return NS_OK;
}

}  // extern "C"
