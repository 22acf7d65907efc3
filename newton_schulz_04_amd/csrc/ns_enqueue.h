// ns_enqueue.h -- host pieces shared by the entry points of libns.so
// (ns_api.cpp, ns_noalloc.hip): argument validation, the metadata image of a
// plan, the kernel sequence, and the thread's error message.
#pragma once

#include <hip/hip_runtime.h>

#include <string>
#include <vector>

#include "ns.h"
#include "ns_plan.h"

namespace ns {

// Where the caller's matrices live: one contiguous row-major buffer each, or
// (chunked) a vertical stack of row blocks, matrix i taking the next
// nchunks[i] blocks of chunk_ptrs / chunk_rows.
struct Layout {
    void* const* ptrs = nullptr;
    void* const* chunk_ptrs = nullptr;
    const int64_t* chunk_rows = nullptr;
    const int32_t* nchunks = nullptr;
    int32_t total_chunks = 0;
    bool chunked() const { return chunk_ptrs != nullptr; }
};

// Sets the calling thread's ns_last_error message and returns s.
ns_status fail(ns_status s, const std::string& msg);
ns_status hip_fail(hipError_t e, const char* what);
void clear_error();

// Argument checks of ns_orthogonalize_batched(_sched) (per_step: one triple
// per step), before any HIP call.
ns_status validate_batched(void* const* ptrs, const int64_t* shapes, int32_t count, int32_t steps,
                           const float* coeffs, int32_t per_step, int32_t dtype);

// Row tables of a chunked call after the plan's metadata; returns their bytes.
size_t rowtab_layout(const Plan& p, const Layout& L, int32_t count, std::vector<size_t>* off);

// Host image of the metadata block: descriptors pointing into the workspace
// `ws`, tile lists, prefixes (and, chunked, the row tables, addressed at the
// device block `meta`). Its size is p.meta_inv (whole-matrix calls).
void build_meta(const Plan& p, const Layout& L, int32_t count, char* ws, char* meta,
                std::vector<char>* out);

// Enqueues the kernel sequence of a planned batch on `stream`: `meta` is the
// device metadata block (uploaded image, then the device-written norm
// scratch up to p.meta_end). Nothing is allocated and nothing waits (but in
// the NS_CHECK=1 debug mode, which waits after every launch).
ns_status enqueue(const Plan& p, char* meta, int32_t steps, const float* coeffs, int32_t per_step,
                  int32_t dtype, hipStream_t stream);
ns_status enqueue_launches(const Plan& p, char* meta, int32_t steps, const float* coeffs, int32_t per_step,
                           int32_t dtype, hipStream_t stream);

}  // namespace ns
