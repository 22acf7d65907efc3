// ns_plan.h -- host-side batch planner: classification, cost ordering, tile
// lists and workspace layout. No HIP calls; unit-tested on the CPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "ns_internal.h"

namespace ns {

enum MatClass : int32_t { kEmpty = 0, kSmall = 1, kLarge = 2 };

// max(M,N) * min(M,N)^2 (the Megatron-LM page's Newton-Schulz cost).
int64_t ns_cost(int64_t rows, int64_t cols);

// Largest min(rows, cols) of the small-matrix path: kSmallMax, or the value
// of the environment variable NS_SMALL_M when it holds an integer in
// [0, kSmallMax] (other values are ignored). Read at every planning.
int32_t small_threshold();

struct PlanMat {
    int32_t index;          // position in the caller's batch
    int64_t rows, cols;
    int32_t m, n, mp, np, trans;
    int32_t ldx, ldt;  // row pitches in elements (see row_pitch)
    int64_t cost;
    MatClass cls;
};

// Byte offsets into the workspace; the planner lays everything out from 0.
struct LargeOffsets {
    size_t xlo, xb[2], xt[2], a, b, adiag, bdiag;
};
struct SmallOffsets {
    size_t gram, norm;
    int32_t mr, nslices, slice_cols;
};

struct Plan {
    int dtype = 0;                       // ns_dtype
    int32_t small_max = kSmallMax;       // small-path threshold the plan was made with
    size_t elt = 2;                      // operand element bytes
    std::vector<PlanMat> mats;           // one per input, batch order
    std::vector<int32_t> large;          // batch indices, launch order
    std::vector<int32_t> small;          // batch indices, launch order
    std::vector<LargeOffsets> large_off; // parallel to `large`
    std::vector<SmallOffsets> small_off; // parallel to `small`
    std::vector<int32_t> small_prefix;   // slices (workgroups) per small matrix, prefix, size nsmall+1
    int32_t total_small = 0;
    std::vector<Tile> syrk_tiles;        // stage XX^T   (upper tiles, K = np)
    std::vector<Tile> poly_tiles;        // stage bA+cA^2 (upper tiles, K = mp)
    std::vector<Tile> update_tiles;      // stage aX+BX  (all tiles,   K = mp)
    // bf16: the last syrk_split / poly_split tiles of those lists (a launch's
    // partial last round, off-diagonal) run as two half tiles each, after the
    // other tiles in the same launch; *_run is the uploaded list: the other
    // tiles, then the half tiles (bit 30 of the matrix index = which half).
    int32_t syrk_split = 0, poly_split = 0;
    std::vector<Tile> syrk_run, poly_run;
    std::vector<int32_t> part_prefix;    // size nlarge+1
    std::vector<int32_t> prep_prefix;    // size nlarge+1
    int32_t total_parts = 0, total_prep = 0;
    // Device memory: the data workspace [0, data_bytes) holds X, A, B per
    // matrix; the metadata block [0, meta_end) holds descriptors and tile
    // lists (uploaded, [0, meta_inv)) and per-call scalars (inv, partials).
    size_t data_bytes = 0;
    size_t meta_large = 0, meta_small = 0, meta_syrk = 0, meta_poly = 0, meta_update = 0,
           meta_part_prefix = 0, meta_prep_prefix = 0, meta_small_prefix = 0, meta_inv = 0,
           meta_partials = 0, meta_end = 0;
    size_t total_bytes() const { return data_bytes + meta_end; }
};

// Validates and plans. Returns 0 (NS_OK) or an ns_status code with `err`
// set. Host-only.
int make_plan(const int64_t* shapes, int32_t count, int32_t dtype, Plan* plan,
              std::string* err);

}  // namespace ns
