// ns_internal.h -- descriptors shared by the host planner and the gfx950
// kernels of libns.so. Plain structs, laid out identically on both sides.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace ns {

// Macro tile of the grouped MFMA GEMMs: 256 x 256 outputs per workgroup.
constexpr int kTile = 256;
// Matrices with min(rows, cols) <= kSmallMax (or the NS_SMALL_M environment
// variable's lower threshold, see small_threshold) run the small-matrix
// kernel, which works in fp64.
constexpr int kSmallMax = 32;
// Elements per workgroup in the norm's partial-sum pass.
constexpr int kNormChunk = 16384;
// Edge of the normalize/transpose tile.
constexpr int kPrepTile = 64;

enum Kind : int32_t {
    kKindNormPartial = 0,
    kKindNormFinal = 1,
    kKindPrep = 2,
    kKindSyrk = 3,
    kKindPoly = 4,
    kKindUpdate = 5,
    kKindSmall = 6,
    kKindScaleOut = 7,
    kNumKinds = 8
};

// One matrix of the tiled path. X is the oriented m x n matrix (m <= n),
// stored zero-padded to mp x np (multiples of kTile).
struct LargeMat {
    void* user;        // caller buffer, rows x cols row-major: G in, Y out
    void* const* rows_tab;   // or, when not NULL, row r of G / Y is rows_tab[r]
                             // (a matrix passed as row blocks)
    int64_t rows, cols;
    int32_t m, n;      // oriented dims
    int32_t mp, np;    // padded dims
    int32_t ldx;       // row pitch (elements) of xb: rows of np
    int32_t ldt;       // row pitch (elements) of xt, a, b: rows of mp
    int32_t trans;     // 1 when rows > cols (X = G^T)
    int32_t batch_index;
    int32_t part_begin, nparts;   // norm partial sums [part_begin, +nparts)
    int32_t prep_begin, nprep;    // normalize tiles   [prep_begin, +nprep)
    void* xlo;         // bf16 path: X - bf16(X), bf16, stored like X^T (np x ldt);
                       // with xt it carries X to about 17 significant bits
    void* xb[2];       // X operand copies, mp x np, ping-pong
    void* xt[2];       // X^T operand copies, np x mp, ping-pong
    void* a;           // A = X X^T, mp x mp
    void* b;           // B = bA + cA^2, mp x mp
    float* adiag;      // bf16 path: A_ii - bf16(A_ii), mp floats
    float* bdiag;      // bf16 path: B_ii - bf16(B_ii), mp floats
};

// Longest per-step coefficient schedule.
constexpr int kMaxScheduleSteps = 64;

// (a, b, c) of the steps, passed by value to the small-path kernel: step s
// uses v[3 s .. 3 s + 2] when per_step, else v[0 .. 2] (any step count).
struct SmallCoeffs {
    float v[3 * kMaxScheduleSteps];
    int32_t per_step;
};

// Small path (m <= kSmallMax): X's n columns are cut into slices of
// slice_cols columns, kSmallSlice or, for very wide matrices, a multiple of it
// that keeps a matrix at kSmallMaxSlices slices; one workgroup per slice and
// phase (norm pieces; Gram pieces; the m x m recurrence and the result).
constexpr int kSmallSlice = 512;
constexpr int kSmallMaxSlices = 256;

// One matrix of the small path.
struct SmallMat {
    void* user;
    void* const* rows_tab;   // as in LargeMat
    int64_t rows, cols;
    int32_t m, n, trans, batch_index;
    int32_t mr;              // m rounded up to a multiple of 8
    int32_t nslices, slice_cols;
    int32_t slice_begin;     // its first workgroup in a small-path launch
    double* gram;            // Gram pieces of X0 = G / (||G|| + eps): nslices x mr x mr
    double* norm;            // norm pieces: nslices sums of squares
};

// Grouped-GEMM tile: matrix index into the LargeMat array and block coords.
struct Tile {
    int32_t mat;
    int16_t bi, bj;
};
static_assert(sizeof(Tile) == 8, "tile is 8 bytes");

}  // namespace ns
