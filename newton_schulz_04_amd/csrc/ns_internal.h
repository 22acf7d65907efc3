// ns_internal.h -- descriptors shared by the host planner and the gfx950
// kernels of libns.so. Plain structs, laid out identically on both sides.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace ns {

// Macro tile of the grouped MFMA GEMMs: 256 x 256 outputs per workgroup.
constexpr int kTile = 256;
// Matrices with min(rows, cols) <= kSmallMax run the fused one-workgroup
// kernel in fp32.
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

// Iteration coefficients for the fused small path, passed by value: step s
// uses row s when per_step, else row 0 for every step.
constexpr int kMaxScheduleSteps = 64;
struct CoeffTable {
    float v[kMaxScheduleSteps][3];
    int32_t per_step;
};

// One matrix of the fused small path.
struct SmallMat {
    void* user;
    void* const* rows_tab;   // as in LargeMat
    int64_t rows, cols;
    int32_t m, n, trans, batch_index;
    float* xw;         // fp32 working copy of X, m x n
};

// Grouped-GEMM tile: matrix index into the LargeMat array and block coords.
struct Tile {
    int32_t mat;
    int16_t bi, bj;
};
static_assert(sizeof(Tile) == 8, "tile is 8 bytes");

}  // namespace ns
