// ns_kernels.h -- launch wrappers of the gfx950 kernels (ns_kernels.hip).
// All launches are asynchronous on `stream`; each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>

#include "ns_internal.h"

namespace ns {

// Small path (min dim <= kSmallMax, fp64 arithmetic): one workgroup per
// column slice of each of `count` matrices (SmallMat, all with MR = mr,
// whose slices are workgroups slice_prefix[0] .. slice_prefix[count]).
//   phase 0   the slices' pieces of ||G||^2
//   phase 1   X0 = G / (||G|| + eps) and the slices' pieces of A0 = X0 X0^T
//             (with steps == 0: X0 written to the caller's buffer instead)
//   phase 2   A0 from its pieces; the steps on the m x m matrices,
//             B'_k = aI + b A_k + c A_k^2, Q <- B'_k Q, A_{k+1} = B'_k A_k B'_k;
//             the caller's buffer <- Q X0
// A matrix of one slice runs all of its phases in the phase-0 launch; when
// every matrix has one slice, later phases need no launch.
hipError_t launch_small(int dtype, int mr, const SmallMat* mats, int count, const int32_t* slice_prefix,
                        int nslices, int phase, int steps, const SmallCoeffs& co, hipStream_t stream);

// Sum of squares of each large matrix in kNormChunk pieces (one workgroup per
// piece; partials holds 2 total_parts floats: the pieces' scaled sums, then
// their power-of-two exponents) ...
hipError_t launch_norm_partial(int dtype, const LargeMat* mats, int nmats,
                               const int32_t* part_prefix, int total_parts,
                               float* partials, hipStream_t stream);
// ... then one workgroup per matrix folds its pieces in a fixed order into
// the pair inv[2i] = 1 / (sqrt(T) + 1e-7 2^E), inv[2i + 1] = 2^E, where
// ||G||^2 = T 2^(-2E) (E = 0 unless G has entries of 2^40 or more), so that
// X = (G 2^E) inv[2i].
hipError_t launch_norm_final(int nmats, const int32_t* part_prefix,
                             const float* partials, int total_parts, float* inv,
                             hipStream_t stream);

// X = G / (||G|| + eps), transposed when rows > cols, zero-padded to mp x np.
// bf16: writes X^T as X_hi = bf16(X) (column panels, slot 0) and
// X_lo = bf16(X - X_hi); fp32: writes X^T and X (slot 0).
hipError_t launch_prep(int dtype, const LargeMat* mats, int nmats,
                       const int32_t* prep_prefix, int total_prep,
                       const float* inv, hipStream_t stream);

// steps == 0: G <- G / (||G|| + eps) in place.
hipError_t launch_scale_out(int dtype, const LargeMat* mats, int nmats,
                            const int32_t* part_prefix, int total_parts,
                            const float* inv, hipStream_t stream);

// Grouped GEMM stages over a tile list (one workgroup per 256x256 tile).
//   stage 0: A = X X^T          (upper-triangle tiles, mirrored)
//   stage 1: B = b A + c A A    (upper-triangle tiles, mirrored)
//   stage 2: X <- a X + B X     (all tiles); `last` writes the caller buffer
// `cur` selects the X operand slot read (the other slot is written).
// tiles[0, nwhole) are whole tiles; tiles[nwhole, ntiles) (bf16 stages 0 and
// 1 only, else nwhole == ntiles) are half tiles (bit 30 of the matrix index
// selects which half of an off-diagonal tile's columns), run in the same
// launch after the whole ones.
hipError_t launch_gemm(int dtype, int stage, const LargeMat* mats,
                       const Tile* tiles, int ntiles, int nwhole, int cur, int last,
                       float a, float b, float c, hipStream_t stream);

}  // namespace ns
