// ns_kernels.hip -- gfx950 (CDNA4) kernels of libns.so.
//
// The operation is Muon's quintic Newton-Schulz orthogonalization (see
// include/ns.h): X = G/(||G||_F + 1e-7), oriented so X is m x n with m <= n,
// then `steps` times A = X X^T, B = bA + cA^2, X = aX + BX.
//
// Kernels:
//   k_small        min(rows, cols) <= 32, fp64 arithmetic: the iteration
//                  through the m x m Gram matrix (one Gram matrix, the steps
//                  on m x m matrices, one product at the end); one 512-thread
//                  workgroup per 512-column slice, three launches.
//   k_norm_partial sum of squares of a 16K-element piece of G (wave shuffles).
//   k_norm_final   folds the pieces of a matrix in fixed order -> 1/(||G||+eps)
//                  (with a power-of-two prescale for entries of 2^40 or more).
//   k_prep         X = G/(||G||+eps), transposed when rows > cols, zero-padded
//                  to multiples of 256; writes X^T (bf16: X_hi = bf16(X) in
//                  column panels of 32 and X_lo = bf16(X - X_hi) row-major;
//                  fp32: X^T and X), through a 64x64 LDS tile where it must
//                  transpose.
//   k_gemm<dtype, stage, last, split>
//                  grouped 256x256 MFMA GEMM over a tile list, C = P Q^T:
//                    stage 0  P = Q = X            -> A (upper tiles, mirrored)
//                    stage 1  P = Q = A (= A^T)    -> B = bA + cA^2 (mirrored)
//                    stage 2  P = B, Q = X^T store -> X = aX + BX
//                  last: the final update writes the caller's buffer; split:
//                  a symmetric stage whose last round runs as half tiles,
//                  after the whole tiles in the same grid.
//   k_scale_out    steps == 0: G <- G/(||G||+eps).
//
// Every sum has a fixed order that does not depend on the batch, on the
// position of a matrix in it, or on trailing zero rows, so a matrix gives the
// same bits alone or in any batch.
#include <hip/hip_runtime.h>
#include <stdint.h>


#include "ns_kernels.h"

namespace ns {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 X_hi (the X^T operand of X X^T and of the update) is stored as
// column panels of 32: X^T element (r, c), r < np, c < mp, sits at
// ((c >> 5) np + r) 32 + (c & 31). A K slice of 32 of either product is then
// one panel: the update's 256 rows of it are 16 KB in one piece, and X X^T's
// 32 k-rows of a 256-column block are 8 pieces of 2 KB, so every 1 KB operand
// DMA reads one contiguous kilobyte (a row-major X^T gives the update 64-byte
// pieces, which fetch each 128-byte line twice, once per slot).
constexpr int kPanelCols = 32;
__device__ __forceinline__ int64_t pan_at(int64_t np, int64_t r, int64_t c)
{
    return ((c >> 5) * np + r) * kPanelCols + (c & 31);
}

// Element type of a dtype code (0 = bf16, 1 = fp32). Kernels are templated on
// the code rather than the type so that their names demangle in profilers.
template <int DT> struct Elt;
template <> struct Elt<0> { using type = bf16; };
template <> struct Elt<1> { using type = float; };

constexpr float kEps = 1e-7f;
constexpr int kThreads = 256;

__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }

// Global-memory view of a pointer. Caller buffers and the workspace are all
// device memory, but pointers read from descriptors are generic, and generic
// accesses compile to flat instructions, which count on both the vector
// memory and the LDS counters and may complete out of order with other
// loads: a kernel that waits for its LDS traffic (s_waitcnt lgkmcnt) then
// also waits for every flat store still in flight, and the compiler's own
// waits for a flat load become vmcnt(0), i.e. for every LDS DMA issued after
// it. The GEMM kernels therefore address global memory through this cast.
#define NS_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ NS_GLOBAL T* gbl(T* p)
{
    return (NS_GLOBAL T*)p;
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// 16-byte global store (p 16-byte aligned)
__device__ __forceinline__ void st16(void* p, uint4 v)
{
    *(NS_GLOBAL u32x4*)gbl(p) = u32x4{v.x, v.y, v.z, v.w};
}

// Row r of a caller matrix: contiguous rows of `cols` elements from `user`,
// or the row table's entry when the matrix came as row blocks.
template <typename T>
__device__ __forceinline__ T* grow(void* user, void* const* tab, int64_t cols, int64_t r)
{
    return tab ? static_cast<T*>(gbl(tab)[r]) : static_cast<T*>(user) + r * cols;
}

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }

// Four consecutive elements from four fp32 values (8-byte bf16 / 16-byte fp32
// store to global memory; the caller guarantees alignment).
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d)
{
    bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
    *(NS_GLOBAL bf16x4*)gbl(p) = v;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d)
{
    f32x4 v = {a, b, c, d};
    *(NS_GLOBAL f32x4*)gbl(p) = v;
}
__device__ __forceinline__ f32x4 load4(const bf16* p)
{
    const bf16x4 v = *(NS_GLOBAL const bf16x4*)gbl(p);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 load4(const float* p)
{
    return *(NS_GLOBAL const f32x4*)gbl(p);
}

// Butterfly sum over the 64 lanes of a wavefront (same order on every lane).
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// Sum over a 256-thread workgroup in a fixed order; every thread gets it.
__device__ __forceinline__ float block_sum(float v, float* red4)
{
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        red4[w] = v;
    __syncthreads();
    return ((red4[0] + red4[1]) + red4[2]) + red4[3];
}

// Matrix owning global block `b`: the largest i with prefix[i] <= b.
__device__ __forceinline__ int find_mat(const int32_t* prefix, int nmats, int b)
{
    int lo = 0, hi = nmats - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (prefix[mid] <= b) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Power-of-two scaling of the norm's squares. A piece of the sum of squares
// whose largest magnitude is f 2^e (f in [0.5, 1)) with e > kNormScaleExp is
// summed as (x 2^k)^2 with k = -min(e, 126), so its values lie below 4 and no
// square or sum overflows fp32; k = 0 (no scaling) otherwise, and for Inf or
// NaN, which then propagate. Scaling by 2^k is exact for normal values, so
// where nothing overflows the bits are those of the unscaled sum.
constexpr int kNormScaleExp = 40;
__device__ __forceinline__ int norm_piece_exp(float mx)
{
    if (!(mx < __builtin_inff()))
        return 0;
    int e = 0;
    (void)frexpf(mx, &e);
    return e > kNormScaleExp ? -(e < 126 ? e : 126) : 0;
}

// Scale of a matrix from its pieces: E = min k_p, T = sum_p s_p 2^(2 (E - k_p))
// (so ||G||^2 = T 2^(-2E)). Returns (1 / (sqrt(T) + eps 2^E), 2^E): X is
// (G 2^E) times the first, i.e. G / (||G|| + eps) up to one rounding, and with
// E = 0 exactly the unscaled 1 / (sqrt(sum) + eps).
__device__ __forceinline__ float2 norm_scale(float t, int e)
{
    return make_float2(1.f / (sqrtf(t) + ldexpf(kEps, e)), ldexpf(1.f, e));
}

// Largest value over a 256-thread workgroup (order-free: max is exact).
__device__ __forceinline__ float block_max(float v, float* red4)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        red4[w] = v;
    __syncthreads();
    return fmaxf(fmaxf(red4[0], red4[1]), fmaxf(red4[2], red4[3]));
}

// ---------------------------------------------------------------------------
// Small matrices (m <= 32), fp64 arithmetic.
//
// Every step of the iteration multiplies X by an m x m polynomial in its own
// Gram matrix: X_{k+1} = B'_k X_k with B'_k = aI + b A_k + c A_k^2 and
// A_k = X_k X_k^T. Since X_k = Q_k X0 with Q_k = B'_{k-1} ... B'_0 (all of
// them polynomials in A0, so symmetric and commuting), A_{k+1} =
// B'_k A_k B'_k. The small path evaluates the iteration in that form: one
// Gram matrix A0 = X0 X0^T over the n columns, the steps on m x m matrices,
// and one product Q X0 at the end: 2 m^2 n + O(m^3) multiply-adds in all
// instead of 2 m^2 n + m^3 per step, and three launches whatever the step
// count. In exact
// arithmetic it is the iteration itself; it runs in fp64 (whose vector rate
// equals the unpacked fp32 one), so only the final rounding to the
// caller's dtype is visible.
//
// X's n columns are cut into slices (SmallMat::slice_cols columns, 512 or a
// multiple), one 512-thread workgroup per slice and launch, so a batch of
// such matrices spreads over the device. Sums that cross slices (||G||^2,
// A0) go through per-slice pieces in the workspace that the next phase
// folds in slice order. MR is m rounded up to a multiple of 8: rows
// m .. MR - 1 of X are zeros, so every product is the exact m x m / m x n one
// plus zeros. Every sum has a fixed order that depends only on (m, n): a
// matrix gives the same bits in any batch, and trailing zero rows leave the
// others' bits unchanged.
constexpr int kSmallThreads = 512;
constexpr int kSmallWaves = kSmallThreads / 64;
constexpr int kSmallChunk = 256;          // columns of X0 per Gram chunk
constexpr int kSmallPx = 34;              // doubles per X0 column in LDS (>= MR + 2, 16-byte rows)
constexpr int kSmallPartDoubles = 8192;   // Gram pieces of the column groups
constexpr double kEps64 = 1e-7;
static_assert(kSmallSlice == kSmallThreads, "one column per thread in a full slice");

struct SmallLds {
    union {
        struct {
            double xs[kSmallChunk * kSmallPx];   // a chunk of X0's columns
            double part[kSmallPartDoubles];      // Gram pieces per column group
        } g;
        double mats[6][32 * 32];                 // the m x m matrices, 32 x 32, zero-padded
    };
    double red[kSmallWaves];
};

__device__ __forceinline__ double wave_sum_d(double v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// Sum over the workgroup in a fixed order; every thread gets it.
__device__ __forceinline__ double block_sum_d(double v, double* red)
{
    v = wave_sum_d(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = v;
    __syncthreads();
    double t = red[0];
#pragma unroll
    for (int w = 1; w < kSmallWaves; ++w)
        t += red[w];
    return t;
}

// Element (r, c) of X = G or G^T, r < m, c < n, from the caller's buffer.
template <typename T>
__device__ __forceinline__ double small_g(const SmallMat& S, int r, int64_t c)
{
    return (double)to_f32(S.trans ? grow<const T>(S.user, S.rows_tab, S.cols, c)[r]
                                  : grow<const T>(S.user, S.rows_tab, S.cols, r)[c]);
}

template <typename T>
__device__ __forceinline__ void small_put(const SmallMat& S, int r, int64_t c, double v)
{
    if (S.trans)
        gbl(grow<T>(S.user, S.rows_tab, S.cols, c))[r] = from_f32<T>((float)v);
    else
        gbl(grow<T>(S.user, S.rows_tab, S.cols, r))[c] = from_f32<T>((float)v);
}

// 1 / (||G|| + eps) from the slices' norm pieces (thread-strided, then the
// workgroup, in a fixed order).
__device__ __forceinline__ double small_inv(const SmallMat& S, double* red)
{
    const NS_GLOBAL double* nrm = gbl(S.norm);
    double t = 0.0;
    for (int i = threadIdx.x; i < S.nslices; i += kSmallThreads)
        t += nrm[i];
    t = block_sum_d(t, red);
    return 1.0 / (sqrt(t) + kEps64);
}

// Phase 0: the slice's piece of ||G||^2. RG threads share a column (RG = 2
// for n <= 256, else 1): thread t takes column t mod (512 / RG) of each
// 512 / RG-column chunk and rows (t / (512 / RG)) MR / RG .. + MR / RG,
// summed in order, then the workgroup in a fixed order.
template <int DT, int MR, int RG>
__device__ __forceinline__ void small_norm_piece(const SmallMat& S, int slice, SmallLds& L)
{
    using T = typename Elt<DT>::type;
    constexpr int H = MR / RG, CW = kSmallThreads / RG;
    const int tid = threadIdx.x, col = tid % CW, r0 = (tid / CW) * H;
    const int m = S.m;
    const int64_t c0 = (int64_t)slice * S.slice_cols;
    const int64_t c1 = min(c0 + S.slice_cols, (int64_t)S.n);
    double s = 0.0;
    for (int64_t c = c0 + col; c < c1; c += CW) {
        double v[H];
#pragma unroll
        for (int r = 0; r < H; ++r)
            v[r] = r0 + r < m ? small_g<T>(S, r0 + r, c) : 0.0;
#pragma unroll
        for (int r = 0; r < H; ++r)
            s = fma(v[r], v[r], s);
    }
    s = block_sum_d(s, L.red);
    if (threadIdx.x == 0)
        gbl(S.norm)[slice] = s;
}

// Phase 1: the slice's piece of A0 = X0 X0^T, in chunks of 256 columns of X0
// staged in LDS (threads t and t + 256 fill the two halves of column t's
// rows): 4 x 4 blocks of A0 per thread (NBLK = (MR / 4)^2 blocks), the
// 512 / NBLK column groups summed in group order. With `out` (no steps) X0
// goes to the caller's buffer instead.
template <int DT, int MR>
__device__ __forceinline__ void small_gram_piece(const SmallMat& S, int slice, bool out, SmallLds& L)
{
    using T = typename Elt<DT>::type;
    constexpr int NB = MR / 4, NBLK = NB * NB, G = kSmallThreads / NBLK, MM = MR * MR, H = MR / 2;
    static_assert(G * MM <= kSmallPartDoubles, "Gram pieces exceed their LDS");
    const int tid = threadIdx.x, col = tid % kSmallChunk, r0 = (tid / kSmallChunk) * H;
    const int m = S.m;
    const int64_t c0 = (int64_t)slice * S.slice_cols;
    const int64_t c1 = min(c0 + S.slice_cols, (int64_t)S.n);
    const double inv = small_inv(S, L.red);
    const int blk = tid % NBLK, kg = tid / NBLK, ti = blk / NB, tj = blk % NB;
    double acc[4][4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            acc[p][q] = 0.0;
    for (int64_t cc0 = c0; cc0 < c1; cc0 += kSmallChunk) {
        const int64_t c = cc0 + col;
        const int ncols = (int)min((int64_t)kSmallChunk, c1 - cc0);
        double x[H];
#pragma unroll
        for (int r = 0; r < H; ++r)
            x[r] = (c < c1 && r0 + r < m) ? small_g<T>(S, r0 + r, c) * inv : 0.0;
        if (out) {
            if (c < c1) {
#pragma unroll
                for (int r = 0; r < H; ++r)
                    if (r0 + r < m)
                        small_put<T>(S, r0 + r, c, x[r]);
            }
            continue;
        }
#pragma unroll
        for (int r = 0; r < H; r += 2)
            *reinterpret_cast<double2*>(L.g.xs + col * kSmallPx + r0 + r) = make_double2(x[r], x[r + 1]);
        __syncthreads();
        if (kg < G) {
            for (int jj = kg; jj < ncols; jj += G) {
                const double* xc = L.g.xs + jj * kSmallPx;
                const double2 a0 = *reinterpret_cast<const double2*>(xc + 4 * ti);
                const double2 a1 = *reinterpret_cast<const double2*>(xc + 4 * ti + 2);
                const double2 b0 = *reinterpret_cast<const double2*>(xc + 4 * tj);
                const double2 b1 = *reinterpret_cast<const double2*>(xc + 4 * tj + 2);
                const double xr[4] = {a0.x, a0.y, a1.x, a1.y}, xq[4] = {b0.x, b0.y, b1.x, b1.y};
#pragma unroll
                for (int p = 0; p < 4; ++p)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[p][q] = fma(xr[p], xq[q], acc[p][q]);
            }
        }
        __syncthreads();
    }
    if (out)
        return;
    if (kg < G) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                L.g.part[(kg * MR + 4 * ti + p) * MR + 4 * tj + q] = acc[p][q];
    }
    __syncthreads();
    NS_GLOBAL double* gq = gbl(S.gram) + (size_t)slice * MM;
    for (int e = tid; e < MM; e += kSmallThreads) {
        double v = L.g.part[e];
        for (int k = 1; k < G; ++k)
            v += L.g.part[k * MM + e];
        gq[e] = v;
    }
}

// Z = X^T Y for 32 x 32 matrices in LDS (row-major, zero outside the m x m
// corner but for the identity parts of B', which keep every product
// block-diagonal): with X symmetric, X Y. fp64 MFMA 16 x 16 x 4: wavefront
// w < 4 computes output block (w >> 1, w & 1), eight MFMAs over k. Lane l's
// operands are a = X^T[16 bi + l % 16][4 kb + l / 16] = X[4 kb + l / 16][16 bi
// + l % 16] and b = Y[4 kb + l / 16][16 bj + l % 16] (both rows read across 16
// lanes); accumulator register r of lane l is Z[16 bi + 4 r + l / 16][16 bj +
// l % 16] (lane layout checked with an in-bounds probe on gfx950).
constexpr int kMx = 32;
typedef double d4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void small_mm(const double* X, const double* Y, double* Z)
{
    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
    if (wave < 4) {
        const int bi = wave >> 1, bj = wave & 1, kl = l >> 4, il = l & 15;
        d4 c = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int kb = 0; kb < kMx / 4; ++kb) {
            const double a = X[(4 * kb + kl) * kMx + 16 * bi + il];
            const double b = Y[(4 * kb + kl) * kMx + 16 * bj + il];
            c = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Z[(16 * bi + 4 * r + kl) * kMx + 16 * bj + il] = c[r];
    }
    __syncthreads();
}

// Phase 2: A0 from the slices' pieces (in slice order, eight pieces' loads
// in flight at once); the steps on the m x m matrices; Y = Q X0 on the
// slice's columns, written to the caller's buffer (RG threads per column as
// in phase 0, each taking its rows).
template <int DT, int MR, int RG>
__device__ __forceinline__ void small_finish(const SmallMat& S, int slice, int steps, const SmallCoeffs& co,
                                             SmallLds& L)
{
    using T = typename Elt<DT>::type;
    constexpr int MM = MR * MR, H = MR / RG, CW = kSmallThreads / RG;
    const int tid = threadIdx.x, col = tid % CW, r0 = (tid / CW) * H;
    const int m = S.m;
    const int64_t c0 = (int64_t)slice * S.slice_cols;
    const int64_t c1 = min(c0 + S.slice_cols, (int64_t)S.n);
    double* A = L.mats[0];
    double* Sq = L.mats[1];
    double* P = L.mats[2];
    double* Q = L.mats[3];
    double* T2 = L.mats[4];
    double* W = L.mats[5];

    // A0 (32 x 32, zero outside the MR x MR pieces)
    const NS_GLOBAL double* gp = gbl(S.gram);
    constexpr int EPX = kMx * kMx / kSmallThreads;
    double av[EPX];
#pragma unroll
    for (int i = 0; i < EPX; ++i)
        av[i] = 0.0;
    for (int q = 0; q < S.nslices; q += 8) {
        double t[8][EPX];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int i = 0; i < EPX; ++i) {
                const int x = tid + kSmallThreads * i, r = x / kMx, c = x % kMx;
                t[u][i] = (q + u < S.nslices && r < MR && c < MR) ? gp[(size_t)(q + u) * MM + r * MR + c] : 0.0;
            }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int i = 0; i < EPX; ++i)
                if (q + u < S.nslices)
                    av[i] += t[u][i];
    }
#pragma unroll
    for (int i = 0; i < EPX; ++i)
        A[tid + kSmallThreads * i] = av[i];
    const double inv = small_inv(S, L.red);   // (its barriers also publish A)

    // the steps: B'_k = aI + b A_k + c A_k^2; Q <- B'_k Q; A <- A B'_k^2
    // (the padding rows and columns only ever meet the identity: every
    // product stays zero outside the m x m corner but on the diagonal)
    for (int k = 0; k < steps; ++k) {
        const float* c3 = co.v + (co.per_step ? 3 * k : 0);
        const double ca = c3[0], cb = c3[1], cc = c3[2];
        small_mm(A, A, Sq);
        for (int e = tid; e < kMx * kMx; e += kSmallThreads) {
            const double v = cb * A[e] + cc * Sq[e];
            P[e] = e / kMx == e % kMx ? v + ca : v;
        }
        __syncthreads();
        if (k == 0) {
            for (int e = tid; e < kMx * kMx; e += kSmallThreads)
                Q[e] = P[e];
            __syncthreads();
        } else {
            small_mm(P, Q, W);
            double* sw = Q; Q = W; W = sw;
        }
        if (k + 1 < steps) {
            small_mm(P, P, T2);
            small_mm(A, T2, W);
            double* sw = A; A = W; W = sw;
        }
    }

    // Y = Q X0 (Q's row i read as 16-byte pieces, the same address in every lane)
    for (int64_t c = c0 + col; c < c1; c += CW) {
        double x[MR];
#pragma unroll
        for (int r = 0; r < MR; ++r)
            x[r] = r < m ? small_g<T>(S, r, c) * inv : 0.0;
#pragma unroll 2
        for (int r = 0; r < H; ++r) {
            const int row = r0 + r;
            double y0 = 0.0, y1 = 0.0;
#pragma unroll
            for (int t = 0; t < MR; t += 2) {
                const double2 q2 = *reinterpret_cast<const double2*>(Q + row * kMx + t);
                y0 = fma(q2.x, x[t], y0);
                y1 = fma(q2.y, x[t + 1], y1);
            }
            if (row < m)
                small_put<T>(S, row, c, y0 + y1);
        }
    }
}

// Phases [p0, p1) of one slice, in order. A matrix of one slice runs every
// phase in the launch of phase 0 (the same code in the same order, so the
// same bits) and its workgroup returns at once in the later launches;
// between the phases its pieces pass through global memory within the
// workgroup, ordered by __syncthreads.
template <int DT, int MR, int RG>
__device__ __forceinline__ void small_phases(const SmallMat& S, int slice, int p0, int p1, int steps,
                                             const SmallCoeffs& co, SmallLds& L)
{
    for (int ph = p0; ph < p1; ++ph) {
        if (ph > p0)
            __syncthreads();
        if (ph == 0)
            small_norm_piece<DT, MR, RG>(S, slice, L);
        else if (ph == 1)
            small_gram_piece<DT, MR>(S, slice, steps == 0, L);
        else
            small_finish<DT, MR, RG>(S, slice, steps, co, L);
    }
}

// One launch covers the small matrices of one MR (the planner groups them);
// workgroup b (counted from prefix[0]) is slice b - prefix[i] of matrix i.
template <int DT, int MR>
__global__ __launch_bounds__(kSmallThreads) void k_small(const SmallMat* __restrict__ mats, int nmats,
                                                         const int32_t* __restrict__ prefix, int phase,
                                                         int steps, const SmallCoeffs co)
{
    __shared__ __attribute__((aligned(16))) SmallLds L;
    const int b = prefix[0] + (int)blockIdx.x;
    const int mi = find_mat(prefix, nmats, b);
    const SmallMat& S = mats[mi];
    const int slice = b - prefix[mi];
    const int last = steps > 0 ? 2 : 1;   // the last phase
    int p0 = phase, p1 = phase + 1;
    if (S.nslices == 1)
        p1 = phase == 0 ? last + 1 : phase;
    if (S.n <= kSmallThreads / 2)   // two threads per column
        small_phases<DT, MR, 2>(S, slice, p0, p1, steps, co, L);
    else
        small_phases<DT, MR, 1>(S, slice, p0, p1, steps, co, L);
}

// Norm, pass 1: one workgroup per kNormChunk-element piece of a matrix (in its
// row-major order). partials[b] is the piece's sum of squares, scaled by
// 2^(2 k) with k = partials[total + b] (see norm_piece_exp).
template <int DT>
__global__ __launch_bounds__(kThreads) void k_norm_partial(const LargeMat* __restrict__ mats,
                                                           int nmats,
                                                           const int32_t* __restrict__ prefix,
                                                           float* __restrict__ partials, int total)
{
    using T = typename Elt<DT>::type;
    __shared__ float red[4];
    constexpr int V = 16 / sizeof(T);
    constexpr int Q = kNormChunk / (kThreads * V);
    const int b = blockIdx.x;
    const int mi = find_mat(prefix, nmats, b);
    const LargeMat& M = mats[mi];
    const int64_t base = (int64_t)(b - prefix[mi]) * kNormChunk;
    const int64_t left = M.rows * M.cols - base;
    const T* g = static_cast<const T*>(M.user) + base;
    const int tid = threadIdx.x;
    // this thread's Q x V elements, in order (zeros past the matrix's end)
    float f[Q][V];
    if (M.rows_tab) {
        // row blocks: the same elements in the same order, found row by row
#pragma unroll
        for (int q = 0; q < Q; ++q)
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const int64_t idx = (int64_t)(tid + kThreads * q) * V + e;
                f[q][e] = 0.f;
                if (idx < left) {
                    const int64_t flat = base + idx;
                    f[q][e] = to_f32(grow<const T>(nullptr, M.rows_tab, M.cols, flat / M.cols)[flat % M.cols]);
                }
            }
    } else if (left >= kNormChunk && (reinterpret_cast<uintptr_t>(g) & 15) == 0) {
        typedef T vec_t __attribute__((ext_vector_type(V)));
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const vec_t v = *reinterpret_cast<const vec_t*>(g + (int64_t)(tid + kThreads * q) * V);
#pragma unroll
            for (int e = 0; e < V; ++e)
                f[q][e] = to_f32(v[e]);
        }
    } else {
#pragma unroll
        for (int q = 0; q < Q; ++q)
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const int64_t idx = (int64_t)(tid + kThreads * q) * V + e;
                f[q][e] = idx < left ? to_f32(g[idx]) : 0.f;
            }
    }
    float mx = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int e = 0; e < V; ++e)
            mx = fmaxf(mx, fabsf(f[q][e]));
    const int k = norm_piece_exp(block_max(mx, red));
    const float p2 = ldexpf(1.f, k);
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const float v = f[q][e] * p2;
            s = fmaf(v, v, s);
        }
    s = block_sum(s, red);
    if (tid == 0) {
        partials[b] = s;
        partials[total + b] = (float)k;
    }
}

// Norm, pass 2: one workgroup per matrix. E = min over its pieces of k; the
// pieces' sums brought to scale 2^(2E) are added in a fixed order (thread t
// takes pieces t, t+256, ...). scale[2 mi], scale[2 mi + 1] = norm_scale.
__global__ __launch_bounds__(kThreads) void k_norm_final(const int32_t* __restrict__ prefix,
                                                         const float* __restrict__ partials, int total,
                                                         float* __restrict__ scale)
{
    __shared__ float red[4];
    const int mi = blockIdx.x;
    const int p0 = prefix[mi], np = prefix[mi + 1] - p0;
    float kmin = 0.f;
    for (int i = threadIdx.x; i < np; i += kThreads)
        kmin = fminf(kmin, partials[total + p0 + i]);
    const int e = -(int)block_max(-kmin, red);
    float s = 0.f;
    for (int i = threadIdx.x; i < np; i += kThreads)
        s += ldexpf(partials[p0 + i], 2 * (e - (int)partials[total + p0 + i]));
    s = block_sum(s, red);
    if (threadIdx.x == 0) {
        const float2 sc = norm_scale(s, e);
        scale[2 * mi] = sc.x;
        scale[2 * mi + 1] = sc.y;
    }
}

// steps == 0: G <- (G 2^E) inv, same pieces as the norm.
template <int DT>
__global__ __launch_bounds__(kThreads) void k_scale_out(const LargeMat* __restrict__ mats,
                                                        int nmats,
                                                        const int32_t* __restrict__ prefix,
                                                        const float* __restrict__ inv)
{
    using T = typename Elt<DT>::type;
    const int b = blockIdx.x;
    const int mi = find_mat(prefix, nmats, b);
    const LargeMat& M = mats[mi];
    const int64_t base = (int64_t)(b - prefix[mi]) * kNormChunk;
    const int64_t left = M.rows * M.cols - base;
    const float s = inv[2 * mi], p2 = inv[2 * mi + 1];
    for (int i = threadIdx.x; i < kNormChunk; i += kThreads)
        if (i < left) {
            const int64_t flat = base + i;
            T* row = grow<T>(M.user, M.rows_tab, M.cols, flat / M.cols);
            row[flat % M.cols] = from_f32<T>(to_f32(row[flat % M.cols]) * p2 * s);
        }
}

// ---------------------------------------------------------------------------
// Normalize + orient + pad: one workgroup per 64x64 tile of the padded X.
template <typename T>
__device__ __forceinline__ void put_x(const LargeMat& M, int64_t i, int64_t j, float v)
{
    if (M.xb[0])
        static_cast<T*>(M.xb[0])[i * M.ldx + j] = from_f32<T>(v);
}
template <typename T>
__device__ __forceinline__ void put_xt(const LargeMat& M, int64_t i, int64_t j, float v)
{
    const T hi = from_f32<T>(v);
    static_cast<T*>(M.xt[0])[j * M.ldt + i] = hi;
    if (M.xlo)   // bf16 path: the part of X that bf16 drops
        static_cast<T*>(M.xlo)[j * M.ldt + i] = from_f32<T>(v - to_f32(hi));
}

template <int DT>
__global__ __launch_bounds__(kThreads) void k_prep(const LargeMat* __restrict__ mats, int nmats,
                                                   const int32_t* __restrict__ prefix,
                                                   const float* __restrict__ inv)
{
    using T = typename Elt<DT>::type;
    __shared__ float tile[kPrepTile][kPrepTile + 1];
    const int b = blockIdx.x;
    const int mi = find_mat(prefix, nmats, b);
    const LargeMat& M = mats[mi];
    const int local = b - prefix[mi];
    const int per_row = M.np / kPrepTile;
    const int64_t i0 = (int64_t)(local / per_row) * kPrepTile;
    const int64_t j0 = (int64_t)(local % per_row) * kPrepTile;
    // X = (G 2^E) s (see k_norm_final); 2^E = 1 unless G has huge entries
    const float s = inv[2 * mi], p2 = inv[2 * mi + 1];
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    if constexpr (DT == 0) {
        if (M.trans) {
            // bf16, rows > cols: X^T = G row for row, so no transpose. Thread
            // t writes elements i0 + 16 (t & 3) .. + 15 of X^T row j0 + (t >> 2)
            // (X_hi and X_lo) with 16-byte accesses where the row allows.
            const int64_t j = j0 + (threadIdx.x >> 2);
            const int64_t i = i0 + 16 * (threadIdx.x & 3);
            const bf16* src = grow<const bf16>(M.user, M.rows_tab, M.cols, j < M.n ? j : 0) + i;
            float v[16];
            if (j < M.n && i + 16 <= M.m && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(src);
                const bf16x8 b = *reinterpret_cast<const bf16x8*>(src + 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    v[e] = (float)a[e] * p2 * s;
                    v[8 + e] = (float)b[e] * p2 * s;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    v[e] = (j < M.n && i + e < M.m) ? to_f32(src[e]) * p2 * s : 0.f;
            }
            bf16x8 h[2], l[2];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const bf16 hb = (bf16)v[e];
                h[e >> 3][e & 7] = hb;
                l[e >> 3][e & 7] = (bf16)(v[e] - (float)hb);
            }
            // (i is a multiple of 16: the 16 elements stay in one panel)
            bf16* xt = static_cast<bf16*>(M.xt[0]) + pan_at(M.np, j, i);
            bf16* xl = static_cast<bf16*>(M.xlo) + j * M.ldt + i;
            *reinterpret_cast<bf16x8*>(xt) = h[0];
            *reinterpret_cast<bf16x8*>(xt + 8) = h[1];
            *reinterpret_cast<bf16x8*>(xl) = l[0];
            *reinterpret_cast<bf16x8*>(xl + 8) = l[1];
            return;
        }
        // bf16, rows <= cols: X = G, X^T through the LDS tile. Thread t reads
        // 16 consecutive elements of G row i0 + (t >> 2) (16-byte loads where
        // the row allows) and later writes 16 consecutive elements of X^T row
        // j0 + (t >> 2); the column reads tile[16 q + e][jj] hit 64 distinct
        // banks across a wavefront (row pitch 65 floats).
        {
            const int r = threadIdx.x >> 2, q = threadIdx.x & 3;
            const int64_t i = i0 + r, j = j0 + 16 * q;
            const bf16* src = grow<const bf16>(M.user, M.rows_tab, M.cols, i < M.m ? i : 0) + j;
            if (i < M.m && j + 16 <= M.n && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(src);
                const bf16x8 b = *reinterpret_cast<const bf16x8*>(src + 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    tile[r][16 * q + e] = (float)a[e] * p2 * s;
                    tile[r][16 * q + 8 + e] = (float)b[e] * p2 * s;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    tile[r][16 * q + e] = (i < M.m && j + e < M.n) ? to_f32(src[e]) * p2 * s : 0.f;
            }
            __syncthreads();
            bf16x8 h[2], l[2];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float v = tile[16 * q + e][r];
                const bf16 hb = (bf16)v;
                h[e >> 3][e & 7] = hb;
                l[e >> 3][e & 7] = (bf16)(v - (float)hb);
            }
            const int64_t jt = j0 + r, it = i0 + 16 * q;   // X^T row, first element
            bf16* xt = static_cast<bf16*>(M.xt[0]) + pan_at(M.np, jt, it);
            bf16* xl = static_cast<bf16*>(M.xlo) + jt * M.ldt + it;
            *reinterpret_cast<bf16x8*>(xt) = h[0];
            *reinterpret_cast<bf16x8*>(xt + 8) = h[1];
            *reinterpret_cast<bf16x8*>(xl) = l[0];
            *reinterpret_cast<bf16x8*>(xl + 8) = l[1];
            return;
        }
    }
    if (!M.trans) {
        // X[i][j] = G[i][j]: read G rows, write X direct, X^T through LDS.
        for (int p = 0; p < 16; ++p) {
            const int r = ty + 4 * p;
            const int64_t i = i0 + r, j = j0 + tx;
            const float v = (i < M.m && j < M.n) ? to_f32(grow<const T>(M.user, M.rows_tab, M.cols, i)[j]) * p2 * s : 0.f;
            tile[r][tx] = v;
            put_x<T>(M, i, j, v);
        }
        __syncthreads();
        for (int p = 0; p < 16; ++p) {
            const int r = ty + 4 * p;
            put_xt<T>(M, i0 + tx, j0 + r, tile[tx][r]);
        }
    } else {
        // X[i][j] = G[j][i] (G is n x m): read G rows = X columns, write X^T
        // direct, X through LDS.
        for (int p = 0; p < 16; ++p) {
            const int r = ty + 4 * p;
            const int64_t j = j0 + r, i = i0 + tx;
            const float v = (i < M.m && j < M.n) ? to_f32(grow<const T>(M.user, M.rows_tab, M.cols, j)[i]) * p2 * s : 0.f;
            tile[r][tx] = v;
            put_xt<T>(M, i, j, v);
        }
        __syncthreads();
        for (int p = 0; p < 16; ++p) {
            const int r = ty + 4 * p;
            put_x<T>(M, i0 + r, j0 + tx, tile[tx][r]);
        }
    }
}

// ---------------------------------------------------------------------------
// Grouped GEMM, C = P Q^T on a 256x256 tile, in general both operands
// row-major with K contiguous (bf16 operands are also read as k-rows or from
// X_hi's column panels, see k_gemm). One workgroup of 4 wavefronts (2 x 2),
// each wavefront 128x128 = 4x4 MFMA blocks of 32x32 (16 fp32 accumulators
// per lane per block). The tile is as large as the accumulators allow (the
// 256 AGPRs of each lane), and it sets what the kernels cost: 32 KB of
// operands per 32-deep slot, streamed from L2 at ~12 TB/s over the chip,
// whose power is what lowers the shader clock under these kernels.
//
// K advances in slots of 64 bytes per row (32 bf16 / 16 fp32): one slot of
// one operand is 256 rows x 64 B = 16 KB, and P and Q slots go through a ring
// of four LDS slots (32 KB each). While slot s is multiplied, slots s + 1 ..
// s + 3 stream in: 96 KB of operand loads in flight per compute unit. The
// global -> L2 -> LDS stream is latency-bound at this depth (measured: with one
// 64 KB stage in flight it moved ~11.6 TB/s, with two ~18 TB/s), which is why
// the ring is deep rather than the stages large. Global -> LDS moves use
// buffer_load_dwordx4 ... lds: each lane's 16 bytes land at M0 + 16 * lane, so
// one wavefront instruction fills 1 KB of LDS, and which global chunk a lane
// fetches decides the LDS layout.
//
// LDS layout of a slot operand: row r occupies the 64 bytes at r * 64; its
// logical 16-byte chunk c (0..3) is stored at chunk c ^ g(r), g(r) = (r >> 2) & 3.
// A 16-lane group of an MFMA operand read touches 16 consecutive rows at one
// logical chunk; rows r and r + 4j share a 64-byte bank window and g gives
// them distinct chunks, so the group covers all 64 banks once.
//
// Lane l of an MFMA operand read takes row (l & 31) of its 32-row block and
// logical chunk 2*ks + (l >> 5); A and B operands use the same (lane group,
// element) -> k assignment, so every k meets itself.
// (A slot holds k-steps 0 and 1.)
//   bf16: a chunk is 8 values = one v_mfma_f32_32x32x16_bf16.
//   fp32: a chunk is 4 values = four v_mfma_f32_32x32x2_f32, element e of both
//         lane groups in MFMA e.
// Accumulator register r of lane l holds row (r>>2)*8 + (l>>5)*4 + (r&3), column
// l & 31 of the 32x32 block.
constexpr int kSlotRowBytes = 64;
constexpr int kSlotOpBytes = kTile * kSlotRowBytes;   // 16 KB

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int H> struct Peel { static constexpr int value = H; };

template <typename OpT> struct Mfma;
template <> struct Mfma<bf16> {
    __device__ static __forceinline__ void mac(f32x16& acc, const uint4& a, const uint4& b)
    {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
};
template <> struct Mfma<float> {
    __device__ static __forceinline__ void mac(f32x16& acc, const uint4& a, const uint4& b)
    {
        const f32x4 av = __builtin_bit_cast(f32x4, a), bv = __builtin_bit_cast(f32x4, b);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[0], bv[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[1], bv[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[2], bv[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[3], bv[3], acc, 0, 0, 0);
    }
};

// Byte offset of (row r, logical chunk c) inside a slot operand.
__device__ __forceinline__ int lds_swz(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int lds_off(int r, int c) { return r * kSlotRowBytes + ((c ^ lds_swz(r)) << 4); }

// X X^T on the bf16 path reads X from its transposed copy X^T (np x mp), so
// no row-major copy of X is kept. A slot of an operand is then 32 rows of
// X^T (32 k) x 256 columns (256 rows of X): 32 LDS rows of 512 bytes, the
// 16-byte chunk c of row k stored at chunk c ^ ((k & 3) << 2).
//
// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, the 16 8-byte
// chunks the lanes address form a 4 x 16 matrix of 16-bit values (row r =
// the chunks of lanes 4r..4r+3) and lane j receives column j. Lane x of a
// group addressing row k0 + x/4, columns i0 + 4 (x % 4) .. +3 of the k-tile
// therefore receives the four values at rows k0..k0+3 of column i0 + x:
// four consecutive k of one row of X, half an MFMA operand.
template <typename T> struct IsBf16 { static constexpr bool value = false; };
template <> struct IsBf16<bf16> { static constexpr bool value = true; };
constexpr int kTrRowBytes = 512;
__device__ __forceinline__ int tr_swz(int k) { return (k & 3) << 2; }
typedef short v4i16 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 ds_read_tr(const char* p)
{
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(p)));
}

// After the K loop the four LDS slots (128 KB) hold one 256 x 256 bf16 tile
// for the epilogues: row R (0..255) is 512 bytes at (R & 63) * 512 of slot
// R >> 6, and its 16-byte chunk q (elements 8q .. 8q + 7) is stored at chunk
// q ^ (R & 31). Accesses of 32 rows x one chunk (the accumulator order) and of
// whole rows then spread over the LDS banks, and global memory sees whole
// 512-byte rows instead of 16-byte pieces of 32 rows. The slots are separate
// objects, so code picks a slot pointer by values it knows statically or per
// wavefront, never by a per-lane row.

// element x (0..255) of row R, R in the slot starting at `slot`
__device__ __forceinline__ char* tile_at(char* slot, int R, int x)
{
    return slot + (R & 63) * 512 + (((x >> 3) ^ (R & 31)) << 4) + (x & 7) * 2;
}

// Whole-tile copy from the LDS tile to global rows of 256 bf16 at a pitch of
// ld elements. Wavefront w moves rows 64w .. 64w + 63 (its slot `ws`), two
// per instruction (lanes 0-31 and 32-63), lane p = l & 31 taking stored chunk p.
// own >= 0: only the columns of 64-column pieces own and own + 2 (a half
// tile's), i.e. logical chunks c with (c >> 3) & 1 == own.
__device__ __forceinline__ void tile_store(const char* ws, bf16* dst, int64_t ld, int wave, int lane,
                                           int own = -1)
{
    const int half = lane >> 5, p = lane & 31;
#pragma unroll 4
    for (int q = 0; q < 32; ++q) {
        const int R = wave * 64 + 2 * q + half;
        const int c = p ^ (R & 31);
        const uint4 v = *reinterpret_cast<const uint4*>(ws + (2 * q + half) * 512 + p * 16);
        if (own < 0 || ((c >> 3) & 1) == own)
            st16(dst + R * ld + 8 * c, v);
    }
}

// Whole-tile copy from the LDS tile into the panel layout of X_hi: tile row
// R is X^T row r0 + R, its 256 elements are panels pc0 .. pc0 + 7 (64 bytes
// each). One instruction writes one panel's 16 consecutive rows, a contiguous
// kilobyte: lane l = 16 g + 4 a + b takes row 16 rb + g + 4 a, chunk b of
// panel pp. Within a 16-lane group the stored chunks ((4 pp + b) ^ (R & 31))
// differ in bits 0-1 (b ^ g) and 2-3 ((pp ^ a) & 3), so the group covers all
// 64 LDS banks once.
__device__ __forceinline__ void tile_store_pan(const char* ws, bf16* xt, int64_t np, int64_t r0, int64_t pc0,
                                               int wave, int lane)
{
    const int g = lane >> 4, a = (lane >> 2) & 3, b = lane & 3;
#pragma unroll 4
    for (int q = 0; q < 32; ++q) {
        const int rb = q >> 3, pp = q & 7;
        const int R = wave * 64 + 16 * rb + g + 4 * a;
        const uint4 v = *reinterpret_cast<const uint4*>(ws + (R & 63) * 512 + (((4 * pp + b) ^ (R & 31)) << 4));
        st16(xt + ((pc0 + pp) * np + r0 + R) * kPanelCols + 8 * b, v);
    }
}

// Whole-tile copy into the caller's matrix (the last step): tile row R goes
// to row row0 + R of the caller's buffer (rows of `cols` elements, or the row
// table), elements col0 .. col0 + 255; rows >= nrows and elements >= ncols
// (the padding) are not written. Same lane mapping as tile_store.
__device__ __forceinline__ void tile_store_user(const char* ws, bf16* user, void* const* rows_tab, int64_t cols,
                                                int64_t row0, int64_t nrows, int64_t col0, int64_t ncols,
                                                int wave, int lane)
{
    const int half = lane >> 5, p = lane & 31;
#pragma unroll 4
    for (int q = 0; q < 32; ++q) {
        const int R = wave * 64 + 2 * q + half;
        const int64_t row = row0 + R, c0 = col0 + 8 * (p ^ (R & 31));
        const uint4 v = *reinterpret_cast<const uint4*>(ws + (2 * q + half) * 512 + p * 16);
        if (row < nrows) {
            bf16* dst = grow<bf16>(user, rows_tab, cols, row) + c0;
            if (c0 + 8 <= ncols && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
                st16(dst, v);
            } else {
                const bf16x8 h = __builtin_bit_cast(bf16x8, v);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (c0 + e < ncols)
                        gbl(dst)[e] = h[e];
            }
        }
    }
}

// Writes a 256 x 256 bf16 tile held in the accumulator order (hv[i][j][rg]:
// rows r0 .. r0 + 3 of column c, r0 = 128 wr + 32 i + 8 rg + 4 fg,
// c = 128 wc + 32 j + fr) into the LDS tile with LDS row = tile row (slot
// r >> 6 = 2 wr + (i >> 1): rs0 for i < 2, rs1 otherwise). Lanes fr and
// fr ^ 1 hold adjacent columns of the same four rows; one exchange of a dword
// gives each of them two rows of a column pair, written as 4-byte pieces:
// an even lane keeps rows r0, r0+1 (d.x) for columns c, c+1, an odd lane
// rows r0+2, r0+3 (d.y) for columns c-1, c. v_perm_b32 picks the 16-bit
// halves (bytes 0..3 = the kept dword, 4..7 = the received one).
template <int NJ>
__device__ __forceinline__ void write_tile_by_rows(char* rs0, char* rs1, const uint2 (&hv)[4][NJ][4], int wr,
                                                   int wc, int fr, int fg, int jbase = 0)
{
    const uint32_t odd = fr & 1;
    const uint32_t keep_y = 0u - odd;
    const uint32_t sel0 = odd ? 0x01000504u : 0x05040100u;
    const uint32_t sel1 = odd ? 0x03020706u : 0x07060302u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        char* rslot = i < 2 ? rs0 : rs1;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int c = wc * 128 + (jbase + j) * 32 + fr;
                const int r0 = wr * 128 + i * 32 + rg * 8 + fg * 4;
                const uint2 d = hv[i][j][rg];   // x: rows r0, r0+1; y: rows r0+2, r0+3
                const uint32_t mine = (d.y & keep_y) | (d.x & ~keep_y);
                const uint32_t send = (d.x & keep_y) | (d.y & ~keep_y);
                // lane fr ^ 1 (same rows, column c ^ 1)
                const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);
                const uint32_t w0 = __builtin_amdgcn_perm(recv, mine, sel0);
                const uint32_t w1 = __builtin_amdgcn_perm(recv, mine, sel1);
                const int rr = r0 + 2 * (int)odd;
                const int cc0 = c - (int)odd;
                *reinterpret_cast<uint32_t*>(tile_at(rslot, rr, cc0)) = w0;
                *reinterpret_cast<uint32_t*>(tile_at(rslot, rr + 1, cc0)) = w1;
            }
    }
}

#define NS_WAIT_ALL_BARRIER() asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")
#define NS_WAIT_DMA_BARRIER() asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory")
#define NS_WAIT_LDS_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

// In the epilogues, lane (fr, fg) of wavefront (wr, wc) holds, in block
// (i, j) register 4 rg + e, tile element (r, c) with
// r = 128 wr + 32 i + 8 rg + 4 fg + e and c = 128 wc + 32 j + fr: four
// consecutive r of one c, i.e. 8 bytes of LDS tile row c.

// Loads rows 64 quarter .. 64 quarter + 63 of a 256 x 256 bf16 block (row c =
// tile column c: the update's X_lo in the X^T layout, or the mirrored block of
// the symmetric A for bA + cA^2) into LDS slot `sp` in the tile layout: 32
// instructions of two rows, 8 per wavefront (I = wave + 4q). Row
// R = 64 quarter + 2I + (l >> 5) has R & 31 = (2 wave + (l >> 5)) | 8 (q & 3),
// so the chunk swizzle splits into a per-lane part and (q & 3) << 7, and the
// row offset into a per-lane part and a uniform one. `blk` points at the
// block's first element; rows are ld elements apart.
__device__ __forceinline__ void issue_blk_quarter(const bf16* blk, int64_t ld, char* sp, int quarter, int wave,
                                                  int lane, int q0 = 0, int q1 = 8)
{
    const int ldb2 = (int)ld * 2;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)blk, (short)0, kTile * ldb2, 0x00020000);
    const int vrow = (lane >> 5) * ldb2;
    const int vchunk = ((lane & 31) ^ (2 * wave + (lane >> 5))) << 4;
#pragma unroll
    for (int q = q0; q < q1; ++q) {
        const int I = wave + 4 * q;
        const int soff = (quarter * 64 + 2 * I) * ldb2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(sp + I * 1024), 16,
                                                 vrow + (vchunk ^ ((q & 3) << 7)), soff, 0, 0);
    }
}

// Epilogue of the bf16 update (X^T layout, LDS tile row = tile column c):
//   X_lo tile -> LDS (quarter 3 in its own slot, loaded before the K loop;
//   quarters 0..2 by the K loop's last steps), y = acc + a X_lo,
//   LDS <- bf16(y), X_lo <- bf16(y - bf16(y)) (global, in place, from
//   registers: lanes l and l + 32 trade register groups so that each holds 8
//   consecutive rows of its column, one 16-byte store)
//   LDS -> X_hi (next slot)
// Every element is read and rewritten by the same lane in the accumulator
// passes, so only the copies need barriers. On the last step bf16(y) goes to
// the caller's buffer instead.
template <bool LAST>
__device__ __forceinline__ void update_epilogue_bf16(const LargeMat& M, char* sl0, char* sl1,
                                                     char* sl2, char* sl3, bool lo_pre,
                                                     f32x16 (&acc)[4][4],
                                                     int64_t gbi, int64_t gbj, int nxt,
                                                     float ca, int wave, int lane)
{
    const int64_t ldt = M.ldt;
    const int fr = lane & 31, fg = lane >> 5;
    const int wr = wave >> 1, wc = wave & 1;
    bf16* lo_g = static_cast<bf16*>(M.xlo) + gbj * ldt + gbi;
    // this wavefront's rows in the copies; its columns 128 wc .. + 63 and
    // 128 wc + 64 .. + 127 in the accumulator passes
    char* ws = wave < 2 ? (wave == 0 ? sl0 : sl1) : (wave == 2 ? sl2 : sl3);
    char* cs0 = wc ? sl2 : sl0;
    char* cs1 = wc ? sl3 : sl1;

    // Quarters 0..2 of the X_lo tile were loaded by the K loop's last steps
    // (lo_pre) or are loaded here, once every wavefront is done with the
    // ring; quarter 3 (slot sl3, outside the ring) was loaded before the loop.
    NS_WAIT_ALL_BARRIER();
    if (!lo_pre) {
        const bf16* blk = static_cast<const bf16*>(M.xlo) + gbj * ldt + gbi;
        issue_blk_quarter(blk, ldt, sl0, 0, wave, lane);
        issue_blk_quarter(blk, ldt, sl1, 1, wave, lane);
        issue_blk_quarter(blk, ldt, sl2, 2, wave, lane);
        NS_WAIT_DMA_BARRIER();
    }

    // last step, rows <= cols: the caller's buffer is X itself, so the tile
    // is restaged with LDS row = tile row
    const bool by_rows = LAST && !M.trans;
    bf16* user = static_cast<bf16*>(M.user);
    uint2 hv[4][4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // The 16 reads of a block row go out together: the writes below could
        // alias them as far as the compiler knows, so reads interleaved with
        // writes would each wait out the LDS latency.
        bf16x4 los[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg)
                los[j][rg] = *reinterpret_cast<const bf16x4*>(
                    tile_at(j < 2 ? cs0 : cs1, wc * 128 + j * 32 + fr, wr * 128 + i * 32 + rg * 8 + fg * 4));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint2 l2[4];   // new X_lo of rows r0..r0+3, register groups 0..3
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int c = wc * 128 + j * 32 + fr;
                const int r0 = wr * 128 + i * 32 + rg * 8 + fg * 4;
                bf16x4* a = reinterpret_cast<bf16x4*>(tile_at(j < 2 ? cs0 : cs1, c, r0));
                const bf16x4 lo = los[j][rg];
                bf16x4 hi, lo2;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float y = fmaf(ca, (float)lo[e], acc[i][j][rg * 4 + e]);
                    hi[e] = (bf16)y;
                    lo2[e] = (bf16)(y - (float)hi[e]);
                }
                l2[rg] = __builtin_bit_cast(uint2, lo2);
                if (LAST && by_rows)
                    hv[i][j][rg] = __builtin_bit_cast(uint2, hi);
                else
                    *a = hi;
            }
            if (!LAST) {
                // Lane fr holds rows 8 rg + (0..3) of the block row, lane
                // fr + 32 rows 8 rg + (4..7). Swapping group 2h + 1 of the
                // lower lane with group 2h of the upper one leaves the lower
                // lane rows 16h + (0..7) and the upper one rows 16h + (8..15).
                // The new X_lo goes straight to this tile's own X_lo block
                // (its loads have landed).
                const int c = wc * 128 + j * 32 + fr;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const auto sx = __builtin_amdgcn_permlane32_swap(l2[2 * h].x, l2[2 * h + 1].x, false, false);
                    const auto sy = __builtin_amdgcn_permlane32_swap(l2[2 * h].y, l2[2 * h + 1].y, false, false);
                    const uint4 v = make_uint4(sx[0], sy[0], sx[1], sy[1]);
                    const int r = wr * 128 + i * 32 + 16 * h + 8 * fg;
                    st16(lo_g + (int64_t)c * ldt + r, v);
                }
            }
        }
    }
    NS_WAIT_LDS_BARRIER();
    if (LAST) {
        if (by_rows) {
            // (the barrier above: every wavefront has read its X_lo)
            write_tile_by_rows<4>(wr ? sl2 : sl0, wr ? sl3 : sl1, hv, wr, wc, fr, fg);
            NS_WAIT_LDS_BARRIER();
            tile_store_user(ws, user, M.rows_tab, M.cols, gbi, M.m, gbj, M.n, wave, lane);
        } else {
            // rows > cols: the caller's buffer is X^T, rows of M.cols
            tile_store_user(ws, user, M.rows_tab, M.cols, gbj, M.n, gbi, M.m, wave, lane);
        }
        return;
    }
    tile_store_pan(ws, static_cast<bf16*>(M.xt[nxt]), M.np, gbj, gbi / kPanelCols, wave, lane);
}

// Epilogue of the bf16 symmetric products A = X X^T (STAGE 0) and
// B = bA + cA^2 (STAGE 1) on tile (bi, bj), bi <= bj. Both blocks (bi, bj) and
// (bj, bi) of the output are written, as whole 512-byte rows from the LDS
// tile (slots s0..s3, 64 rows each):
//   1. LDS row = tile column c (the accumulator order, 8 bytes per lane and
//      register group; for STAGE 1 the same places hold the block of A read
//      by the K loop's last steps, A[c][r] = A[r][c]) -> block (bj, bi).
//   2. LDS row = tile row r -> block (bi, bj) (write_tile_by_rows).
// On a diagonal tile only the upper triangle is used: pass 1 writes each
// upper element at both (c, r) and (r, c), so the block is exactly symmetric,
// and pass 2 is not needed. The diagonal keeps its bf16 rounding residue
// (d_i = v_ii - bf16(v_ii)), and for B the first-order terms of A's residue:
// B_ij = (b + c (dA_i + dA_j)) A_ij + c (A A)_ij, plus b dA_i on the diagonal.
// NJ == 2: a half tile (never diagonal); its wavefront blocks j are
// 2 hsel + (0, 1), so all its columns of pass 1 lie in one slot per
// wavefront (2 wc + hsel) and block (bj, bi) is stored by the two
// wavefronts whose own slot that is; block (bi, bj) keeps only its columns.
template <int STAGE, int NJ>
__device__ __forceinline__ void sym_epilogue_bf16(const LargeMat& M, char* s0, char* s1, char* s2, char* s3,
                                                  f32x16 (&acc)[4][NJ], int64_t gbi, int64_t gbj, bool diag,
                                                  float cb, float cc, int wave, int lane, int hsel)
{
    constexpr bool kHalf = NJ == 2;
    const int jbase = kHalf ? 2 * hsel : 0;
    const int64_t ld = M.ldt;
    const int fr = lane & 31, fg = lane >> 5;
    const int wr = wave >> 1, wc = wave & 1;
    bf16* out = static_cast<bf16*>(STAGE == 0 ? M.a : M.b);
    float* dout = STAGE == 0 ? M.adiag : M.bdiag;
    char* ws = wave < 2 ? (wave == 0 ? s0 : s1) : (wave == 2 ? s2 : s3);
    // pass 1: tile column c lives in slot c >> 6 = 2 wc + (j >> 1)
    char* cs0 = kHalf ? (wc ? (hsel ? s3 : s2) : (hsel ? s1 : s0)) : (wc ? s2 : s0);
    char* cs1 = kHalf ? cs0 : (wc ? s3 : s1);
    // pass 2 (and the mirrored writes of a diagonal tile): tile row r lives
    // in slot r >> 6 = 2 wr + (i >> 1)
    char* rs0 = wr ? s2 : s0;
    char* rs1 = wr ? s3 : s1;

    // A's diagonal residues at this lane's rows and columns, all requested
    // at once (they cross the barrier below in flight)
    float dcol[NJ] = {};
    f32x4 drows[4][4];
    if constexpr (STAGE == 1) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            dcol[j] = gbl(M.adiag)[gbj + wc * 128 + (jbase + j) * 32 + fr];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg)
                drows[i][rg] =
                    *(NS_GLOBAL const f32x4*)gbl(M.adiag + gbi + wr * 128 + i * 32 + rg * 8 + fg * 4);
    }
    // Every wavefront is done with the ring; each has waited for its own
    // block loads (STAGE 1) at the end of the K loop.
    NS_WAIT_LDS_BARRIER();

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x4 (&drow)[4] = drows[i];
        // (A's 16 reads of a block row go out together, ahead of the writes
        // that the compiler cannot tell apart from them)
        bf16x4 as[NJ][4];
        if constexpr (STAGE == 1) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg)
                    as[j][rg] = *reinterpret_cast<const bf16x4*>(tile_at(
                        j < 2 ? cs0 : cs1, wc * 128 + (jbase + j) * 32 + fr, wr * 128 + i * 32 + rg * 8 + fg * 4));
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int c = wc * 128 + (jbase + j) * 32 + fr;
                const int r0 = wr * 128 + i * 32 + rg * 8 + fg * 4;
                char* cslot = j < 2 ? cs0 : cs1;
                bf16x4* loc = reinterpret_cast<bf16x4*>(tile_at(cslot, c, r0));
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = acc[i][j][rg * 4 + e];
                if constexpr (STAGE == 1) {
                    const bf16x4 a = as[j][rg];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float ce = fmaf(cc, drow[rg][e] + dcol[j], cb);
                        v[e] = ce * (float)a[e] + cc * v[e];
                    }
                }
                if (kHalf || !diag) {
                    bf16x4 h;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        h[e] = (bf16)v[e];
                    *loc = h;
                } else {
                    char* rslot = i < 2 ? rs0 : rs1;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = r0 + e;
                        if (r <= c) {
                            float x = v[e];
                            if (r == c) {
                                if constexpr (STAGE == 1)
                                    x = fmaf(cb, drow[rg][e], x);
                                gbl(dout)[gbi + c] = x - (float)(bf16)x;
                            }
                            const bf16 h = (bf16)x;
                            *reinterpret_cast<bf16*>(tile_at(cslot, c, r)) = h;
                            if (r < c)
                                *reinterpret_cast<bf16*>(tile_at(rslot, r, c)) = h;
                        }
                    }
                }
            }
    }
    NS_WAIT_LDS_BARRIER();
    // block (bj, bi): global row gbj + c, columns gbi ..
    if (!kHalf || (wave & 1) == hsel)
        tile_store(ws, out + gbj * ld + gbi, ld, wave, lane);
    if (!kHalf && diag)
        return;

    // this lane's bf16(v) back from the tile (rows r0..r0+3 of column c)
    uint2 hv[4][NJ][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg)
                hv[i][j][rg] = *reinterpret_cast<const uint2*>(tile_at(
                    j < 2 ? cs0 : cs1, wc * 128 + (jbase + j) * 32 + fr, wr * 128 + i * 32 + rg * 8 + fg * 4));
    // pass 2 overwrites the tile: every wavefront's copy and reads are done
    NS_WAIT_LDS_BARRIER();
    write_tile_by_rows<NJ>(rs0, rs1, hv, wr, wc, fr, fg, jbase);
    NS_WAIT_LDS_BARRIER();
    // block (bi, bj): global row gbi + r, columns gbj ..
    tile_store(ws, out + gbi * ld + gbj, ld, wave, lane, kHalf ? hsel : -1);
}

// One workgroup's tile t of a grouped GEMM stage, with the workgroup's LDS
// slots (sl0 .. sl3 the ring, lo3 the epilogue block's quarter 3).
// HALF (bf16 X X^T and bA + cA^2 only): the workgroup computes half of an
// off-diagonal tile's columns, those in 64-column pieces 2 hsel and 2 hsel + 2
// (wavefront column wc takes its 32-column blocks 2 hsel and 2 hsel + 1);
// hsel is bit 30 of the tile's matrix index. Every element gets the same MFMA
// sequence as in a whole tile, so the bits are the same; the half tiles of a
// launch's last, partial round run on twice as many compute units.
template <int DT, int STAGE, int LAST, int HALF>
__device__ __forceinline__ void gemm_tile(const LargeMat* __restrict__ mats, const Tile t, int cur, int last,
                                          float ca, float cb, float cc, char* sl0, char* sl1, char* sl2,
                                          char* sl3, char* lo3)
{
    using OpT = typename Elt<DT>::type;
    constexpr int NJ = HALF ? 2 : 4;   // 32-column blocks per wavefront
    const int hsel = HALF ? (int)((uint32_t)t.mat >> 30) : 0;
    const int jbase = 2 * hsel;
    const LargeMat& M = mats[HALF ? (t.mat & 0x3FFFFFFF) : t.mat];
    const char* P;
    const char* Q;
    // Operands read as k-rows (32 rows of 512 bytes per slot, see above)
    // instead of the tile's rows (256 rows of 64 bytes): on the bf16 path X^T
    // for X X^T, and A, B, which are symmetric, so that their k-rows restricted
    // to a block's columns are that block's rows. The update's X^T operand has
    // k contiguous in its rows. Long row pieces move faster: a 1 KB DMA covers
    // 2 rows of 512 bytes instead of 16 of 64.
    constexpr bool kTP = IsBf16<OpT>::value;
    constexpr bool kTQ = IsBf16<OpT>::value && STAGE != 2;
    // X_hi is stored as column panels (pan_at): X X^T reads its k-rows from
    // them into an LDS slot laid out as the 8 panels of the block (kPT: 32
    // rows of 64 bytes each, 2 KB per panel); the update reads its X^T
    // operand, k contiguous, as usual rows of 64 bytes, from one panel per
    // slot (kPQ).
    constexpr bool kPT = IsBf16<OpT>::value && STAGE == 0;
    constexpr bool kPQ = IsBf16<OpT>::value && STAGE == 2;
    int64_t K, pitch;
    if (STAGE == 0 && IsBf16<OpT>::value) {
        P = Q = static_cast<const char*>(M.xt[cur]);
        K = M.np;
        pitch = M.ldt;
    } else if (STAGE == 0) {
        P = Q = static_cast<const char*>(M.xb[cur]);
        K = M.np;
        pitch = M.ldx;
    } else if (STAGE == 1) {
        P = Q = static_cast<const char*>(M.a);
        K = M.mp;
        pitch = M.ldt;
    } else {
        P = static_cast<const char*>(M.b);
        Q = static_cast<const char*>(M.xt[cur]);
        K = M.mp;
        pitch = M.ldt;
    }
    const int ldb = (int)(pitch * (int64_t)sizeof(OpT));        // row pitch, bytes
    // slots: 64 bytes of K per row, or 32 rows of X^T (the same 32 bf16)
    const int ns = (int)(K * (int64_t)sizeof(OpT) / kSlotRowBytes);   // a multiple of 8 (K % 256 == 0)

    // wave is the same for all lanes of a wavefront; saying so keeps the
    // values derived from it (LDS DMA targets, buffer offsets) in SGPRs
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave >> 1, wc = wave & 1;

    // Buffer resources over the 256-row blocks of P and Q (out-of-range reads
    // return 0 without touching memory; only the K loop's loads past the last
    // slot use that, see issue()).
    // (k-row operands: the blocks are column ranges and the resource spans
    // all K rows.)
    // (panels: bytes per panel, np rows of 64 bytes; P and Q of X X^T are
    // the 8 panels of block bi, bj on, the update's Q rows 256 bj on of every
    // panel)
    // (all offsets into the panels fit 31 bits: the array is mp np 2 bytes)
    const int panb = M.np * kSlotRowBytes;
    const int pan_all = (M.mp / kPanelCols) * panb;
    const int64_t poff = kPT ? (int64_t)t.bi * 8 * panb
                       : kTP ? (int64_t)t.bi * kTile * 2 : (int64_t)t.bi * kTile * ldb;
    const int64_t qoff = kPT ? (int64_t)t.bj * 8 * panb
                       : kPQ ? (int64_t)t.bj * kTile * kSlotRowBytes
                       : kTQ ? (int64_t)t.bj * kTile * 2 : (int64_t)t.bj * kTile * ldb;
    const int range_p = kPT ? (int)(pan_all - poff) : kTP ? (int)(K * ldb - poff) : kTile * ldb;
    const int range_q = (kPT || kPQ) ? (int)(pan_all - qoff) : kTQ ? (int)(K * ldb - qoff) : kTile * ldb;
    const __amdgpu_buffer_rsrc_t rp =
        __builtin_amdgcn_make_buffer_rsrc((void*)(P + poff), (short)0, range_p, 0x00020000);
    const __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Q + qoff), (short)0, range_q, 0x00020000);

    // DMA mapping: wavefront w fills instructions I = w + 4 q (q = 0..3) of a
    // slot operand, 1 KB = rows 16I..16I+15 each. Lane l writes stored chunk
    // l & 3 of row 16I + (l >> 2), i.e. logical chunk (l & 3) ^ g(row); the
    // q offset (64 rows) leaves g unchanged.
    // k-rows: instruction I fills LDS rows 2I, 2I+1 (k); lane l writes
    // stored chunk l & 31 of row 2I + (l >> 5); the q offset (8 rows) leaves
    // the swizzle unchanged.
    // panel k-rows: instruction I fills panel I >> 1, rows 16 (I & 1) + 0..15
    // of the slot, lane l row 16 (I & 1) + (l >> 2), chunk l & 3: 1 KB of one
    // panel in global memory and in LDS (no swizzle: a transposing read of 16
    // lanes covers 4 consecutive 64-byte rows, 64 distinct banks per 32
    // lanes). The q offset moves two panels.
    const int row_n = 16 * wave + (lane >> 2), row_t = 2 * wave + (lane >> 5);
    const int ldn = kPQ ? kSlotRowBytes : ldb;
    const int voff_n = row_n * ldn + (((lane & 3) ^ lds_swz(row_n)) << 4);
    const int voff_t = row_t * ldb + (((lane & 31) ^ tr_swz(row_t)) << 4);
    const int voff_pt = (wave >> 1) * panb + (16 * (wave & 1) + (lane >> 2)) * kSlotRowBytes + ((lane & 3) << 4);
    const int voff_p = kPT ? voff_pt : kTP ? voff_t : voff_n;
    const int voff_q = kPT ? voff_pt : kTQ ? voff_t : voff_n;

    // In the bf16 update, slots sb .. sb + 7 are this tile's own 256 rows.
    // Slot positions past the end (s >= ns) are loads that nobody reads but
    // that keep the per-slot load count (and so the wait counts) uniform:
    // their scalar offset is past the end of both resources, so they return
    // zeros without memory traffic. (voffset < 2^29 and ranges < 2^31, so the
    // 32-bit offset sum cannot wrap back into range.)
    constexpr bool kIdent = STAGE == 2 && IsBf16<OpT>::value;
    // epilogue block preloaded into LDS: X_lo (bf16 update), A (bf16 bA + cA^2)
    constexpr bool kPre = kIdent || (STAGE == 1 && IsBf16<OpT>::value);
    const int sb = kIdent ? t.bi * 8 : 0;
    const int soff_end = range_p > range_q ? range_p : range_q;
    // X X^T half tiles read only the 4 Q panels their columns lie in
    // (2 hsel, 2 hsel + 1, 2 hsel + 4, 2 hsel + 5: instructions q = hsel and
    // q = hsel + 2), 6 DMAs per wavefront and slot instead of 8 (3 in each
    // half of a step), which the wait counts below follow.
    constexpr bool kHalfQ = HALF && kPT;
    auto issue = [&](char* sp, int s, int q0 = 0, int q1 = 4) __attribute__((always_inline)) {
#pragma unroll
        for (int q = q0; q < q1; ++q) {
            const int soff_t = s >= ns ? soff_end : (s * 32 + 8 * q) * ldb;
            const int soff_n = s >= ns ? soff_end : s * kSlotRowBytes + q * 64 * ldb;
            const int soff_pt = s >= ns ? soff_end : 2 * q * panb + s * 32 * kSlotRowBytes;
            const int soff_pq = s >= ns ? soff_end : s * panb + q * 64 * kSlotRowBytes;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rp, (lds_ptr_t)(sp + (wave + 4 * q) * 1024), 16, voff_p, kPT ? soff_pt : kTP ? soff_t : soff_n,
                0, 0);
            if (!kHalfQ || (q & 1) == hsel)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rq, (lds_ptr_t)(sp + kSlotOpBytes + (wave + 4 * q) * 1024), 16, voff_q,
                    kPT ? soff_pt : kPQ ? soff_pq : kTQ ? soff_t : soff_n, 0, 0);
        }
    };

    const int fr = lane & 31, fg = lane >> 5;
    const int64_t gbi = (int64_t)t.bi * kTile, gbj = (int64_t)t.bj * kTile;
    f32x16 acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.f;

    // Fragment offsets (k-step 0) of this lane's rows inside a stage; k-step
    // ks is logical chunk 2 ks + fg, which XORs the stored chunk with 2 ks.
    // k-rows: lane l (group g = l >> 4, x = l & 15) reads row
    // ks*16 + 8 (g >> 1) + 4 e + (x >> 2), columns base + 16 (g & 1) + 4 (x & 3);
    // k-step ks and half e only add whole rows (ks * 8192 + e * 2048 bytes).
    // Both layouts give lane l the k values 16 ks + 8 (l >> 5) + 0..7 of its
    // row or column, so they can be mixed.
    // Panel k-rows: the same lane -> (row, column) map; column cl sits in
    // panel cl >> 5, rows of 64 bytes, so k-step ks adds 1 KB and half e 256 B.
    auto off_t = [&](int base) {
        const int g = lane >> 4, x = lane & 15;
        const int kr = 8 * (g >> 1) + (x >> 2);
        const int cl = base + 16 * (g & 1) + 4 * (x & 3);
        if (kPT)
            return (cl >> 5) * (32 * kSlotRowBytes) + kr * kSlotRowBytes + (((cl >> 3) & 3) << 4) + (cl & 7) * 2;
        return kr * kTrRowBytes + (((cl >> 3) ^ tr_swz(kr)) << 4) + (cl & 7) * 2;
    };
    int aoff[4], boff[NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        aoff[i] = kTP ? off_t(wr * 128 + i * 32) : lds_off(wr * 128 + i * 32 + fr, fg);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int cb0 = wc * 128 + (jbase + j) * 32;
        boff[j] = kSlotOpBytes + (kTQ ? off_t(cb0) : lds_off(cb0 + fr, fg));
    }
    constexpr int kTrStep = kPT ? 16 * kSlotRowBytes : 16 * kTrRowBytes;   // 16 k-rows
    constexpr int kTrHalf = kPT ? 4 * kSlotRowBytes : 4 * kTrRowBytes;     // 4 k-rows
    auto read_frag = [&](const char* sp, int off, int ks, bool tr) __attribute__((always_inline)) {
        if (tr) {
            const uint2 v0 = ds_read_tr(sp + off + ks * kTrStep);
            const uint2 v1 = ds_read_tr(sp + off + ks * kTrStep + kTrHalf);
            return make_uint4(v0.x, v0.y, v1.x, v1.y);
        }
        return *reinterpret_cast<const uint4*>(sp + (off ^ (ks << 5)));
    };
    auto read_frags = [&](const char* sp, int ks, uint4 (&af)[4], uint4 (&bfr)[NJ]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            af[i] = read_frag(sp, aoff[i], ks, kTP);
            if (i < NJ)
                bfr[i] = read_frag(sp, boff[i], ks, kTQ);
        }
    };
    auto mfma_block = [&](const uint4 (&af)[4], const uint4 (&bfr)[NJ]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                Mfma<OpT>::mac(acc[i][j], af[i], bfr[j]);
    };
    auto interleave = []() __attribute__((always_inline)) {
        // Per k-step: the 4 NJ MFMAs with the LDS reads of the next k-step
        // (8 transposed 8-byte reads or 4 16-byte reads per operand and 4
        // blocks) and half of the refill's DMAs (4) spread between them.
        // Issued in one burst, the DMAs stall the wavefront at issue while
        // the memory pipeline is full, and that pipeline then runs dry during
        // the MFMAs.
        constexpr int nmf = 4 * NJ;
        constexpr int nreads = (kTP ? 8 : 4) + (kTQ ? 2 : 1) * NJ;
#pragma unroll
        for (int q = 0; q < nmf; ++q) {
            if (q % (nmf / 4) == 0)
                __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
            // whole tiles: one read per MFMA while reads last; half tiles
            // (12 reads, 8 MFMAs): two per MFMA first, then one
            const int nr = NJ == 4 ? (q < nreads ? 1 : 0) : (q < nreads - nmf ? 2 : 1);
            if (nr >= 1)
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (nr >= 2)
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
    };

    // Pipeline over the ring. Step s multiplies slot s (k-steps 0 and 1) while
    // slots s + 1 .. s + 3 are in flight: it refills the ring position of slot
    // s - 1 (freed by the barrier that ended step s - 1) with slot s + 3, four
    // of the eight DMAs per wavefront between each k-step's MFMAs. It reads
    // k-step 1's fragments while k-step 0's MFMAs run, then waits until its
    // own DMAs of slot s + 1 have landed (younger: the 8 of slot s + 2 and the
    // first 4 of slot s + 3) and passes the barrier (slot s + 1 complete,
    // nobody reads slot s any more), reads k-step 0 of slot s + 1 and issues
    // k-step 1's MFMAs to cover that read.
    //
    // bf16 X <- aX + BX: the a X_hi part (X_hi = bf16(X), the Q operand
    // itself) is added by the MFMAs too. Slots sb .. sb + 7 (sb = 8 bi) are
    // the tile's own 256 rows; slot sb + P covers rows 32 P .. 32 P + 31, block
    // P & 3 of wavefront row P >> 2. There an identity A fragment scaled by
    // s_hi = bf16(s) and one scaled by s_lo = bf16(s - s_hi) multiply the Q
    // fragments already in registers; the other wavefront row adds zeros, so
    // the code stays straight. Those products are exact in fp32; a X_lo is
    // added in the epilogue.
    // Per-row scale of the identity: a + (B_ii - bf16(B_ii)), which also
    // restores the part of B's diagonal that its bf16 operand dropped (the
    // diagonal dominates B when the singular values are clustered).
    float rowscale[4];
    if constexpr (kIdent) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            rowscale[ii] = ca + gbl(M.bdiag)[gbi + wr * 128 + ii * 32 + fr];
    }
    // peel slot P, k-step ks of the slot
    auto ident = [&](int P, int ks, const uint4 (&bfr)[NJ]) {
        const int ii = P & 3;
        // A fragment: lane l holds row l & 31, k = 8 (l >> 5) + e of the
        // 32 x 16 block; the identity sits at e = (l & 31) - 16 ks - 8 (l >> 5).
        const int e = fr - 16 * ks - 8 * fg;
        const bool mine = (P >> 2) == wr;
        const bf16 ahi = (bf16)rowscale[ii];
        const bf16 alo = (bf16)(rowscale[ii] - (float)ahi);
        const uint32_t hb = mine ? __builtin_bit_cast(uint16_t, ahi) : 0u;
        const uint32_t lb = mine ? __builtin_bit_cast(uint16_t, alo) : 0u;
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const bool on = (e >> 1) == w && e >= 0 && e < 8;
            const int sh = (e & 1) * 16;
            wh[w] = on ? hb << sh : 0u;
            wl[w] = on ? lb << sh : 0u;
        }
        const uint4 fh = make_uint4(wh[0], wh[1], wh[2], wh[3]);
        const uint4 fl = make_uint4(wl[0], wl[1], wl[2], wl[3]);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            Mfma<OpT>::mac(acc[ii][j], fh, bfr[j]);
            Mfma<OpT>::mac(acc[ii][j], fl, bfr[j]);
        }
    };

    // The bf16 update's epilogue reads the tile's X_lo through LDS, and the
    // bf16 bA + cA^2 epilogue the mirrored block of A (row c = tile column c,
    // 64 rows per slot). The last three steps have no operand slot left to
    // load; they load quarters 0..2 of that block into the ring positions
    // they free instead (8 loads per wavefront, like a slot). Quarter 3 goes
    // to a fifth slot before the K loop.
    const bf16* pre_blk = nullptr;
    if constexpr (kPre)
        pre_blk = static_cast<const bf16*>(kIdent ? M.xlo : M.a) + gbj * M.ldt + gbi;
    auto issue_lo = [&](char* sp, int quarter, int q0, int q1) __attribute__((always_inline)) {
        issue_blk_quarter(pre_blk, M.ldt, sp, quarter, wave, lane, q0, q1);
    };

    uint4 fa[4], fb[NJ], ga[4], gb[NJ];
    // H >= 0: slot sb + H of the bf16 update (adds a X_hi);
    // L >= 0: instead of a slot, load quarter L of the update's X_lo tile
    auto step = [&](const char* cur, char* refill, const char* next, int s, auto peel, auto lq) __attribute__((always_inline)) {
        constexpr int H = decltype(peel)::value;
        constexpr int L = decltype(lq)::value;
        if constexpr (L >= 0)
            issue_lo(refill, L, 0, 4);
        else
            issue(refill, s + 3, 0, 2);
        read_frags(cur, 1, ga, gb);
        mfma_block(fa, fb);
        interleave();
        if constexpr (H >= 0) ident(H, 0, fb);
        // slot s + 1 complete: younger are slot s + 2 and half of s + 3
        if constexpr (kHalfQ)
            asm volatile("s_waitcnt vmcnt(9)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(12)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if constexpr (L >= 0)
            issue_lo(refill, L, 4, 8);
        else
            issue(refill, s + 3, 2, 4);
        read_frags(next, 0, fa, fb);
        mfma_block(ga, gb);
        interleave();
        if constexpr (H >= 0) ident(H, 1, gb);
    };
    // four steps from ring position 0 (slot s, s % 4 == 0)
    auto ring = [&](int s, auto p0, auto p1, auto p2, auto p3) __attribute__((always_inline)) {
        step(sl0, sl3, sl1, s, p0, Peel<-1>{});
        step(sl1, sl0, sl2, s + 1, p1, Peel<-1>{});
        step(sl2, sl1, sl3, s + 2, p2, Peel<-1>{});
        step(sl3, sl2, sl0, s + 3, p3, Peel<-1>{});
    };
    // the last four steps (s = ns - 4); the refills of slots ns .. ns + 2
    // are the epilogue block's quarters where there is one, dummy reloads
    // otherwise
    auto ring_last = [&](int s, auto p0, auto p1, auto p2, auto p3) __attribute__((always_inline)) {
        if constexpr (kPre) {
            step(sl0, sl3, sl1, s, p0, Peel<-1>{});
            step(sl1, sl0, sl2, s + 1, p1, Peel<0>{});
            step(sl2, sl1, sl3, s + 2, p2, Peel<1>{});
            step(sl3, sl2, sl0, s + 3, p3, Peel<2>{});
        } else {
            ring(s, p0, p1, p2, p3);
        }
    };

    // The epilogue block's quarter 3 goes out right after slot 0: the first
    // wait is for slot 0 alone (16 younger loads without it, 24 with it), and
    // from step 0 on it is older than every slot waited for, so the wait
    // counts in the loop, which bound the number of younger loads, still hold.
    issue(sl0, 0);
    if constexpr (kPre)
        issue_blk_quarter(pre_blk, M.ldt, lo3, 3, wave, lane);
    issue(sl1, 1);
    issue(sl2, 2);
    if constexpr (kPre)
        asm volatile("s_waitcnt vmcnt(24)\n\ts_barrier" ::: "memory");
    else if constexpr (kHalfQ)
        asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
    read_frags(sl0, 0, fa, fb);
    // Every tile visits the slots in the same order, so tiles that share an
    // operand block read the same k-slice at about the same time (L2 reuse);
    // the bf16 update's identity slots are peeled in place.
    int s = 0;
    bool lo_pre = false;   // epilogue block quarters 0..2 already in slots 0..2
    if constexpr (kIdent) {
        for (; s < sb; s += 4)
            ring(s, Peel<-1>{}, Peel<-1>{}, Peel<-1>{}, Peel<-1>{});
        ring(s, Peel<0>{}, Peel<1>{}, Peel<2>{}, Peel<3>{});
        ring(s + 4, Peel<4>{}, Peel<5>{}, Peel<6>{}, Peel<7>{});
        s += 8;
        for (; s + 4 < ns; s += 4)
            ring(s, Peel<-1>{}, Peel<-1>{}, Peel<-1>{}, Peel<-1>{});
        // (when the identity slots are the last ones, the epilogue loads all
        // four quarters itself)
        if (s < ns) {
            ring_last(s, Peel<-1>{}, Peel<-1>{}, Peel<-1>{}, Peel<-1>{});
            lo_pre = true;
        }
    } else if constexpr (kPre) {
        // (ns >= 8 and a multiple of 4)
        for (; s + 4 < ns; s += 4)
            ring(s, Peel<-1>{}, Peel<-1>{}, Peel<-1>{}, Peel<-1>{});
        ring_last(s, Peel<-1>{}, Peel<-1>{}, Peel<-1>{}, Peel<-1>{});
        lo_pre = true;
    } else {
        for (; s < ns; s += 4)
            ring(s, Peel<-1>{}, Peel<-1>{}, Peel<-1>{}, Peel<-1>{});
    }
    // (the builtin, not inline asm: the compiler's own wait insertion then
    // knows that no LDS DMA is in flight and adds no waits before the
    // epilogues' LDS writes; 0x0F70 = vmcnt(0), other counters untouched)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("" ::: "memory");

    // Epilogues. Lane l, block (i, j), register group rg holds rows
    // lr0..lr0+3 of column lc (tile-local).
    if constexpr (STAGE == 0 && IsBf16<OpT>::value) {
        sym_epilogue_bf16<0, NJ>(M, sl0, sl1, sl2, sl3, acc, gbi, gbj, !HALF && t.bi == t.bj, cb, cc, wave, lane,
                                 hsel);
        return;
    } else if constexpr (STAGE == 1 && IsBf16<OpT>::value) {
        sym_epilogue_bf16<1, NJ>(M, sl0, sl1, sl2, lo3, acc, gbi, gbj, !HALF && t.bi == t.bj, cb, cc, wave, lane,
                                 hsel);
        return;
    }
    if constexpr (!HALF) {
    // fp32 path: the epilogues store straight from the accumulators (a
    // 256 x 256 fp32 tile does not fit the LDS), and there are no residues.
    if (STAGE == 0 || STAGE == 1) {
        const int64_t ld = M.ldt;
        OpT* out = static_cast<OpT*>(STAGE == 0 ? M.a : M.b);
        const OpT* ain = static_cast<const OpT*>(M.a);
        const bool diag = t.bi == t.bj;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // bA + cA^2 needs A at the same places; A is exactly symmetric, so
            // rows r0..r0+3 of column c are A[c][r0..r0+3], one vector load.
            // All 16 loads of a block row are issued before any is used.
            f32x4 a4[4][4];
            if (STAGE == 1) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const int64_t r0 = gbi + wr * 128 + i * 32 + rg * 8 + fg * 4;
                        const int64_t c = gbj + wc * 128 + j * 32 + fr;
                        a4[j][rg] = load4(ain + c * ld + r0);
                    }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int lr0 = wr * 128 + i * 32 + rg * 8 + fg * 4;
                    const int lc = wc * 128 + j * 32 + fr;
                    const int64_t r0 = gbi + lr0, c = gbj + lc;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = acc[i][j][rg * 4 + e];
                    if (STAGE == 1) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            v[e] = cb * a4[j][rg][e] + cc * v[e];
                    }
                    if (!diag) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            gbl(out)[(r0 + e) * ld + c] = from_f32<OpT>(v[e]);
                        store4(out + c * ld + r0, v[0], v[1], v[2], v[3]);
                    } else {
                        // Diagonal tile: take the upper triangle and mirror it,
                        // so the stored matrix is exactly symmetric.
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (lr0 + e < lc) {
                                gbl(out)[(r0 + e) * ld + c] = from_f32<OpT>(v[e]);
                                gbl(out)[c * ld + r0 + e] = from_f32<OpT>(v[e]);
                            }
                        }
                    }
                }
        }
        if (diag && wr == wc) {
            // The diagonal: in block (i, i), lane (fr, fg) holds element
            // (fr, fr) when fg == (fr >> 2) & 1, in register 4 (fr >> 3) + (fr & 3).
            const int sel = 4 * (fr >> 3) + (fr & 3);
            const bool has = fg == ((fr >> 2) & 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    v = r == sel ? acc[i][i][r] : v;
                const int64_t rc = gbi + wr * 128 + i * 32 + fr;
                if (has) {
                    if (STAGE == 1)
                        v = cb * to_f32(gbl(ain)[rc * ld + rc]) + cc * v;
                    gbl(out)[rc * ld + rc] = from_f32<OpT>(v);
                }
            }
        }
    } else {
        const int nxt = cur ^ 1;
        const int64_t ldx = M.ldx, ldt = M.ldt;
        if constexpr (kIdent) {
            update_epilogue_bf16<LAST != 0>(M, sl0, sl1, sl2, lo3, lo_pre, acc, gbi, gbj, nxt, ca, wave, lane);
            return;
        }
        // a X, per lane four rows of a column, from X^T (this launch's
        // operand copy, read-only here)
        const OpT* src = static_cast<const OpT*>(M.xt[cur]);
        OpT* xb = static_cast<OpT*>(M.xb[nxt]);
        OpT* xt = static_cast<OpT*>(M.xt[nxt]);
        OpT* user = static_cast<OpT*>(M.user);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // All 16 loads of a block row first, then the sums and stores.
            f32x4 xv[4][4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int64_t r0 = gbi + wr * 128 + i * 32 + rg * 8 + fg * 4;
                    const int64_t c = gbj + wc * 128 + j * 32 + fr;
                    xv[j][rg] = load4(src + c * ldt + r0);
                }
            auto group = [&](int64_t r0, int64_t c, const f32x4& x, float v0, float v1, float v2,
                             float v3) __attribute__((always_inline)) {
                float y[4] = {fmaf(ca, x[0], v0), fmaf(ca, x[1], v1), fmaf(ca, x[2], v2),
                              fmaf(ca, x[3], v3)};
                if (!last) {
                    store4(xt + c * ldt + r0, y[0], y[1], y[2], y[3]);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        gbl(xb)[(r0 + e) * ldx + c] = from_f32<OpT>(y[e]);
                } else if (c < M.n) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (r0 + e < M.m) {
                            OpT* row = grow<OpT>(user, M.rows_tab, M.cols, M.trans ? c : r0 + e);
                            gbl(row)[M.trans ? r0 + e : c] = from_f32<OpT>(y[e]);
                        }
                    }
                }
            };
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x16 a = acc[i][j];
                const int64_t r0 = gbi + wr * 128 + i * 32 + fg * 4;
                const int64_t c = gbj + wc * 128 + j * 32 + fr;
                group(r0, c, xv[j][0], a[0], a[1], a[2], a[3]);
                group(r0 + 8, c, xv[j][1], a[4], a[5], a[6], a[7]);
                group(r0 + 16, c, xv[j][2], a[8], a[9], a[10], a[11]);
                group(r0 + 24, c, xv[j][3], a[12], a[13], a[14], a[15]);
            }
        }
    }
    }
}

// A grouped GEMM stage over tiles[0 .. ntiles): one workgroup per tile.
// SPLIT (bf16 X X^T and bA + cA^2): workgroups [0, nwhole) run whole tiles
// and the rest the half tiles of the stage's split last round; being in the
// same grid, the half tiles go to the compute units that finish their whole
// tiles first.
template <int DT, int STAGE, int LAST, int SPLIT>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(const LargeMat* __restrict__ mats,
                                                      const Tile* __restrict__ tiles, int cur, int last,
                                                      float ca, float cb, float cc, int nwhole)
{
    // Four LDS slots (P then Q, 16 KB each), one object each: with the k loop
    // unrolled over the ring, every LDS read and every DMA names its slot
    // statically, so the compiler can see that a refill does not touch the
    // slots being read and does not wait for them.
    __shared__ __attribute__((aligned(1024))) char sl0[2 * kSlotOpBytes];
    __shared__ __attribute__((aligned(1024))) char sl1[2 * kSlotOpBytes];
    __shared__ __attribute__((aligned(1024))) char sl2[2 * kSlotOpBytes];
    __shared__ __attribute__((aligned(1024))) char sl3[2 * kSlotOpBytes];
    // bf16 update and bA + cA^2 only: quarter 3 of the epilogue's block,
    // loaded before the K loop so that the epilogue need not wait for it
    // (160 KB of LDS in all)
    __shared__ __attribute__((aligned(1024))) char lo3[2 * kSlotOpBytes];

    const Tile t = tiles[blockIdx.x];
    if constexpr (SPLIT) {
        if ((int)blockIdx.x >= nwhole) {
            gemm_tile<DT, STAGE, LAST, 1>(mats, t, cur, last, ca, cb, cc, sl0, sl1, sl2, sl3, lo3);
            return;
        }
    }
    gemm_tile<DT, STAGE, LAST, 0>(mats, t, cur, last, ca, cb, cc, sl0, sl1, sl2, sl3, lo3);
}

template <typename OpT, int STAGE>
hipError_t launch_gemm_t(const LargeMat* mats, const Tile* tiles, int ntiles, int nwhole, int cur, int last,
                         float a, float b, float c, hipStream_t stream)
{
    // The bf16 update's last step (it writes the caller's buffer) is its own
    // instantiation, so the other steps' epilogue carries no code for it; so
    // is a bf16 symmetric stage with half tiles.
    constexpr int DT = IsBf16<OpT>::value ? 0 : 1;
    if (nwhole < 0 || nwhole > ntiles)
        return hipErrorInvalidValue;
    if constexpr (STAGE == 2 && DT == 0) {
        if (last) {
            hipLaunchKernelGGL((k_gemm<DT, STAGE, 1, 0>), dim3(ntiles), dim3(kThreads), 0, stream, mats,
                               tiles, cur, last, a, b, c, ntiles);
            return hipGetLastError();
        }
    }
    if constexpr (STAGE < 2 && DT == 0) {
        if (nwhole < ntiles) {
            hipLaunchKernelGGL((k_gemm<DT, STAGE, 0, 1>), dim3(ntiles), dim3(kThreads), 0, stream, mats,
                               tiles, cur, last, a, b, c, nwhole);
            return hipGetLastError();
        }
    }
    if (nwhole < ntiles)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_gemm<DT, STAGE, 0, 0>), dim3(ntiles), dim3(kThreads), 0, stream, mats, tiles,
                       cur, last, a, b, c, ntiles);
    return hipGetLastError();
}
}  // namespace

template <int DT, int MR>
hipError_t launch_small_t(const SmallMat* mats, int count, const int32_t* slice_prefix, int nslices, int phase,
                          int steps, const SmallCoeffs& co, hipStream_t stream)
{
    hipLaunchKernelGGL((k_small<DT, MR>), dim3(nslices), dim3(kSmallThreads), 0, stream, mats, count, slice_prefix,
                       phase, steps, co);
    return hipGetLastError();
}

hipError_t launch_small(int dtype, int mr, const SmallMat* mats, int count, const int32_t* slice_prefix,
                        int nslices, int phase, int steps, const SmallCoeffs& co, hipStream_t stream)
{
    switch (mr) {
    case 8:
        return dtype == 0 ? launch_small_t<0, 8>(mats, count, slice_prefix, nslices, phase, steps, co, stream)
                          : launch_small_t<1, 8>(mats, count, slice_prefix, nslices, phase, steps, co, stream);
    case 16:
        return dtype == 0 ? launch_small_t<0, 16>(mats, count, slice_prefix, nslices, phase, steps, co, stream)
                          : launch_small_t<1, 16>(mats, count, slice_prefix, nslices, phase, steps, co, stream);
    case 24:
        return dtype == 0 ? launch_small_t<0, 24>(mats, count, slice_prefix, nslices, phase, steps, co, stream)
                          : launch_small_t<1, 24>(mats, count, slice_prefix, nslices, phase, steps, co, stream);
    case 32:
        return dtype == 0 ? launch_small_t<0, 32>(mats, count, slice_prefix, nslices, phase, steps, co, stream)
                          : launch_small_t<1, 32>(mats, count, slice_prefix, nslices, phase, steps, co, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_norm_partial(int dtype, const LargeMat* mats, int nmats, const int32_t* part_prefix,
                               int total_parts, float* partials, hipStream_t stream)
{
    if (dtype == 0)
        hipLaunchKernelGGL(k_norm_partial<0>, dim3(total_parts), dim3(kThreads), 0, stream, mats,
                           nmats, part_prefix, partials, total_parts);
    else
        hipLaunchKernelGGL(k_norm_partial<1>, dim3(total_parts), dim3(kThreads), 0, stream, mats,
                           nmats, part_prefix, partials, total_parts);
    return hipGetLastError();
}

hipError_t launch_norm_final(int nmats, const int32_t* part_prefix, const float* partials, int total_parts,
                             float* inv, hipStream_t stream)
{
    hipLaunchKernelGGL(k_norm_final, dim3(nmats), dim3(kThreads), 0, stream, part_prefix, partials, total_parts,
                       inv);
    return hipGetLastError();
}

hipError_t launch_prep(int dtype, const LargeMat* mats, int nmats, const int32_t* prep_prefix,
                       int total_prep, const float* inv, hipStream_t stream)
{
    if (dtype == 0)
        hipLaunchKernelGGL(k_prep<0>, dim3(total_prep), dim3(kThreads), 0, stream, mats, nmats,
                           prep_prefix, inv);
    else
        hipLaunchKernelGGL(k_prep<1>, dim3(total_prep), dim3(kThreads), 0, stream, mats, nmats,
                           prep_prefix, inv);
    return hipGetLastError();
}

hipError_t launch_scale_out(int dtype, const LargeMat* mats, int nmats, const int32_t* part_prefix,
                            int total_parts, const float* inv, hipStream_t stream)
{
    if (dtype == 0)
        hipLaunchKernelGGL(k_scale_out<0>, dim3(total_parts), dim3(kThreads), 0, stream, mats,
                           nmats, part_prefix, inv);
    else
        hipLaunchKernelGGL(k_scale_out<1>, dim3(total_parts), dim3(kThreads), 0, stream, mats,
                           nmats, part_prefix, inv);
    return hipGetLastError();
}

hipError_t launch_gemm(int dtype, int stage, const LargeMat* mats, const Tile* tiles, int ntiles, int nwhole,
                       int cur, int last, float a, float b, float c, hipStream_t stream)
{
    if (dtype == 0) {
        if (stage == 0) return launch_gemm_t<bf16, 0>(mats, tiles, ntiles, nwhole, cur, last, a, b, c, stream);
        if (stage == 1) return launch_gemm_t<bf16, 1>(mats, tiles, ntiles, nwhole, cur, last, a, b, c, stream);
        return launch_gemm_t<bf16, 2>(mats, tiles, ntiles, nwhole, cur, last, a, b, c, stream);
    }
    if (stage == 0) return launch_gemm_t<float, 0>(mats, tiles, ntiles, nwhole, cur, last, a, b, c, stream);
    if (stage == 1) return launch_gemm_t<float, 1>(mats, tiles, ntiles, nwhole, cur, last, a, b, c, stream);
    return launch_gemm_t<float, 2>(mats, tiles, ntiles, nwhole, cur, last, a, b, c, stream);
}

}  // namespace ns
