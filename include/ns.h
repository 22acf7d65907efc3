/*
 * ns.h -- C ABI of libns.so: batched Newton-Schulz orthogonalization on
 * MI355X (gfx950).
 *
 * The operation. Each matrix G (rows x cols, row-major) of a batch is replaced
 * in place by its Newton-Schulz orthogonalization:
 *
 *     X = G / (||G||_F + 1e-7)
 *     if rows > cols: X = X^T                    (X is m x n, m <= n)
 *     repeat `steps` times:  A = X X^T;  B = b A + c A^2;  X = a X + B X
 *     if transposed: X = X^T;  G <- X rounded to the buffer's dtype
 *
 * The pages this library is built from name this operation as the compute
 * that Muon-family optimizers run on every assembled 2-D update matrix
 * (microsoft/dion PR #74, "Fix megabatch_orthogonalize_async hang on empty
 * FSDP2 shards", Fix section, which also states that zero rows stay zero) and
 * rank its cost as max(M,N)*min(M,N)^2 (NVIDIA/Megatron-LM PR #6379, "Balance
 * LayerWise optimizer shards by Newton-Schulz cost, not parameter size",
 * Changes item 1). They give neither the iteration's coefficients nor its
 * normalization; the specification this library implements fixes them: the
 * Frobenius normalization with eps = 1e-7 added to the norm, the orientation
 * rows <= cols, 5 steps and (a, b, c) = (3.4445, -4.7750, 2.0315), which
 * NS_QUINTIC_* below hold.
 *
 * Precision (what the result is computed with, not a promise of bits):
 *  - bf16 matrices with min(rows, cols) > 32: products on bf16 MFMA with fp32
 *    accumulation. X is carried between steps as two bf16 arrays,
 *    X_hi = bf16(X) and X_lo = bf16(X - X_hi), about 17 significant bits; A
 *    and B are stored as bf16 operands (the same bf16 A in b A and in A^2),
 *    with the rounding residues of their diagonals kept in fp32 and added
 *    back (first-order terms in B, the diagonal of B in the update). The
 *    result is rounded to bf16 (round-to-nearest-even). Relative Frobenius
 *    error against an fp64 evaluation of the same iteration: 2.6e-3 on the
 *    dense low-rank 8192 x 6144 batch, 6e-3 to 1e-2 on Gaussian inputs, up
 *    to 1.4e-2 on small nearly square ones; within 2e-2 at 5 steps.
 *  - matrices of either dtype with min(rows, cols) <= 32 (the small-matrix
 *    path, see NS_SMALL_M): the iteration evaluated in fp64 through the m x m
 *    Gram matrix, which reaches the same result up to rounding: with
 *    X_k = Q_k X_0, A_0 = X_0 X_0^T over the n columns, then per step
 *    B'_k = a I + b A_k + c A_k^2, Q_(k+1) = B'_k Q_k and
 *    A_(k+1) = B'_k A_k B'_k on m x m matrices, and finally Q X_0, rounded to
 *    the buffer's dtype.
 *  - fp32 matrices with min(rows, cols) > 32: fp32 arithmetic throughout
 *    (fp32 MFMA), within 1e-4 of the fp64 evaluation for inputs whose
 *    singular values are not exactly zero. On an exactly rank-deficient
 *    input the rounding noise in its null space grows by about a per step,
 *    as in any fp32 evaluation (e.g. 6e-5 after 5 steps, 2e-3 after 8, on a
 *    rank-4 856 x 535 matrix, within 2x of a plain fp32 evaluation).
 *  - Errors grow with the step count: the bounds above are for the 5 steps
 *    of the specification (bf16 Gaussian inputs reached 1.3e-2 to 1.9e-2
 *    after 8 steps in a seeded sweep).
 *  - The tiled path's norm sums squares in fp32 with per-piece power-of-two
 *    scaling, the small path's in fp64, so every finite input normalizes
 *    (entries up to FLT_MAX); an Inf or NaN entry propagates (see
 *    ns_orthogonalize_batched).
 * Zero rows and columns of G come back as exact +0.0, and a matrix gives the
 * same bits alone, in any batch, at any position and with trailing zero rows
 * appended.
 *
 * Threading. Entry points may be called from several host threads; calls
 * that share a (device, stream) pair are serialized on a lock. All GPU work
 * is enqueued on the caller's stream and no entry point waits for the device,
 * except ns_profile_read and ns_release_workspace as documented, and the
 * NS_CHECK debug mode below.
 *
 * Environment (read at every call):
 *   NS_SMALL_M=t  an integer 0..32: matrices with min(rows, cols) <= t take
 *                 the small-matrix path (default 32); others the tiled path.
 *                 Other values are ignored.
 *   NS_CHECK=1    debug mode: the call waits for the stream after every
 *                 kernel launch and returns NS_EHIP naming the first kernel
 *                 that failed.
 */
#ifndef NS_H
#define NS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NS_BF16 = 0, /* bfloat16 storage */
    NS_FP32 = 1  /* float32 storage  */
} ns_dtype;

typedef enum {
    NS_OK = 0,      /* success (work enqueued)                                */
    NS_EINVAL = 1,  /* invalid argument; nothing was enqueued                 */
    NS_EDTYPE = 2,  /* unknown dtype; nothing was enqueued                    */
    NS_ENOMEM = 3,  /* device or host allocation failed; nothing enqueued     */
    NS_EHIP = 4     /* a HIP call or kernel launch failed; see ns_last_error  */
} ns_status;

#define NS_QUINTIC_A 3.4445f
#define NS_QUINTIC_B (-4.7750f)
#define NS_QUINTIC_C 2.0315f

/*
 * Orthogonalize `count` matrices in place.
 *
 *   ptrs    host array of `count` device pointers. ptrs[i] points at matrix i:
 *           shapes[2i] x shapes[2i+1] elements of `dtype`, row-major and
 *           contiguous (leading dimension = cols), aligned to the element
 *           size. Read as G, overwritten with the result. Matrices must not
 *           overlap. A pointer may be NULL only for an empty matrix.
 *   shapes  host array of 2*count int64: (rows, cols) per matrix, each >= 0.
 *           rows == 0 or cols == 0 is an empty matrix (an empty shard): it is
 *           accepted and never touched.
 *   count   number of matrices, >= 0; 0 enqueues nothing.
 *   steps   iterations, >= 0. steps == 0 writes G / (||G||_F + 1e-7).
 *   coeffs  host array of 3 floats (a, b, c) applied at every step; may be
 *           NULL only when steps == 0.
 *   dtype   an ns_dtype; all matrices of a call share it.
 *   stream  a hipStream_t (NULL = the legacy default stream) on the current
 *           device. All work is enqueued on it; the results are complete in
 *           stream order. Host arrays are only read before the call returns.
 *
 * Workspace: the library keeps a device workspace per (device, stream) pair,
 * grown on demand with stream-ordered allocation (hipMallocAsync /
 * hipFreeAsync), plus a cache of up to 64 batch plans keyed by the argument
 * values (shapes, pointers, dtype). Two calls on the same stream are ordered
 * by the stream; calls on different streams use separate workspaces.
 *
 * Never blocks: the call enqueues its work and returns without waiting for
 * the device, however much work is already queued on the stream (the hang
 * and hidden sync point microsoft/dion PR #74, "Fix
 * megabatch_orthogonalize_async hang on empty FSDP2 shards", Concrete repro
 * and review thread, are about). A batch not in the plan cache uploads its
 * descriptors and tile lists from pinned host staging buffers; one still
 * feeding an earlier upload is never waited for: a new buffer is allocated
 * instead, up to 256 MiB of them per (device, stream), past which the call
 * returns NS_ENOMEM (with nothing enqueued) rather than wait.
 *
 * Errors (all reported before anything is enqueued, except NS_EHIP):
 *   NS_EINVAL  negative count, steps or dimension; NULL ptrs/shapes with
 *              count > 0; NULL pointer for a non-empty matrix; a pointer not
 *              aligned to the element size; NULL coeffs with steps > 0; a
 *              dimension above 2^24; a tiled-path matrix (min(rows, cols)
 *              above the small-path threshold) whose padded operand is too large for 32-bit buffer
 *              offsets: with m, n rounded up to multiples of 256 (mp, np),
 *              np x mp x element size must stay below 2 GiB and
 *              np x 256 x element size below 2 GiB (e.g. 32768 x 32768 bf16
 *              or 8192 x 131072 bf16 is rejected; 10240 x 10240 and
 *              8192 x 65536 bf16 are accepted).
 *   NS_EDTYPE  unknown dtype.
 *   NS_ENOMEM  the workspace or the metadata staging cannot be allocated.
 *   NS_EHIP    a HIP call or kernel launch failed.
 * On any error the message is available from ns_last_error(). NaN and Inf
 * propagate unchecked: a NaN entry makes the whole result NaN.
 */
ns_status ns_orthogonalize_batched(void* const* ptrs, const int64_t* shapes,
                                   int32_t count, int32_t steps,
                                   const float* coeffs, int32_t dtype,
                                   void* stream);

/* Longest coefficient schedule ns_orthogonalize_batched_sched accepts. */
#define NS_MAX_SCHEDULE_STEPS 64

/*
 * As ns_orthogonalize_batched, but step s (0-based) uses its own polynomial:
 *
 *   coeffs  host array of 3*steps floats; (coeffs[3s], coeffs[3s+1],
 *           coeffs[3s+2]) are (a, b, c) of step s. May be NULL only when
 *           steps == 0.
 *   steps   0 .. NS_MAX_SCHEDULE_STEPS.
 *
 * With every triple equal to (a, b, c) the result is bit for bit that of
 * ns_orthogonalize_batched with (a, b, c). This serves iterations whose
 * polynomial changes from step to step, e.g. a few quintic steps followed by
 * cubic (1.5, -0.5, 0) steps that converge to the polar factor UV^T.
 * Errors as ns_orthogonalize_batched, plus NS_EINVAL for steps above
 * NS_MAX_SCHEDULE_STEPS.
 */
ns_status ns_orthogonalize_batched_sched(void* const* ptrs, const int64_t* shapes,
                                         int32_t count, int32_t steps,
                                         const float* coeffs, int32_t dtype,
                                         void* stream);

/*
 * As ns_orthogonalize_batched, for matrices that arrive as row blocks: the
 * row shards an all-to-all hands to the rank that orthogonalizes a matrix
 * (microsoft/dion PR #74, "Fix megabatch_orthogonalize_async hang on empty
 * FSDP2 shards", Summary and Fix: shards of a padded split, some of them
 * empty; InternLM/xtuner PR #2069, the ragged exchange that sends each shard
 * at its own length). Matrix i is the vertical concatenation of its
 * nchunks[i] blocks; it is orthogonalized as that whole matrix and the result
 * is written back into the same blocks, so no assembly or split copy is made.
 * Result bits equal those of ns_orthogonalize_batched on the concatenated
 * matrix.
 *
 *   chunk_ptrs  host array of sum(nchunks) device pointers, matrix 0's blocks
 *               first, each block top to bottom. Block k holds chunk_rows[k]
 *               rows of cols[i] elements, row-major and contiguous, aligned
 *               to the element size; NULL only for an empty block.
 *   chunk_rows  host array of sum(nchunks) int64 row counts, each >= 0. A
 *               block of 0 rows (an empty shard) is never touched.
 *   nchunks     host array of `count` int32 block counts, each >= 0.
 *   cols        host array of `count` int64 column counts, each >= 0.
 *   count, steps, coeffs, dtype, stream: as ns_orthogonalize_batched.
 *
 * Blocks must not overlap. Errors as ns_orthogonalize_batched (NS_EINVAL
 * also for a negative block count or block row count, and for a matrix whose
 * rows add up above 2^24).
 */
ns_status ns_orthogonalize_chunked(void* const* chunk_ptrs, const int64_t* chunk_rows,
                                   const int32_t* nchunks, const int64_t* cols,
                                   int32_t count, int32_t steps,
                                   const float* coeffs, int32_t dtype,
                                   void* stream);

/* Device scratch of ns_orthogonalize_batched_noalloc, per device. */
#define NS_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/*
 * As ns_orthogonalize_batched (same arguments, results bit for bit the same),
 * for callers that cannot allocate: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation. This call makes no device
 * or pinned-host allocation (no hipMalloc, hipMallocAsync, hipHostMalloc or
 * hipFree of any kind) and never waits for the device.
 *
 * Workspace: a static device array of NS_NOALLOC_SCRATCH_BYTES that each
 * device this library runs on holds until the process ends (reserved when
 * the library's code is loaded on the device). The batch's workspace and
 * metadata must fit it: ns_workspace_bytes(shapes, count, dtype) + 256 <=
 * NS_NOALLOC_SCRATCH_BYTES (e.g. the 32 attention-gate matrices of 24 x 2304,
 * or one 2048 x 6144 bf16 matrix); a larger batch is rejected with NS_EINVAL
 * before anything is enqueued. The metadata goes up through kernel
 * arguments (one small copy kernel per 2 KB).
 *
 * Every call on a device shares that device's array, which keeps the last
 * call's contents: calls that overlap on one device race (two streams, or two
 * host threads); calls on one stream are ordered by it. Nothing in the array
 * needs to start at any value.
 *
 * Errors as ns_orthogonalize_batched, plus NS_EINVAL for a batch that does
 * not fit the scratch array.
 */
ns_status ns_orthogonalize_batched_noalloc(void* const* ptrs, const int64_t* shapes,
                                           int32_t count, int32_t steps,
                                           const float* coeffs, int32_t dtype,
                                           void* stream);

/*
 * Placement of whole matrices onto `world` data-parallel ranks (host-only; no
 * device is touched): which rank orthogonalizes each matrix and where it sits
 * in that rank's shard of its bucket buffer. NVIDIA/Megatron-LM PR #6379,
 * "Balance LayerWise optimizer shards by Newton-Schulz cost, not parameter
 * size", Problem, Changes 1-3 and Notes.
 *
 *   numel        count element counts of the parameters as stored (a GTP
 *                shard's local count), in backprop order.
 *   cost         count Newton-Schulz costs of the full shapes
 *                (ns_compute_cost of the all-gathered matrix; the element count
 *                for a non-matrix parameter).
 *   world        ranks (> 0); bucket_size: element threshold of a bucket
 *                (>= 0); align: shard start alignment in elements (>= 1).
 *   by_cost      1: largest cost first onto the rank with the least cost so far
 *                (loads kept across buckets) among ranks whose shard stays under
 *                1.3 x (bucket numel / world); a matrix that fits nowhere goes to
 *                the rank with the least numel in the bucket. 0: the earlier
 *                rule, largest numel first onto the rank with the least numel.
 *   absorb       1: bucket_size is a soft minimum: once a bucket reaches it, a
 *                further parameter still joins while a least-loaded placement in
 *                backprop order puts it into existing padding. 0: a bucket
 *                closes as soon as it reaches bucket_size.
 *   rank, offset, bucket  count outputs: rank, element offset within that
 *                rank's shard of the bucket, bucket index.
 *   bucket_elems outputs per bucket (room for count entries): elements the
 *                bucket's buffer holds, world x the largest shard.
 *   nbuckets     output: number of buckets.
 *   rank_cost    optional (may be NULL) world outputs: total cost per rank.
 *
 * Returns NS_EINVAL for negative counts/sizes/costs, world < 1, align < 1 or a
 * NULL output; NS_OK otherwise.
 */
ns_status ns_plan_ranks(const int64_t* numel, const int64_t* cost, int32_t count, int32_t world,
                        int64_t bucket_size, int64_t align, int32_t by_cost, int32_t absorb,
                        int32_t* rank, int64_t* offset, int32_t* bucket, int64_t* bucket_elems,
                        int32_t* nbuckets, int64_t* rank_cost);

/*
 * Device workspace bytes a call with these shapes and dtype needs (host-only;
 * touches no device): lets a caller check the footprint before a call. Same
 * validation of shapes/count/dtype as ns_orthogonalize_batched, including the
 * too-large-for-the-tiled-path NS_EINVAL.
 */
ns_status ns_workspace_bytes(const int64_t* shapes, int32_t count,
                             int32_t dtype, size_t* out_bytes);

/*
 * Free the workspace and plan cache held for (current device, stream): the
 * ownership half of the per-stream workspace that ns_orthogonalize_batched
 * grows on demand. Device memory is released with stream-ordered frees on
 * `stream`, so this is safe while earlier calls are in flight; the pinned
 * host staging buffers are freed after a host wait for their pending uploads
 * (the one entry point that waits). Returns NS_OK if nothing was held.
 */
ns_status ns_release_workspace(void* stream);

/* Message of the last non-OK status on the calling thread ("" if none): the
 * error channel of every entry point above. The string stays valid until the
 * thread's next call into the library. */
const char* ns_last_error(void);

/* Library version string. */
const char* ns_version(void);

/*
 * Newton-Schulz cost of a rows x cols matrix, max(M,N) * min(M,N)^2, the
 * model the Megatron-LM page (PR #6379, Changes item 1) ranks work by and the
 * batch scheduler orders matrices by. 0 for an empty matrix, -1 for a
 * negative dimension. Host-only.
 */
int64_t ns_compute_cost(int64_t rows, int64_t cols);

/*
 * Host-only view of the batch plan, for tests and tools.
 *
 * ns_plan_classify: kinds[i] = 0 (empty), 1 (small: min(rows, cols) <= the
 * NS_SMALL_M threshold, the fp64 Gram-form kernel, one workgroup per
 * 512-column slice), 2 (large: tiled MFMA path).
 *
 * ns_plan_tiles: the tile list of one grouped GEMM stage in launch order.
 *   stage 0 = A = X X^T (upper-triangle tiles), 1 = B = bA + cA^2 (same
 *   tiles), 2 = X <- aX + BX (all tiles). Each tile is 4 int32:
 *   (matrix index into the caller's batch, block row, block column, K depth
 *   in elements). Writes min(capacity, total) tiles to `out` (which may be
 *   NULL when capacity is 0) and the total count to *n_tiles.
 *   *tile_size receives the tile edge in elements.
 */
ns_status ns_plan_classify(const int64_t* shapes, int32_t count, int32_t dtype,
                           int32_t* kinds);
ns_status ns_plan_tiles(const int64_t* shapes, int32_t count, int32_t dtype,
                        int32_t stage, int32_t* out, int64_t capacity,
                        int64_t* n_tiles, int32_t* tile_size);

/*
 * Per-kernel timing with HIP events recorded on the call's stream around
 * every launch the library makes while profiling is on.
 *
 * Kinds: 0 norm partial sums, 1 norm finalize, 2 normalize/transpose/pad,
 * 3 X X^T, 4 bA + cA^2, 5 aX + BX (and final write-back), 6 small-matrix
 * fused kernel, 7 steps==0 write-back.
 *
 * ns_profile_enable(1) clears the accumulators and starts recording;
 * ns_profile_enable(0) stops. ns_profile_read waits for every recorded event
 * (a host wait on the events only), then writes, for the first n_kinds kinds,
 * the total milliseconds and the launch count since the last clear.
 */
#define NS_PROFILE_KINDS 8
ns_status ns_profile_enable(int32_t on);
ns_status ns_profile_read(double* total_ms, int64_t* launches, int32_t n_kinds);

#ifdef __cplusplus
}
#endif

#endif /* NS_H */
