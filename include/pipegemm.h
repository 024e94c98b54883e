/*
 * pipegemm — a software-pipelined tiled half-precision GEMM for MI355X (gfx950).
 *
 *   C[M,N] = A[M,K] x B          fp16 or bf16 inputs, fp32 accumulation,
 *                                C written in the input dtype (round to
 *                                nearest, ties to even)
 *
 * Two storage forms of B:
 *   gemm_nt  B stored [N,K] row-major (the transpose_B form of the TileLang
 *            tutorial, chapter 11 "pipeline and autotuning", sections 1.1/3.5:
 *            the kernel signature takes A (M,K), B (N,K), C (M,N)).
 *   gemm_nn  B stored [K,N] row-major (the plain form C = A @ B of the
 *            "Stage 04 - GEMM" notes, "concepts" and "code").
 *
 * Each workgroup owns a block_M x block_N tile of C and walks the K dimension
 * in block_K steps.  The tiles of A and B it needs are copied from HBM into a
 * ring of num_stages LDS buffers; copies for later K steps are in flight while
 * the matrix cores work on the current one (chapter 11, sections 1.1-1.3 and
 * 2.3: multi-buffering lets the copy of round ko+1 overlap the compute of round
 * ko; section 4.3: prologue, steady state, epilogue).
 *
 * Shared conventions for every entry point below:
 *  - All sizes are in elements; all matrices are dense, row-major, with no
 *    padding (leading dimension = number of columns).
 *  - A, B and C are DEVICE pointers owned by the caller.  The library never
 *    allocates, frees, or retains them, and keeps no state except a per-device
 *    cache of the LDS limit and a per-thread error message.
 *  - Calls that launch work are asynchronous on the caller's HIP stream
 *    (hip_stream is a hipStream_t; NULL means the null stream).  They return
 *    once the kernel is enqueued.
 *  - Validation is synchronous and happens before any launch.  On any status
 *    other than GEMM_OK nothing is launched and C is not touched;
 *    gemm_last_error() then describes the failure.
 *  - Validation order: (1) arguments, (2) LDS budget, (3) alignment,
 *    (4) supported configuration.  An over-budget request therefore always
 *    reports GEMM_ERR_LDS_BUDGET, whatever else is wrong with its tile.
 *
 * The a_lead option (an MI355X addition to the tutorial's ring): with a_lead = 1 the
 * A tiles get a ring of num_stages + 1 LDS buffers and are copied one K step
 * further ahead than the B tiles, which keep num_stages buffers.  It spends
 * LDS a full extra stage would not fit in (256 x 256 x 64 tiles: two stages
 * are 128 KiB, three would be 192 KiB; two stages plus one A tile are exactly
 * gfx950's 160 KiB) on more copy latency hiding.  The result is bit-identical
 * to a_lead = 0: only the order in which copies are issued changes.
 */
#ifndef PIPEGEMM_H
#define PIPEGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gemm_dtype {
    GEMM_F16 = 0,  /* IEEE binary16 */
    GEMM_BF16 = 1  /* bfloat16 */
};

enum gemm_layout {
    GEMM_NT = 0, /* B stored [N,K] */
    GEMM_NN = 1  /* B stored [K,N] */
};

enum gemm_status {
    GEMM_OK = 0,
    GEMM_ERR_ARG = 1,         /* negative size, null pointer, unknown dtype/layout, bad block/stage/thread value */
    GEMM_ERR_LDS_BUDGET = 2,  /* num_stages x (block_M + block_N) x block_K x 2 bytes (+ block_M x block_K x 2
                                 with a_lead) exceeds the LDS limit */
    GEMM_ERR_UNSUPPORTED = 3, /* no kernel is built for this (dtype, layout, tile, threads), or a size limit of
                                 the kernels' 32-bit buffer offsets is exceeded: M, N, K below 2^31, and below
                                 2 GiB each of max(block_M, block_N) x K x 2 (a workgroup's A or B panel),
                                 block_M x N x 2 (its rows of C) and, for NN, K x N x 2 (B) */
    GEMM_ERR_ALIGN = 4,       /* K (and N for NN) not a multiple of 8, or misaligned pointers */
    GEMM_ERR_HIP = 5          /* a HIP runtime call failed (no device, launch failure) */
};

/*
 * gemm_nt: C[M,N] = A[M,K] . B[N,K]^T.
 *
 * Defined by: TileLang tutorial, chapter 11, section 1.1 (the tiled loop with
 * transpose_B) and section 3.5 (the kernel signature and its parameters with
 * defaults block 128x128x32, num_stages 3, threads 128, fp16 in, fp32
 * accumulate); section 2.1 / 5.4 for num_stages = 0.
 *
 * Arguments:
 *   A           device pointer, [M,K] row-major, dtype elements, 16-byte aligned
 *   B           device pointer, [N,K] row-major, 16-byte aligned
 *   C           device pointer, [M,N] row-major, written in dtype, 8-byte aligned
 *   M, N, K     sizes, >= 0.  M == 0 or N == 0 is a no-op; K == 0 writes C = 0.
 *               K must be a multiple of 8.
 *   dtype       GEMM_F16 or GEMM_BF16 (A, B and C share it)
 *   block_M/N/K the C tile one workgroup owns and the K step (elements)
 *   num_stages  number of LDS ring buffers; 1 = single buffer, no overlap
 *               (the non-pipelined control); 0 = alias of 1 (a loop that is not
 *               pipelined is single-buffered)
 *   a_lead      0, or 1 to give A one more buffer and copy it one K step
 *               earlier (needs num_stages >= 2; built for num_stages <= 4)
 *   threads     threads per workgroup, a multiple of 64 (0 selects 256)
 *   hip_stream  hipStream_t to launch on, or NULL
 * Returns a gemm_status.  Partial tiles at the M, N and K edges are handled:
 * out-of-range A/B elements are read as zero and out-of-range C is never written.
 */
int gemm_nt(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int dtype,
            int block_M, int block_N, int block_K, int num_stages, int a_lead, int threads, void *hip_stream);

/*
 * gemm_nn: C[M,N] = A[M,K] . B[K,N].
 *
 * Defined by: "Stage 04 - GEMM" notes ("concepts": C[M,N] = A[M,K] @ B[K,N],
 * fp32 accumulation; "code": T.gemm(A_shared, B_shared, C_local) inside a
 * T.Pipelined K loop).  Arguments and behaviour as gemm_nt, except B is
 * [K,N] row-major and N must also be a multiple of 8.
 */
int gemm_nn(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int dtype,
            int block_M, int block_N, int block_K, int num_stages, int a_lead, int threads, void *hip_stream);

/*
 * gemm_nt_relu, gemm_nn_relu: C = relu(A . B) with the ReLU fused into the
 * store of C: each fp32 sum s becomes (s > 0 ? s : +0) before it is rounded to
 * the input dtype (a NaN sum gives +0).
 *
 * Defined by: TileLang tutorial, chapter 11, section 4.6 (the GEMM+ReLU
 * example on the same pipelined K loop).  Arguments, layouts, validation and
 * errors exactly as gemm_nt / gemm_nn.
 */
int gemm_nt_relu(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int dtype,
                 int block_M, int block_N, int block_K, int num_stages, int a_lead, int threads, void *hip_stream);
int gemm_nn_relu(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int dtype,
                 int block_M, int block_N, int block_K, int num_stages, int a_lead, int threads, void *hip_stream);

/*
 * gemm_stamped: gemm_nt (layout GEMM_NT) or gemm_nn (GEMM_NN) that also
 * records, per workgroup, when its phases ran, so the stage-count knee can be
 * read off measured cycles per K tile: the prologue, steady state and
 * epilogue of chapter 11, section 4.3, and the copy/compute period of
 * sections 1.2-1.3 and 2.2.
 *
 * Workgroup w (its dispatch index, 0 .. ceil(M/block_M) ceil(N/block_N) - 1;
 * it runs on XCD w mod 8) writes six counters to stamps[6w .. 6w+5]:
 *   [0] shader-clock cycle counter (s_memtime) at its start,
 *   [1] the same once its first K tile has landed (after the prologue),
 *   [2] the same after its K loop,
 *   [3] the same at its end (after it issued its stores of C),
 *   [4] the constant 100 MHz real-time counter (s_memrealtime) at its start,
 *   [5] the same at its end.
 * The shader clock of the run is (stamps[3] - stamps[0]) / (stamps[5] -
 * stamps[4]) x 100 MHz.  The values of different XCDs' cycle counters are
 * not comparable with each other; differences within one workgroup are.
 *
 * stamps: device pointer, 8-byte aligned, to at least 6 x grid uint64 values,
 * owned by the caller; the kernel only writes it (no count is checked).  All
 * other arguments, the validation and the errors are those of gemm_nt /
 * gemm_nn; a null or misaligned stamps pointer is an argument error
 * (GEMM_ERR_ARG).
 * The computation and C are the same as without stamps.
 */
int gemm_stamped(int layout, const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int dtype,
                 int block_M, int block_N, int block_K, int num_stages, int a_lead, int threads, void *hip_stream,
                 uint64_t *stamps);

/*
 * gemm_lds_bytes: LDS the pipeline of one workgroup needs,
 *   max(num_stages, 1) x (block_M x block_K + block_K x block_N) x 2 bytes,
 *   plus block_M x block_K x 2 bytes when a_lead is 1.
 *
 * Defined by: TileLang tutorial, chapter 11, section 4.5 (per-stage bytes of
 * the A and B tiles times the stage count; the accumulator lives in registers).
 * Pure host arithmetic.  Returns -1 for a negative block size, a negative stage
 * count, an a_lead other than 0 or 1, or an unknown dtype.
 */
int64_t gemm_lds_bytes(int block_M, int block_N, int block_K, int num_stages, int a_lead, int dtype);

/*
 * gemm_lds_budget: the LDS limit of one workgroup on the current HIP device
 * (hipDeviceAttributeMaxSharedMemoryPerBlock; 163840 bytes on gfx950).
 * Returns -1 if no device is available (see gemm_last_error()).
 */
int64_t gemm_lds_budget(void);

/*
 * gemm_check: run the validation of gemm_nt / gemm_nn (layout selects which)
 * on sizes and configuration alone, against the given LDS budget in bytes
 * (0 = the current device's, which needs a device).  Pointer checks are
 * skipped.  Pure host code when lds_budget > 0: no device is touched.
 * Defined by: chapter 11, sections 4.5 and 5.1 (over budget is a hard
 * failure, never a slowdown).  Returns a gemm_status.
 */
int gemm_check(int layout, int64_t M, int64_t N, int64_t K, int dtype, int block_M, int block_N,
               int block_K, int num_stages, int a_lead, int threads, int64_t lds_budget);

/*
 * Tuning (TileLang tutorial, chapter 11, sections 3.5-3.8: a configuration
 * space given per problem, pre-pruned of tiles that do not divide the problem
 * and of over-budget combinations, every candidate measured on the same
 * operands, and the result fixed as a per-device default).
 *
 * gemm_config: the tuned parameters of gemm_nt / gemm_nn.
 */
typedef struct gemm_config {
    int32_t block_M, block_N, block_K;
    int32_t num_stages;
    int32_t a_lead;
    int32_t threads;
} gemm_config;

/* gemm_prune status of a candidate whose tile does not divide M, N or K */
#define GEMM_PRUNE_NODIV 16

/*
 * gemm_configs: the built configuration space for (layout, dtype): every tile
 * and thread count with a kernel, with every ring depth the kernel is built
 * for (num_stages 1..10, a_lead 0 or 1) whose LDS fits 160 KiB.  Writes up to
 * `max` entries to `out` (out may be NULL when max is 0) and returns the total
 * number, or -1 for an unknown layout or dtype.  Pure host.
 */
int gemm_configs(int layout, int dtype, gemm_config *out, int max);

/*
 * gemm_prune: pre-pruning (chapter 11, section 3.7).  For each of the n
 * candidates writes status[i]: GEMM_PRUNE_NODIV if its tile does not divide
 * M, N and K, otherwise what gemm_check returns for it against lds_budget
 * (0 = the current device's).  Returns the number of candidates left with
 * GEMM_OK, or -1 for bad arguments.  Pure host when lds_budget > 0.
 */
int gemm_prune(int layout, int64_t M, int64_t N, int64_t K, int dtype, const gemm_config *cands, int n,
               int64_t lds_budget, int *status);

/*
 * gemm_rank: an analytic cost for each of the n candidates (chapter 11,
 * section 3.9: a cost model that knows the hardware orders the search and
 * flags ties; it does not replace measurement).  cost[i] is a modelled time in
 * microseconds for an M x N x K problem: per K tile the larger of MFMA time,
 * copy time (with a measured penalty for block_K = 32) and LDS read time,
 * plus the copy latency the ring depth leaves uncovered, times the rounds of
 * workgroups that fit the 256 compute units at the occupancy LDS and an
 * estimate of the registers allow, plus the C store.  The constants were
 * fitted to measured gfx950 tuning tables (see the library source); the pages
 * print no model to pin against, so its only test is how it orders measured
 * candidates.
 * Returns GEMM_OK, or GEMM_ERR_ARG for negative sizes, null arrays or a
 * malformed candidate (threads must be a positive multiple of 128 or 0).
 * Pure host.
 */
int gemm_rank(int64_t M, int64_t N, int64_t K, const gemm_config *cands, int n, double *cost);

/*
 * gemm_tune: measures every candidate whose status[i] is GEMM_OK on the same
 * operands (chapter 11, sections 3.5-3.6): `warmup` launches, then `reps`
 * launches timed together with HIP events on hip_stream.  Writes the mean
 * milliseconds per launch to ms[i] (-1 for skipped candidates) and the index
 * of the fastest to *best (-1 if none ran).  A, B, C and the sizes are as for
 * gemm_nt / gemm_nn (layout selects which).  The accumulation order over K
 * does not depend on the tile or the ring, and the two MFMA shapes gave
 * bit-identical C on every input tested, so in practice every candidate
 * writes the same C.
 * Synchronous: returns after the last timed launch has finished.  Returns
 * GEMM_OK or the status of the first failing launch (then the remaining ms[i]
 * are not written).
 */
int gemm_tune(int layout, const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int dtype,
              const gemm_config *cands, const int *status, int n, int warmup, int reps, void *hip_stream,
              float *ms, int *best);

/*
 * gemm_default_config: the configuration this library picks for a problem on
 * gfx950 without tuning (chapter 11, section 3.8: fix the tuned result as a
 * per-device default): one entry per tile, each with the ring and thread count
 * measured best for it on gfx950 -- 256x256x64 (2 stages + a_lead, 512
 * threads), 256x128x64 (3, 256), 128x256x64 (3, 512), 128x128x64 (3, 512),
 * 64x128x64 (4, 256) -- and among them the one gemm_rank models
 * cheapest for the problem.  Pure host.  Returns GEMM_OK or GEMM_ERR_ARG.
 */
int gemm_default_config(int layout, int64_t M, int64_t N, int64_t K, int dtype, gemm_config *out);

/*
 * gemm_last_error: message describing the last non-OK status returned on
 * this thread ("" if none).  The string is owned by the library and stays
 * valid until the next call on this thread.
 */
const char *gemm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PIPEGEMM_H */
