/*
 * pipeattn — the attention forward pass on the same software-pipelined LDS
 * ring as the GEMM (MI355X, gfx950).  Exported by the same library
 * (libpipegemm.so); errors are reported through gemm_last_error().
 *
 *   O[b,h,i,:] = sum_j softmax_j( scale * Q[b,h,i,:] . K[b,h/g,j,:] ) V[b,h/g,j,:]
 *
 * Defined by: TileLang tutorial, chapter 11, section 1.4 (the attention
 * KV-length loop is a long reduction loop pipelined like the GEMM K loop) and
 * section 3.8 (the flashattn(batch, heads, seq_len, dim, is_causal, groups,
 * block_M, block_N, num_stages, threads) kernel); Tilelang-Learning notes
 * "Stage 04 - GEMM" (QK^T and P@V are the two GEMMs of attention).
 *
 * Conventions (as pipegemm.h): device pointers owned by the caller, dense
 * row-major tensors, asynchronous on the caller's stream, synchronous
 * validation in the order arguments, LDS budget, alignment, supported
 * configuration; on any error nothing is launched and O is untouched.
 */
#ifndef PIPEATTN_H
#define PIPEATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * attn_fwd: the attention forward pass.
 *
 *   Q          device pointer, [batch, heads, seq_q, dim], dtype elements, 16-byte aligned
 *   K, V       device pointers, [batch, kv_heads, seq_kv, dim], 16-byte aligned
 *   O          device pointer, [batch, heads, seq_q, dim], written in dtype, 16-byte aligned;
 *              nothing outside it is written (streaming stores)
 *   batch, heads, kv_heads, seq_q, seq_kv   >= 1; heads a multiple of kv_heads
 *              (query head h reads KV head h / (heads / kv_heads))
 *   dim        head dimension; 64 and 128 are built
 *   dtype      GEMM_F16 or GEMM_BF16 (pipegemm.h); fp32 scores, softmax and
 *              accumulation; P is rounded to dtype for the second product and
 *              for the row sum
 *   is_causal  1: query i sees keys j <= i (needs seq_q == seq_kv)
 *   scale      softmax scale: 0 selects 1 / sqrt(dim); otherwise it must be
 *              positive and finite (a negative, infinite or NaN scale is an
 *              argument error, GEMM_ERR_ARG, reported before anything else)
 *   block_M    queries per workgroup, 32 or 64 per wave (threads = 2 x block_M
 *              or block_M); built, for each dim: (block_M, block_N, threads) =
 *              (128, 64, 256), (256, 64, 512), (128, 128, 256), (256, 128, 512),
 *              (256, 64, 256); for dim 64 also (512, 64, 512), (512, 128, 512)
 *   block_N    keys per LDS tile: 64 or 128
 *   num_stages LDS ring slots, each holding one K and one V tile
 *              (num_stages x 2 x block_N x dim x 2 bytes of LDS); 1 = single
 *              buffer; 0 = alias of 1
 *   threads    64 x waves (0 selects 2 x block_M, i.e. 32 queries per wave)
 * Returns a gemm_status (pipegemm.h).
 */
int attn_fwd(const void *Q, const void *K, const void *V, void *O, int64_t batch, int64_t heads, int64_t kv_heads,
             int64_t seq_q, int64_t seq_kv, int64_t dim, int dtype, int is_causal, float scale, int block_M,
             int block_N, int num_stages, int threads, void *hip_stream);

/*
 * attn_lds_bytes: max(num_stages, 1) x (block_N x dim) x 2 tiles x 2 bytes
 * (chapter 11, section 4.5: the versioned buffers times the stage count).
 * Returns -1 for negative arguments.  Pure host.
 */
int64_t attn_lds_bytes(int block_N, int dim, int num_stages);

/*
 * attn_check: the validation of attn_fwd on sizes and configuration alone,
 * against lds_budget bytes (0 = the current device's).  Pure host when
 * lds_budget > 0.  Returns a gemm_status.
 */
int attn_check(int64_t batch, int64_t heads, int64_t kv_heads, int64_t seq_q, int64_t seq_kv, int64_t dim, int dtype,
               int is_causal, int block_M, int block_N, int num_stages, int threads, int64_t lds_budget);

/*
 * attn_default_config: the gfx950 default configuration for these sizes
 * (chapter 11, section 3.8: a tuned result fixed as the device's default),
 * from timings of the built tiles at 4096 keys over 4 x 32 heads and on
 * smaller grids:
 *   - dim 128: block_M 256, block_N 128, 2 stages, 512 threads (8 waves);
 *   - dim 64 without the mask: block_M 512, block_N 128, 2 stages, 512
 *     threads (two 32-query blocks per wave);
 *   - dim 64 with the mask, and wherever the 8-wave tile's grid
 *     (batch x heads x ceil(seq_q / block_M)) would be under 256 workgroups,
 *     one per compute unit: block_M 128, block_N 64, 2 stages, 256 threads
 *     (4 waves; two such workgroups share a compute unit).
 * Writes *block_M, *block_N, *num_stages and *threads.  Returns GEMM_OK,
 * GEMM_ERR_ARG (a null output, a size below 1, is_causal not 0 or 1) or
 * GEMM_ERR_UNSUPPORTED (a dim that is not built).  Pure host; the result
 * passes attn_check for every size attn_fwd accepts.
 */
int attn_default_config(int64_t batch, int64_t heads, int64_t seq_q, int64_t dim, int is_causal, int *block_M,
                        int *block_N, int *num_stages, int *threads);

#ifdef __cplusplus
}
#endif

#endif /* PIPEATTN_H */
