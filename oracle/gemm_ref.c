/*
 * CPU oracle for the tiled half-precision GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * loads this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant with the GPU
 * path.
 *
 * What it computes (the plain definition, written out):
 *
 *   NT form  C[m,n] = round( sum_{k=0..K-1} a(A[m,k]) * a(B[n,k]) )   B stored [N,K]
 *   NN form  C[m,n] = round( sum_{k=0..K-1} a(A[m,k]) * a(B[k,n]) )   B stored [K,N]
 *
 * where a() widens an fp16/bf16 encoding to binary32 exactly, the sum is a
 * sequential binary32 sum in ascending k (each addition rounded to nearest,
 * ties to even), and round() narrows the binary32 sum back to the input format
 * with round-to-nearest-even.
 *
 * With the ReLU epilogue the binary32 sum s becomes relu(s) = (s > 0 ? s : +0)
 * before the narrowing (so a NaN sum and -0 both give +0).
 *
 * Sources:
 *  - TileLang tutorial, chapter 11 "pipeline and autotuning", section 1.1
 *    (the tile loop: clear the fp32 fragment, accumulate A-tile x B-tile^T over
 *    the K loop, copy the fragment out in the input dtype) and section 3.6
 *    (the reference program: widen both operands to float, multiply with B
 *    transposed, cast back to the input dtype).
 *  - TileLang tutorial, code/04-tilelang-pipelined-gemm README, "expected
 *    output": results are compared with torch.matmul with fp16 inputs and
 *    fp32 accumulation.
 *  - Tilelang-Learning notes "Stage 04 - GEMM", "concepts": the NN form
 *    C[M,N] = A[M,K] @ B[K,N] with fp32 accumulation for fp16/bf16 inputs.
 *  - TileLang tutorial, chapter 11, section 4.6: the GEMM+ReLU example, a
 *    pipelined K loop whose result goes through ReLU (max with zero); where
 *    ReLU sits relative to the narrowing is not stated, and applying it to the
 *    fp32 sum is the plainest reading (narrowing is monotone and maps 0 to 0,
 *    so for finite sums either order gives the same encoding).
 *  The accumulation order and the rounding mode are not stated by the pages;
 *  ascending k and round-to-nearest-even are the plainest readings.
 *
 * Floating-point formats follow IEEE 754-2008 binary16 (5 exponent bits, 10
 * stored significand bits) and bfloat16 (the upper half of binary32: 8 exponent
 * bits, 7 stored significand bits).  Conversions are written from those
 * definitions, not from any library.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (see build.py).
 * -ffp-contract=off keeps "a*b" and "+" as two rounded operations, exactly as
 * written; for fp16 and bf16 operands the product is exact in binary32 anyway
 * (11x11 and 8x8 significand bits), so the choice cannot change a result
 * unless a bf16 product underflows binary32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1 };
enum { ORACLE_B_NK = 0, ORACLE_B_KN = 1 };

/* Exponent and stored-significand widths of the two 16-bit formats. */
static int exp_bits(int dtype) { return dtype == ORACLE_BF16 ? 8 : 5; }
static int man_bits(int dtype) { return dtype == ORACLE_BF16 ? 7 : 10; }

/* Exact value of a 16-bit encoding, as binary32. */
float oracle_decode(uint16_t bits, int dtype)
{
    const int eb = exp_bits(dtype), mb = man_bits(dtype);
    const int bias = (1 << (eb - 1)) - 1;
    const int emax_field = (1 << eb) - 1;
    const int sign = (bits >> (eb + mb)) & 1;
    const int efield = (bits >> mb) & emax_field;
    const int mant = bits & ((1 << mb) - 1);
    float v;
    if (efield == emax_field) {
        v = mant ? NAN : INFINITY;
    } else if (efield == 0) {
        /* subnormal: mant * 2^(1 - bias - mb) */
        v = ldexpf((float)mant, 1 - bias - mb);
    } else {
        /* normal: (2^mb + mant) * 2^(efield - bias - mb) */
        v = ldexpf((float)((1 << mb) + mant), efield - bias - mb);
    }
    return sign ? -v : v;
}

/*
 * Nearest 16-bit value to x, ties to even, returned as its encoding.
 *
 * For |x| in [2^e, 2^(e+1)) with e at least the format's smallest normal
 * exponent, representable neighbours are spaced q = 2^(e - mb) apart; below
 * the normal range the spacing stays at the subnormal quantum.  |x|/q is an
 * exact scaling by a power of two, and rintf() rounds it to the nearest
 * integer with ties to even (the default rounding mode).  The encoding of the
 * result is then ((e + bias - 1) << mb) + n: for a normal result n carries the
 * hidden bit, which adds the missing 1 to the exponent field; for a subnormal
 * result (e clamped to emin = 1 - bias) the field is 0 and the encoding is n;
 * a carry out of the significand lands in the next exponent automatically.
 */
uint16_t oracle_encode_rne(float x, int dtype)
{
    const int eb = exp_bits(dtype), mb = man_bits(dtype);
    const int bias = (1 << (eb - 1)) - 1;
    const int emin = 1 - bias;
    const uint32_t sign = signbit(x) ? (1u << (eb + mb)) : 0u;
    const uint32_t inf = ((1u << eb) - 1u) << mb;
    if (isnan(x))
        return (uint16_t)(sign | inf | (1u << (mb - 1)));
    const float ax = fabsf(x);
    if (isinf(ax))
        return (uint16_t)(sign | inf);
    if (ax == 0.0f)
        return (uint16_t)sign;
    int E;
    frexpf(ax, &E); /* ax = f * 2^E with f in [0.5, 1) */
    int e = E - 1;  /* 2^e <= ax < 2^(e+1) */
    if (e < emin)
        e = emin;
    const float q = ldexpf(1.0f, e - mb);
    const float n = rintf(ax / q);
    const uint64_t enc = ((uint64_t)(e + bias - 1) << mb) + (uint64_t)n;
    if (enc >= inf)
        return (uint16_t)(sign | inf);
    return (uint16_t)(sign | (uint32_t)enc);
}

void oracle_decode_array(const uint16_t *src, float *dst, int64_t count, int dtype)
{
    for (int64_t i = 0; i < count; ++i)
        dst[i] = oracle_decode(src[i], dtype);
}

void oracle_encode_array(const float *src, uint16_t *dst, int64_t count, int dtype)
{
    for (int64_t i = 0; i < count; ++i)
        dst[i] = oracle_encode_rne(src[i], dtype);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* The ReLU epilogue on a binary32 sum: s if s > 0, else +0 (NaN included). */
static float relu_f32(float s) { return s > 0.0f ? s : 0.0f; }

/*
 * Rows [m_begin, m_end) of C.  b_layout selects B stored [N,K] (NT) or [K,N]
 * (NN); relu = 1 applies the ReLU epilogue.  C receives (m_end - m_begin) x N
 * encodings; S, if not NULL, receives the binary32 sums before the epilogue
 * and the final rounding.  fma_count, if not NULL,
 * receives the number of multiply-adds the loops executed.
 *
 * Loop order m, k, n: every C[m,n] still gets its products added one k at a
 * time in ascending k, exactly as the textbook m, n, k triple loop; walking n
 * innermost only lets each row reuse a decoded B row.
 *
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_gemm_rows(const uint16_t *A, const uint16_t *B, int b_layout,
                     int64_t M, int64_t N, int64_t K, int dtype,
                     int64_t m_begin, int64_t m_end, int relu,
                     uint16_t *C, float *S, int64_t *fma_count)
{
    if (!A || !B || !C || M < 0 || N < 0 || K < 0 || m_begin < 0 ||
        m_end > M || m_begin > m_end || (dtype != ORACLE_F16 && dtype != ORACLE_BF16) ||
        (b_layout != ORACLE_B_NK && b_layout != ORACLE_B_KN) || (relu != 0 && relu != 1))
        return -1;
    /* Decode B once into a [K,N] binary32 array (a transposed copy for NT). */
    float *Bkn = (float *)malloc((size_t)(K * N > 0 ? K * N : 1) * sizeof(float));
    if (!Bkn)
        return -1;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            Bkn[k * N + n] = oracle_decode(b_layout == ORACLE_B_NK ? B[n * K + k] : B[k * N + n], dtype);

    int64_t count = 0;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : count) reduction(| : failed)
    for (int64_t m = m_begin; m < m_end; ++m) {
        float *acc = (float *)malloc((size_t)(N > 0 ? N : 1) * sizeof(float));
        if (!acc) {
            failed = 1;
            continue;
        }
        for (int64_t n = 0; n < N; ++n)
            acc[n] = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            const float a = oracle_decode(A[m * K + k], dtype);
            const float *brow = Bkn + k * N;
            for (int64_t n = 0; n < N; ++n)
                acc[n] = acc[n] + a * brow[n];
            count += N;
        }
        const int64_t r = m - m_begin;
        for (int64_t n = 0; n < N; ++n) {
            C[r * N + n] = oracle_encode_rne(relu ? relu_f32(acc[n]) : acc[n], dtype);
            if (S)
                S[r * N + n] = acc[n];
        }
        free(acc);
    }
    free(Bkn);
    if (fma_count)
        *fma_count = count;
    return failed ? -1 : 0;
}

/*
 * Individual elements C[rows[i], cols[i]] for i in [0, count), each by the
 * textbook dot product in ascending k.  Used to check sampled outputs of
 * shapes too large to compute whole.
 */
int oracle_gemm_points(const uint16_t *A, const uint16_t *B, int b_layout,
                       int64_t M, int64_t N, int64_t K, int dtype, int relu,
                       const int64_t *rows, const int64_t *cols, int64_t count,
                       uint16_t *C, float *S)
{
    if (!A || !B || !C || !rows || !cols || (dtype != ORACLE_F16 && dtype != ORACLE_BF16) ||
        (b_layout != ORACLE_B_NK && b_layout != ORACLE_B_KN) || (relu != 0 && relu != 1))
        return -1;
    for (int64_t i = 0; i < count; ++i)
        if (rows[i] < 0 || rows[i] >= M || cols[i] < 0 || cols[i] >= N)
            return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        const int64_t m = rows[i], n = cols[i];
        float s = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            const float a = oracle_decode(A[m * K + k], dtype);
            const float b = oracle_decode(b_layout == ORACLE_B_NK ? B[n * K + k] : B[k * N + n], dtype);
            s = s + a * b;
        }
        C[i] = oracle_encode_rne(relu ? relu_f32(s) : s, dtype);
        if (S)
            S[i] = s;
    }
    return 0;
}
