// Host side of the pipelined tiled GEMM: validation, the table of built
// kernels, and the C-ABI entry points declared in include/pipegemm.h.
#include "pipegemm.h"
#include "pipeattn.h"

#include <hip/hip_runtime.h>

#include <cmath>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "attn_kernel.hpp"
#include "attn_launch.hpp"
#include "pipegemm_kernel.hpp"
#include "pipegemm_launch.hpp"

namespace pipegemm {
namespace {

thread_local char g_err[512] = "";

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

int ok()
{
    g_err[0] = '\0';
    return GEMM_OK;
}

// ---------------------------------------------------------------------------
// Built kernels.  S is a run-time argument of every kernel; the table lists the
// compile-time tile shapes (PG_TILE_LIST) for each dtype and B layout.
typedef hipError_t (*launch_fn)(const KernelArgs &, int grid, int lds_bytes, hipStream_t);

struct Instance {
    int dtype, layout, bm, bn, bk, threads;
    int a_loads, b_loads;  // 1 KiB copies per wave per K tile of A and of B (bound the vmcnt wait)
    launch_fn launch[2];   // [0]: K a multiple of block_K; [1]: ragged last K tile
};

#define PG_ROW(DT, T, LAYOUT, NN, BM, BN, BK, WM, WN)                                                  \
    {DT, LAYOUT, BM, BN, BK, 64 * WM * WN, loads_per_wave(BM, 0, BK, WM * WN), loads_per_wave(0, BN, BK, WM * WN), \
     {&launch<T, NN, BM, BN, BK, WM, WN, false>, &launch<T, NN, BM, BN, BK, WM, WN, true>}},
#define PG_ROW_F16_NT(BM, BN, BK, WM, WN) PG_ROW(GEMM_F16, _Float16, GEMM_NT, false, BM, BN, BK, WM, WN)
#define PG_ROW_BF16_NT(BM, BN, BK, WM, WN) PG_ROW(GEMM_BF16, __bf16, GEMM_NT, false, BM, BN, BK, WM, WN)
#define PG_ROW_F16_NN(BM, BN, BK, WM, WN) PG_ROW(GEMM_F16, _Float16, GEMM_NN, true, BM, BN, BK, WM, WN)
#define PG_ROW_BF16_NN(BM, BN, BK, WM, WN) PG_ROW(GEMM_BF16, __bf16, GEMM_NN, true, BM, BN, BK, WM, WN)

const Instance kInstances[] = {
    PG_TILE_LIST(PG_ROW_F16_NT) PG_TILE_LIST(PG_ROW_BF16_NT)
    PG_TILE_LIST(PG_ROW_F16_NN) PG_TILE_LIST(PG_ROW_BF16_NN)
};

const Instance *find_instance(int dtype, int layout, int bm, int bn, int bk, int threads)
{
    for (const Instance &in : kInstances)
        if (in.dtype == dtype && in.layout == layout && in.bm == bm && in.bn == bn && in.bk == bk &&
            in.threads == threads)
            return &in;
    return nullptr;
}

constexpr int kDefaultThreads = 256;

// LDS of the two rings: S B tiles and S + lead A tiles (S = max(stages, 1)).
int64_t lds_bytes_of(int bm, int bn, int bk, int stages, int lead)
{
    const int64_t s = stages < 1 ? 1 : stages;
    return ((s + lead) * bm * (int64_t)bk + s * (int64_t)bk * bn) * 2;
}

// The checks shared by gemm_check and the launching entry points, in the
// documented order: arguments, LDS budget, alignment (sizes only), supported
// configuration.  On success *inst receives the kernel to launch.
// ptrs is null for a size-only check; otherwise it holds A, B, C.
int validate(int layout, int64_t M, int64_t N, int64_t K, int dtype, int bm, int bn, int bk, int stages,
             int lead, int threads, int64_t budget, const void *const *ptrs, const Instance **inst)
{
    // (1) arguments
    if (layout != GEMM_NT && layout != GEMM_NN)
        return fail(GEMM_ERR_ARG, "unknown layout %d", layout);
    if (M < 0 || N < 0 || K < 0)
        return fail(GEMM_ERR_ARG, "negative size M=%lld N=%lld K=%lld", (long long)M, (long long)N,
                    (long long)K);
    if (dtype != GEMM_F16 && dtype != GEMM_BF16)
        return fail(GEMM_ERR_ARG, "unknown dtype %d", dtype);
    if (bm <= 0 || bn <= 0 || bk <= 0)
        return fail(GEMM_ERR_ARG, "block sizes must be positive (got %d x %d x %d)", bm, bn, bk);
    if (stages < 0)
        return fail(GEMM_ERR_ARG, "num_stages must be >= 0 (got %d)", stages);
    if (lead != 0 && lead != 1)
        return fail(GEMM_ERR_ARG, "a_lead must be 0 or 1 (got %d)", lead);
    if (lead && stages < 2)
        return fail(GEMM_ERR_ARG, "a_lead needs num_stages >= 2 (got %d)", stages);
    if (threads < 0 || threads % 64 != 0 || threads > 1024)
        return fail(GEMM_ERR_ARG, "threads must be 0 or a multiple of 64 up to 1024 (got %d)", threads);
    if (ptrs && M > 0 && N > 0) {
        if (!ptrs[2])
            return fail(GEMM_ERR_ARG, "C is null");
        if (K > 0 && (!ptrs[0] || !ptrs[1]))
            return fail(GEMM_ERR_ARG, "A or B is null");
    }
    if (budget <= 0)
        return fail(GEMM_ERR_ARG, "LDS budget must be positive");
    // (2) LDS budget: num_stages x (A tile + B tile) (+ one A tile with lead),
    // checked before anything else about the tile
    const int64_t need = lds_bytes_of(bm, bn, bk, stages, lead);
    if (need > budget) {
        if (lead)
            return fail(GEMM_ERR_LDS_BUDGET,
                        "LDS budget exceeded: %d stage(s) x (%d x %d + %d x %d) x 2 B + one leading %d x %d A tile = "
                        "%lld B > %lld B available",
                        stages, bm, bk, bk, bn, bm, bk, (long long)need, (long long)budget);
        return fail(GEMM_ERR_LDS_BUDGET,
                    "LDS budget exceeded: %d stage(s) x (%d x %d + %d x %d) x 2 B = %lld B > %lld B available",
                    stages < 1 ? 1 : stages, bm, bk, bk, bn, (long long)need, (long long)budget);
    }
    // (3) alignment: 16-byte copies along the contiguous dimension of A and B
    if (K % 8 != 0)
        return fail(GEMM_ERR_ALIGN, "K must be a multiple of 8 (got %lld)", (long long)K);
    if (layout == GEMM_NN && N % 8 != 0)
        return fail(GEMM_ERR_ALIGN, "N must be a multiple of 8 for the NN form (got %lld)", (long long)N);
    if (ptrs && ((((uintptr_t)ptrs[0]) & 15) || (((uintptr_t)ptrs[1]) & 15)))
        return fail(GEMM_ERR_ALIGN, "A and B must be 16-byte aligned");
    if (ptrs && (((uintptr_t)ptrs[2]) & 7))
        return fail(GEMM_ERR_ALIGN, "C must be 8-byte aligned");
    // (4) supported configuration and size limits of the kernels' 32-bit offsets
    const int th = threads == 0 ? kDefaultThreads : threads;
    const Instance *in = find_instance(dtype, layout, bm, bn, bk, th);
    if (!in)
        return fail(GEMM_ERR_UNSUPPORTED,
                    "no kernel built for %s %s tile %dx%dx%d with %d threads", dtype == GEMM_F16 ? "fp16" : "bf16",
                    layout == GEMM_NT ? "NT" : "NN", bm, bn, bk, th);
    const int s = stages < 1 ? 1 : stages;
    if (s > kMaxStages)
        return fail(GEMM_ERR_UNSUPPORTED, "num_stages above %d is not supported", kMaxStages);
    if (lead && s > kMaxLeadStages)
        return fail(GEMM_ERR_UNSUPPORTED, "a_lead is built for num_stages up to %d", kMaxLeadStages);
    if (!ring_fits_vmcnt(s, lead, in->a_loads, in->b_loads))
        return fail(GEMM_ERR_UNSUPPORTED,
                    "%d stages%s with %d copies per wave per tile exceed the 63 loads one wave can keep in flight", s,
                    lead ? " and a leading A tile" : "", in->a_loads + in->b_loads);
    if (lds_bytes_of(bm, bn, bk, s, lead) > 160 * 1024)
        return fail(GEMM_ERR_UNSUPPORTED, "no kernel is built for rings above 160 KiB of LDS");
    const int64_t lim = (int64_t)1 << 31;
    if (M >= lim || N >= lim || K >= lim)
        return fail(GEMM_ERR_UNSUPPORTED, "sizes must be below 2^31");
    const int64_t panel = (int64_t)(bm > bn ? bm : bn) * K * 2;
    if (panel >= lim)
        return fail(GEMM_ERR_UNSUPPORTED, "a %lld-byte operand panel exceeds the 2 GiB addressable per workgroup",
                    (long long)panel);
    if (layout == GEMM_NN && K * N * 2 >= lim)
        return fail(GEMM_ERR_UNSUPPORTED, "B of the NN form must be below 2 GiB");
    if ((int64_t)bm * N * 2 >= lim)
        return fail(GEMM_ERR_UNSUPPORTED, "a %lld-byte panel of C rows exceeds the 2 GiB addressable per workgroup",
                    (long long)bm * N * 2);
    if (inst)
        *inst = in;
    return ok();
}

// LDS limit of a device, cached.
std::atomic<int64_t> g_budget[64];

int device_budget(int64_t *out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(GEMM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev >= 0 && dev < 64) {
        const int64_t c = g_budget[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *out = c;
            return GEMM_OK;
        }
    }
    int v = 0;
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess)
        return fail(GEMM_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
    if (dev >= 0 && dev < 64)
        g_budget[dev].store(v, std::memory_order_relaxed);
    *out = v;
    return GEMM_OK;
}

int run(int layout, const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int dtype, int bm,
        int bn, int bk, int stages, int lead, int threads, void *stream, int relu = 0,
        unsigned long long *stamps = nullptr)
{
    const void *ptrs[3] = {A, B, C};
    // Argument errors are reported as such even when no device can be queried:
    // run the checks once against an unlimited budget first.
    int st = validate(layout, M, N, K, dtype, bm, bn, bk, stages, lead, threads, 1LL << 40, ptrs, nullptr);
    if (st == GEMM_ERR_ARG)
        return st;
    int64_t budget = 0;
    st = device_budget(&budget);
    if (st != GEMM_OK)
        return st;
    const Instance *in = nullptr;
    st = validate(layout, M, N, K, dtype, bm, bn, bk, stages, lead, threads, budget, ptrs, &in);
    if (st != GEMM_OK)
        return st;
    if (M == 0 || N == 0)
        return ok();

    KernelArgs a{};
    a.A = A;
    a.B = B;
    a.C = C;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.nk = (int)((K + bk - 1) / bk);
    a.stages = stages < 1 ? 1 : stages;
    a.a_lead = lead;
    a.tiles_m = (int)((M + bm - 1) / bm);
    a.tiles_n = (int)((N + bn - 1) / bn);
    a.group_m = a.tiles_m < 4 ? a.tiles_m : 4;
    a.c_vec = (N % 8) == 0 && ((uintptr_t)C & 15) == 0;
    a.relu = relu;
    a.stamps = stamps;
    const int64_t grid = (int64_t)a.tiles_m * a.tiles_n;
    if (grid >= (1LL << 31))
        return fail(GEMM_ERR_UNSUPPORTED, "too many tiles");
    const int lds = (int)lds_bytes_of(bm, bn, bk, a.stages, lead);
    hipError_t e = in->launch[K % bk != 0](a, (int)grid, lds, (hipStream_t)stream);
    if (e != hipSuccess)
        return fail(GEMM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

// ---------------------------------------------------------------------------
// Configuration space, pre-pruning, tuning and the gfx950 default table.

// Every built (tile, threads) with every ring the kernel builds for it, in
// table order, then S ascending, a_lead 0 before 1.
int enumerate_configs(int layout, int dtype, gemm_config *out, int max)
{
    int n = 0;
    for (const Instance &in : kInstances) {
        if (in.layout != layout || in.dtype != dtype)
            continue;
        for (int s = 1; s <= kMaxStages; ++s)
            for (int lead = 0; lead <= 1; ++lead) {
                if (lead && (s < 2 || s > kMaxLeadStages))
                    continue;
                if (!ring_fits_vmcnt(s, lead, in.a_loads, in.b_loads) ||
                    lds_bytes_of(in.bm, in.bn, in.bk, s, lead) > 160 * 1024)
                    continue;
                if (out && n < max)
                    out[n] = gemm_config{in.bm, in.bn, in.bk, s, lead, in.threads};
                ++n;
            }
    }
    return n;
}

int64_t tiles_of(int64_t M, int64_t N, int bm, int bn)
{
    return ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
}

// Analytic cost of one configuration (microseconds at a nominal 2.1 GHz),
// used only to order candidates before they are measured (chapter 11, section
// 3.9: a cost model prunes and ranks, measurement decides).  Per K tile of one
// workgroup: MFMA time C = 2 bM bN bK / 4096 flop per CU-cycle, divided by
// 1.4 for the 16x16x32 tiles (their higher clock under the power limit with
// random operands); copy time X = (bM + bN) bK 2 B at 48 B per cycle, times
// 1.5 for bK = 32, whose 64-byte rows cost two L2 requests per line; LDS
// operand reads R = waves (TM + TN) bK 2 B at 192 B per cycle; copy latency
// L = 1500 cycles.  `occ` workgroups share a compute unit (bounded by LDS and
// by a register estimate: fp32 accumulators, double-buffered operand
// fragments and 16 address registers per lane).  With S >= 2 a tile's copies
// are issued S - 1 tiles ahead (half a tile more with a_lead), so the latency
// left exposed is max(0, L - (S - 1 + lead / 2) occ max(C, X, R)); with S = 1
// copy, latency and compute add up.  Each round of occ x 256 workgroups adds
// the C store (bM bN 2 B per workgroup at 64 B per cycle) and 500 cycles.
// The rates and L were fitted to two passes of measured tuning tables of
// twelve shapes from 512x512x65536 to 16384x4096x4096 (random fp16 operands,
// every built configuration, about 3 ms of warm-up and 3 ms of timing each).
double model_cost_us(const gemm_config &c, int64_t M, int64_t N, int64_t K)
{
    const int W = c.threads / 64 > 0 ? c.threads / 64 : 4;
    const int MF = W >= 8 ? 16 : 32;
    const double TM = c.block_M / 2.0, TN = (double)c.block_N / (W / 2);
    const int S = c.num_stages < 1 ? 1 : c.num_stages;
    const double lds = (double)lds_bytes_of(c.block_M, c.block_N, c.block_K, S, c.a_lead);
    const int occ_lds = (int)(163840.0 / lds);
    const double regs = TM * TN / 64 + 2 * (TM / MF + TN / MF) * 4 + 16;
    const int waves_simd = (int)(512.0 / regs) < 8 ? (int)(512.0 / regs) : 8;
    int occ = (4 * waves_simd) / W;
    if (occ_lds < occ)
        occ = occ_lds;
    if (occ < 1)
        occ = 1;
    const double tiles = (double)tiles_of(M, N, c.block_M, c.block_N);
    const double rounds = std::ceil(tiles / (256.0 * occ));
    const double nk = (double)((K + c.block_K - 1) / c.block_K);
    const double C = 2.0 * c.block_M * c.block_N * c.block_K / 4096.0 / (MF == 16 ? 1.4 : 1.0);
    const double X = (c.block_M + c.block_N) * c.block_K * 2.0 / 48.0 * (c.block_K == 32 ? 1.5 : 1.0);
    const double R = W * (TM + TN) * c.block_K * 2.0 / 192.0;
    const double L = 1500.0;
    double tile;
    if (S == 1) {
        tile = occ * (C + X) > C + X + L ? occ * (C + X) : C + X + L;
    } else {
        double per = C > X ? C : X;
        per = (per > R ? per : R) * occ;
        const double hidden = (S - 1 + 0.5 * c.a_lead) * per;
        tile = per + (L > hidden ? L - hidden : 0.0);
    }
    const double epi = occ * c.block_M * c.block_N * 2.0 / 64.0 + 500.0;
    return rounds * (nk * tile + epi) / 2100.0;
}

// ---------------------------------------------------------------------------
// Attention.

typedef hipError_t (*attn_launch_fn)(const AttnArgs &, int grid, int lds_bytes, hipStream_t);

struct AttnInstance {
    int dtype, bn, waves, qb, dim;  // qb: 32-query blocks per wave
    int loads_per_wave;  // 1 KiB copies per wave per K/V tile pair
    attn_launch_fn launch;
};

#define PG_ATTN_ROW(DT, T, BN, W, QB, D) \
    {DT, BN, W, QB, D, 2 * BN * D * 2 / (1024 * W), &attn_launch<T, BN, W, QB, D>},
#define PG_ATTN_ROW_F16(BN, W, QB, D) PG_ATTN_ROW(GEMM_F16, _Float16, BN, W, QB, D)
#define PG_ATTN_ROW_BF16(BN, W, QB, D) PG_ATTN_ROW(GEMM_BF16, __bf16, BN, W, QB, D)
const AttnInstance kAttnInstances[] = {PG_ATTN_TILE_LIST(PG_ATTN_ROW_F16) PG_ATTN_TILE_LIST(PG_ATTN_ROW_BF16)};

int64_t attn_lds_of(int bn, int dim, int stages)
{
    return (int64_t)(stages < 1 ? 1 : stages) * 2 * bn * (int64_t)dim * 2;
}

int attn_validate(int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D, int dtype, int causal,
                  int bm, int bn, int stages, int threads, int64_t budget, const void *const *ptrs,
                  const AttnInstance **inst)
{
    // (1) arguments
    if (B < 1 || H < 1 || Hkv < 1 || Sq < 1 || Skv < 1 || D < 1)
        return fail(GEMM_ERR_ARG, "attention sizes must be >= 1");
    if (H % Hkv)
        return fail(GEMM_ERR_ARG, "heads (%lld) must be a multiple of kv_heads (%lld)", (long long)H,
                    (long long)Hkv);
    if (dtype != GEMM_F16 && dtype != GEMM_BF16)
        return fail(GEMM_ERR_ARG, "unknown dtype %d", dtype);
    if (causal != 0 && causal != 1)
        return fail(GEMM_ERR_ARG, "is_causal must be 0 or 1");
    if (causal && Sq != Skv)
        return fail(GEMM_ERR_ARG, "a causal mask needs seq_q == seq_kv");
    if (bm <= 0 || bn <= 0 || stages < 0)
        return fail(GEMM_ERR_ARG, "block sizes must be positive and num_stages >= 0");
    if (threads < 0 || threads % 64 != 0 || threads > 1024)
        return fail(GEMM_ERR_ARG, "threads must be 0 or a multiple of 64 up to 1024 (got %d)", threads);
    if (ptrs && (!ptrs[0] || !ptrs[1] || !ptrs[2] || !ptrs[3]))
        return fail(GEMM_ERR_ARG, "Q, K, V and O must not be null");
    if (budget <= 0)
        return fail(GEMM_ERR_ARG, "LDS budget must be positive");
    // (2) LDS budget: num_stages x (K tile + V tile)
    const int64_t need = attn_lds_of(bn, (int)(D > (1 << 20) ? (1 << 20) : D), stages);
    if (need > budget)
        return fail(GEMM_ERR_LDS_BUDGET,
                    "LDS budget exceeded: %d stage(s) x 2 x (%d x %lld) x 2 B = %lld B > %lld B available",
                    stages < 1 ? 1 : stages, bn, (long long)D, (long long)need, (long long)budget);
    // (3) alignment: 16-byte copies and stores of rows of D elements
    if (D % 8 != 0)
        return fail(GEMM_ERR_ALIGN, "dim must be a multiple of 8 (got %lld)", (long long)D);
    if (ptrs && ((((uintptr_t)ptrs[0]) | ((uintptr_t)ptrs[1]) | ((uintptr_t)ptrs[2]) | ((uintptr_t)ptrs[3])) & 15))
        return fail(GEMM_ERR_ALIGN, "Q, K, V and O must be 16-byte aligned");
    // (4) supported configuration and size limits
    if (D != 64 && D != 128)
        return fail(GEMM_ERR_UNSUPPORTED, "attention is built for dim 64 and 128 (got %lld)", (long long)D);
    // block_M = 32 x (query blocks per wave) x waves; threads 0 = one block per wave
    const int th = threads == 0 ? 2 * bm : threads;
    const int waves = th / 64;
    if (waves < 1 || bm % (32 * waves) != 0)
        return fail(GEMM_ERR_UNSUPPORTED,
                    "block_M must be 32 or 64 queries per wave (got block_M %d with %d threads)", bm, th);
    const int qb = bm / (32 * waves);
    const AttnInstance *in = nullptr;
    for (const AttnInstance &a : kAttnInstances)
        if (a.dtype == dtype && a.bn == bn && a.waves == waves && a.qb == qb && a.dim == D)
            in = &a;
    if (!in)
        return fail(GEMM_ERR_UNSUPPORTED, "no attention kernel built for block_M %d, block_N %d", bm, bn);
    const int s = stages < 1 ? 1 : stages;
    if (s > kAttnMaxStages || (s - 1) * in->loads_per_wave > 63 || attn_lds_of(bn, (int)D, s) > 160 * 1024)
        return fail(GEMM_ERR_UNSUPPORTED, "num_stages %d is not built for block_N %d with %d waves", s, bn,
                    th / 64);
    // the limits are checked by division (for positive x, y: x y >= lim
    // exactly when x > (lim - 1) / y), so that no product of the sizes can
    // overflow whatever the caller passes
    const int64_t lim = (int64_t)1 << 31;
    if (Sq > (lim - 1) / (D * 2) || Skv > (lim - 1) / (D * 2))
        return fail(GEMM_ERR_UNSUPPORTED, "one head's sequence must be below 2 GiB");
    const int64_t nq = Sq / bm + (Sq % bm != 0);
    if (B > (lim - 1) / H || B * H > (lim - 1) / nq)
        return fail(GEMM_ERR_UNSUPPORTED, "too many workgroups");
    if (inst)
        *inst = in;
    return ok();
}

}  // namespace
}  // namespace pipegemm

extern "C" {

int attn_fwd(const void *Q, const void *K, const void *V, void *O, int64_t batch, int64_t heads, int64_t kv_heads,
             int64_t seq_q, int64_t seq_kv, int64_t dim, int dtype, int is_causal, float scale, int block_M,
             int block_N, int num_stages, int threads, void *hip_stream)
{
    using namespace pipegemm;
    // (1) arguments: the scale is 0 (the default 1/sqrt(dim)) or a positive
    // finite number; a negative one would turn the -inf of masked scores
    // into +inf
    if (!(scale >= 0.0f) || !std::isfinite(scale))
        return fail(GEMM_ERR_ARG, "scale must be 0 (1/sqrt(dim)) or positive and finite (got %g)", (double)scale);
    const void *ptrs[4] = {Q, K, V, O};
    int st = attn_validate(batch, heads, kv_heads, seq_q, seq_kv, dim, dtype, is_causal, block_M, block_N,
                           num_stages, threads, 1LL << 40, ptrs, nullptr);
    if (st == GEMM_ERR_ARG)
        return st;
    int64_t budget = 0;
    st = device_budget(&budget);
    if (st != GEMM_OK)
        return st;
    const AttnInstance *in = nullptr;
    st = attn_validate(batch, heads, kv_heads, seq_q, seq_kv, dim, dtype, is_causal, block_M, block_N, num_stages,
                       threads, budget, ptrs, &in);
    if (st != GEMM_OK)
        return st;
    AttnArgs a{};
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.O = O;
    a.B = (int)batch;
    a.H = (int)heads;
    a.Hkv = (int)kv_heads;
    a.Sq = (int)seq_q;
    a.Skv = (int)seq_kv;
    a.groups = (int)(heads / kv_heads);
    a.causal = is_causal;
    const float sc = scale == 0.0f ? 1.0f / sqrtf((float)dim) : scale;
    a.scale_log2 = sc * 1.4426950408889634f;  // log2(e)
    a.stages = num_stages < 1 ? 1 : num_stages;
    a.nq = (int)((seq_q + block_M - 1) / block_M);
    const int grid = (int)(batch * heads * a.nq);
    hipError_t e = in->launch(a, grid, (int)attn_lds_of(block_N, (int)dim, a.stages), (hipStream_t)hip_stream);
    if (e != hipSuccess)
        return fail(GEMM_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
    return ok();
}

int64_t attn_lds_bytes(int block_N, int dim, int num_stages)
{
    if (block_N < 0 || dim < 0 || num_stages < 0)
        return -1;
    return pipegemm::attn_lds_of(block_N, dim, num_stages);
}

int attn_default_config(int64_t batch, int64_t heads, int64_t seq_q, int64_t dim, int is_causal, int *block_M,
                        int *block_N, int *num_stages, int *threads)
{
    using namespace pipegemm;
    if (!block_M || !block_N || !num_stages || !threads)
        return fail(GEMM_ERR_ARG, "block_M, block_N, num_stages and threads must not be null");
    if (batch < 1 || heads < 1 || seq_q < 1)
        return fail(GEMM_ERR_ARG, "attention sizes must be >= 1");
    if (is_causal != 0 && is_causal != 1)
        return fail(GEMM_ERR_ARG, "is_causal must be 0 or 1");
    if (dim != 64 && dim != 128)
        return fail(GEMM_ERR_UNSUPPORTED, "attention is built for dim 64 and 128 (got %lld)", (long long)dim);
    // the 8-wave tiles, unless the grid would leave compute units idle
    int bm = 256, bn = 128, s = 2, th = 512;
    if (dim == 64)
        bm = 512;
    const int64_t nq = seq_q / bm + (seq_q % bm != 0);
    const bool small = batch < 256 && heads < 256 && nq < 256 && batch * heads * nq < 256;
    if ((dim == 64 && is_causal) || small) {
        bm = 128;
        bn = 64;
        th = 256;
    }
    *block_M = bm;
    *block_N = bn;
    *num_stages = s;
    *threads = th;
    return ok();
}

int attn_check(int64_t batch, int64_t heads, int64_t kv_heads, int64_t seq_q, int64_t seq_kv, int64_t dim, int dtype,
               int is_causal, int block_M, int block_N, int num_stages, int threads, int64_t lds_budget)
{
    int64_t budget = lds_budget;
    if (budget == 0) {
        const int st = pipegemm::device_budget(&budget);
        if (st != GEMM_OK)
            return st;
    }
    return pipegemm::attn_validate(batch, heads, kv_heads, seq_q, seq_kv, dim, dtype, is_causal, block_M, block_N,
                                   num_stages, threads, budget, nullptr, nullptr);
}

int gemm_configs(int layout, int dtype, gemm_config *out, int max)
{
    if ((layout != GEMM_NT && layout != GEMM_NN) || (dtype != GEMM_F16 && dtype != GEMM_BF16) || max < 0 ||
        (out == nullptr && max > 0))
        return pipegemm::fail(GEMM_ERR_ARG, "gemm_configs: bad layout, dtype or output array"), -1;
    pipegemm::ok();
    return pipegemm::enumerate_configs(layout, dtype, out, max);
}

int gemm_prune(int layout, int64_t M, int64_t N, int64_t K, int dtype, const gemm_config *cands, int n,
               int64_t lds_budget, int *status)
{
    if (n < 0 || (n > 0 && (cands == nullptr || status == nullptr)))
        return pipegemm::fail(GEMM_ERR_ARG, "gemm_prune: bad candidate array"), -1;
    int64_t budget = lds_budget;
    if (budget == 0 && pipegemm::device_budget(&budget) != GEMM_OK)
        return -1;
    int legal = 0;
    for (int i = 0; i < n; ++i) {
        const gemm_config &c = cands[i];
        // first: tiles that do not divide the problem
        if (c.block_M <= 0 || c.block_N <= 0 || c.block_K <= 0) {
            status[i] = GEMM_ERR_ARG;
            continue;
        }
        if (M % c.block_M || N % c.block_N || K % c.block_K) {
            status[i] = GEMM_PRUNE_NODIV;
            continue;
        }
        // then: the launch-time validation (budget first, then the rest)
        status[i] = pipegemm::validate(layout, M, N, K, dtype, c.block_M, c.block_N, c.block_K, c.num_stages,
                                       c.a_lead, c.threads, budget, nullptr, nullptr);
        legal += status[i] == GEMM_OK;
    }
    pipegemm::ok();
    return legal;
}

int gemm_rank(int64_t M, int64_t N, int64_t K, const gemm_config *cands, int n, double *cost)
{
    if (M < 0 || N < 0 || K < 0 || n < 0 || (n > 0 && (cands == nullptr || cost == nullptr)))
        return pipegemm::fail(GEMM_ERR_ARG, "gemm_rank: bad arguments");
    for (int i = 0; i < n; ++i) {
        const gemm_config &c = cands[i];
        if (c.block_M <= 0 || c.block_N <= 0 || c.block_K <= 0 || c.threads < 0 || c.threads % 128 != 0 ||
            c.num_stages < 0 || (c.a_lead != 0 && c.a_lead != 1))
            return pipegemm::fail(GEMM_ERR_ARG, "gemm_rank: candidate %d is malformed", i);
        cost[i] = pipegemm::model_cost_us(c, M, N, K);
    }
    return pipegemm::ok();
}

int gemm_tune(int layout, const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int dtype,
              const gemm_config *cands, const int *status, int n, int warmup, int reps, void *hip_stream, float *ms,
              int *best)
{
    if (n < 0 || (n > 0 && (cands == nullptr || status == nullptr || ms == nullptr)) || best == nullptr ||
        warmup < 0 || reps < 1)
        return pipegemm::fail(GEMM_ERR_ARG, "gemm_tune: bad arguments");
    *best = -1;
    hipStream_t stream = (hipStream_t)hip_stream;
    hipEvent_t t0 = nullptr, t1 = nullptr;
    hipError_t e = hipEventCreate(&t0);
    if (e == hipSuccess)
        e = hipEventCreate(&t1);
    if (e != hipSuccess) {
        if (t0)
            (void)hipEventDestroy(t0);
        return pipegemm::fail(GEMM_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e));
    }
    int st = GEMM_OK;
    float best_ms = 0.f;
    for (int i = 0; i < n && st == GEMM_OK; ++i) {
        ms[i] = -1.f;
        if (status[i] != GEMM_OK)
            continue;
        const gemm_config &c = cands[i];
        auto launch = [&] {
            return pipegemm::run(layout, A, B, C, M, N, K, dtype, c.block_M, c.block_N, c.block_K, c.num_stages,
                                 c.a_lead, c.threads, hip_stream);
        };
        for (int w = 0; w < warmup && st == GEMM_OK; ++w)
            st = launch();
        if (st == GEMM_OK && (e = hipEventRecord(t0, stream)) != hipSuccess)
            st = pipegemm::fail(GEMM_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
        for (int r = 0; r < reps && st == GEMM_OK; ++r)
            st = launch();
        if (st == GEMM_OK && (e = hipEventRecord(t1, stream)) != hipSuccess)
            st = pipegemm::fail(GEMM_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
        if (st == GEMM_OK && (e = hipEventSynchronize(t1)) != hipSuccess)
            st = pipegemm::fail(GEMM_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(e));
        float t = 0.f;
        if (st == GEMM_OK && (e = hipEventElapsedTime(&t, t0, t1)) != hipSuccess)
            st = pipegemm::fail(GEMM_ERR_HIP, "hipEventElapsedTime: %s", hipGetErrorString(e));
        if (st != GEMM_OK)
            break;
        ms[i] = t / reps;
        if (*best < 0 || ms[i] < best_ms) {
            *best = i;
            best_ms = ms[i];
        }
    }
    (void)hipEventDestroy(t0);
    (void)hipEventDestroy(t1);
    if (st == GEMM_OK)
        pipegemm::ok();
    return st;
}

int gemm_default_config(int layout, int64_t M, int64_t N, int64_t K, int dtype, gemm_config *out)
{
    if ((layout != GEMM_NT && layout != GEMM_NN) || (dtype != GEMM_F16 && dtype != GEMM_BF16) || M < 0 || N < 0 ||
        K < 0 || out == nullptr)
        return pipegemm::fail(GEMM_ERR_ARG, "gemm_default_config: bad arguments");
    // One configuration per tile, each with the ring and wave count measured
    // best for it on gfx950 (tuning tables of twelve shapes, 512 x 512 x 65536
    // to 16384 x 4096 x 4096, random fp16, every built configuration); the
    // analytic cost model (gemm_rank) picks among them, so the choice accounts
    // for how many rounds of workgroups each grid takes on the 256 compute
    // units (a grid just above 256 tiles leaves the second round nearly
    // empty).  On those tables the pick is the measured best or within 2.4 %
    // of it.  Ties keep the earlier, larger tile.
    static const gemm_config kTable[] = {
        {256, 256, 64, 2, 1, 512},
        {256, 128, 64, 3, 0, 256},
        {128, 256, 64, 3, 0, 512},
        {128, 128, 64, 3, 0, 512},
        {64, 128, 64, 4, 0, 256},
    };
    const gemm_config *pick = &kTable[0];
    double best = pipegemm::model_cost_us(kTable[0], M, N, K);
    for (const gemm_config &c : kTable) {
        const double cost = pipegemm::model_cost_us(c, M, N, K);
        if (cost < best) {
            best = cost;
            pick = &c;
        }
    }
    *out = *pick;
    return pipegemm::ok();
}

int gemm_nt(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int dtype, int block_M,
            int block_N, int block_K, int num_stages, int a_lead, int threads, void *hip_stream)
{
    return pipegemm::run(GEMM_NT, A, B, C, M, N, K, dtype, block_M, block_N, block_K, num_stages, a_lead, threads,
                         hip_stream);
}

int gemm_nn(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int dtype, int block_M,
            int block_N, int block_K, int num_stages, int a_lead, int threads, void *hip_stream)
{
    return pipegemm::run(GEMM_NN, A, B, C, M, N, K, dtype, block_M, block_N, block_K, num_stages, a_lead, threads,
                         hip_stream);
}

int gemm_nt_relu(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int dtype, int block_M,
                 int block_N, int block_K, int num_stages, int a_lead, int threads, void *hip_stream)
{
    return pipegemm::run(GEMM_NT, A, B, C, M, N, K, dtype, block_M, block_N, block_K, num_stages, a_lead, threads,
                         hip_stream, 1);
}

int gemm_nn_relu(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int dtype, int block_M,
                 int block_N, int block_K, int num_stages, int a_lead, int threads, void *hip_stream)
{
    return pipegemm::run(GEMM_NN, A, B, C, M, N, K, dtype, block_M, block_N, block_K, num_stages, a_lead, threads,
                         hip_stream, 1);
}

int gemm_stamped(int layout, const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int dtype,
                 int block_M, int block_N, int block_K, int num_stages, int a_lead, int threads, void *hip_stream,
                 uint64_t *stamps)
{
    // an argument error, so it is reported before the budget as the
    // validation order requires
    if (stamps == nullptr || (((uintptr_t)stamps) & 7))
        return pipegemm::fail(GEMM_ERR_ARG, "gemm_stamped: stamps must be a non-null 8-byte aligned pointer");
    return pipegemm::run(layout, A, B, C, M, N, K, dtype, block_M, block_N, block_K, num_stages, a_lead, threads,
                         hip_stream, 0, (unsigned long long *)stamps);
}

int64_t gemm_lds_bytes(int block_M, int block_N, int block_K, int num_stages, int a_lead, int dtype)
{
    if (block_M < 0 || block_N < 0 || block_K < 0 || num_stages < 0 || (a_lead != 0 && a_lead != 1) ||
        (dtype != GEMM_F16 && dtype != GEMM_BF16))
        return -1;
    return pipegemm::lds_bytes_of(block_M, block_N, block_K, num_stages, a_lead);
}

int64_t gemm_lds_budget(void)
{
    int64_t b = 0;
    if (pipegemm::device_budget(&b) != GEMM_OK)
        return -1;
    return b;
}

int gemm_check(int layout, int64_t M, int64_t N, int64_t K, int dtype, int block_M, int block_N, int block_K,
               int num_stages, int a_lead, int threads, int64_t lds_budget)
{
    int64_t budget = lds_budget;
    if (budget == 0) {
        const int st = pipegemm::device_budget(&budget);
        if (st != GEMM_OK)
            return st;
    }
    return pipegemm::validate(layout, M, N, K, dtype, block_M, block_N, block_K, num_stages, a_lead, threads,
                              budget, nullptr, nullptr);
}

const char *gemm_last_error(void)
{
    return pipegemm::g_err;
}

}  // extern "C"
