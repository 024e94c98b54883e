// Device code of the software-pipelined tiled GEMM (gfx950 / MI355X).
//
// One workgroup owns a BM x BN tile of C.  Its K loop streams BM x BK tiles of
// A and BN x BK (NT) or BK x BN (NN) tiles of B from HBM into a ring of S LDS
// slots with direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds), and
// feeds the matrix cores from the slot that has landed:
//
//   prologue      issue tiles 0 .. min(S-1, nk)-1 into slots 0 ..
//   steady state  for kt:  wait until this wave's copies of tile kt landed
//                          barrier   (every wave's copies of kt landed, and every
//                                     wave finished computing kt-1, so slot
//                                     (kt-1) mod S is free)
//                          issue tile kt+S-1 into slot (kt+S-1) mod S
//                          MFMA over slot kt mod S
//   drain         the last S-1 iterations issue nothing
//   S = 1         issue, wait, barrier, compute, barrier (two barriers per
//                 round: copy and compute never overlap)
//
// This is the structure of the TileLang tutorial, chapter 11: section 1.1
// (single buffer: every round costs copy + compute), section 2.3 (S versioned
// buffers indexed by ko mod S), section 4.3 (prologue / body / epilogue with
// max_stage = S - 1) and section 5.2 (write slot s only after its last reader
// is done; read slot s only after its writer is done).
//
// Hardware mapping (gfx950):
//  - copies: each wave issues 1 KiB direct-to-LDS loads (64 lanes x 16 B);
//    lane i of a load lands at LDS base + 16 i, so the bank swizzle is applied
//    by choosing which global 16-byte chunk each lane fetches;
//  - the copy wait is s_waitcnt vmcnt(n), n = loads still allowed in flight
//    (the copies of the tiles issued after kt); vmcnt counts in issue order;
//  - compute: v_mfma_f32_16x16x32_{f16,bf16} (4 fp32 accumulators per lane
//    per 16x16 block) or v_mfma_f32_32x32x16_{f16,bf16} (16 per 32x32 block),
//    operands read from LDS with ds_read_b128 (k-contiguous tiles) or
//    ds_read_b64_tr_b16 (the N-contiguous B tile of the NN form).  The two
//    shapes run at the same nominal rate, but with random operands the 16x16
//    one draws less power per flop (half the accumulator traffic per flop),
//    so the power-limited clock stays higher;
//  - the MFMA is fed the B fragment as its first operand and the A fragment as
//    its second, so it produces C^T blocks: each lane then holds 4 consecutive
//    columns of one row of C;
//  - out-of-range rows and K/N chunks read as zero through the buffer
//    resource's range check (an offset at or beyond num_records returns 0);
//  - 8-wave 256 x 256 tiles put two waves on each SIMD; a wave lowers its
//    priority (s_setprio) only for the stretch that ends in the wait for the
//    next tile, so its SIMD partner keeps the matrix core busy meanwhile;
//  - C leaves through an LDS strip per wave as 16-byte streaming stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "pipegemm_layout.hpp"

namespace pipegemm {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Cache-policy bits of a gfx950 vector memory instruction: sc0 (bit 0), nt
// (bit 1), sc1 (bit 4).
constexpr int kStoreNtSc1 = (1 << 1) | (1 << 4);

typedef __attribute__((address_space(3))) void lds_void;

// Kernel parameters, passed by value.
struct KernelArgs {
    const void *A;
    const void *B;
    void *C;
    int M, N, K;
    int nk;       // number of K tiles, ceil(K / BK)
    int stages;   // LDS ring slots of the B tile, >= 1
    int a_lead;   // 1: the A tile runs one K tile further ahead in S + 1 slots (S >= 2)
    int tiles_m;  // ceil(M / BM)
    int tiles_n;  // ceil(N / BN)
    int group_m;  // tile rows swept before advancing along N (L2 reuse)
    int c_vec;    // 1 when C rows allow 16-byte stores (N % 8 == 0, C 16-byte aligned)
    int relu;     // 1: C = relu(A.B), the fp32 sum s replaced by (s > 0 ? s : +0) before rounding
    // null, or 6 counters per workgroup (stamp_index): shader-clock cycles at
    // start, after the prologue, after the K loop and at the end, then the
    // 100 MHz real-time counter at start and end
    unsigned long long *stamps;
};

// ---------------------------------------------------------------------------
// Element types.
template <class T>
struct Elem;

template <>
struct Elem<_Float16> {
    typedef f16x8 frag;
    typedef f16x4 quad;
    static __device__ __forceinline__ f32x16 mfma(frag a, frag b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Elem<__bf16> {
    typedef bf16x8 frag;
    typedef bf16x4 quad;
    static __device__ __forceinline__ f32x16 mfma(frag a, frag b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

// The GEMM's MFMA per block shape MF (32: 32x32x16, 16: 16x16x32), fed
// (B fragment, A fragment, accumulator).
template <class T, int MF>
struct Mfma;

template <>
struct Mfma<_Float16, 32> {
    typedef f32x16 acc;
    static __device__ __forceinline__ acc run(f16x8 b, f16x8 a, acc c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c, 0, 0, 0);
    }
};

template <>
struct Mfma<_Float16, 16> {
    typedef f32x4 acc;
    static __device__ __forceinline__ acc run(f16x8 b, f16x8 a, acc c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(b, a, c, 0, 0, 0);
    }
};

template <>
struct Mfma<__bf16, 32> {
    typedef f32x16 acc;
    static __device__ __forceinline__ acc run(bf16x8 b, bf16x8 a, acc c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c, 0, 0, 0);
    }
};

template <>
struct Mfma<__bf16, 16> {
    typedef f32x4 acc;
    static __device__ __forceinline__ acc run(bf16x8 b, bf16x8 a, acc c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, a, c, 0, 0, 0);
    }
};

// ---------------------------------------------------------------------------
// Tile geometry.  WM x WN waves; each wave owns a TM x TN sub-tile of C made
// of FM x FN blocks of MF x MF (the MFMA shape).
//
// The shape follows the waves per SIMD.  With 8 waves (two per SIMD, at most
// 256 registers each) the accumulators live in VGPRs and the 16x16x32 MFMA
// runs without overhead, so it is used for its lower power.  With 4 waves
// (one per SIMD) the accumulators go to AGPRs, where the compiler keeps
// 16x16x32 accumulators only by copying them inside the K loop (hundreds of
// v_accvgpr moves per tile); 32x32x16 accumulators stay in place.
template <int WAVES>
constexpr int default_mfma() { return WAVES >= 8 ? 16 : 32; }

template <int BM_, int BN_, int BK_, int WM_, int WN_, int MF_ = default_mfma<WM_ * WN_>()>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, MF = MF_;
    static constexpr int WAVES = WM * WN;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / MF, FN = TN / MF;
    static constexpr int KPS = 512 / MF;               // k per MFMA: 16 (32x32) or 32 (16x16)
    static constexpr int KSTEPS = BK / KPS;            // MFMA k-steps per tile
    static constexpr int A_BYTES = BM * BK * 2;
    static constexpr int B_BYTES = BN * BK * 2;
    static constexpr int SLOT_BYTES = A_BYTES + B_BYTES;
    static constexpr int A_LOADS = A_BYTES / (1024 * WAVES);  // 1 KiB loads per wave per tile
    static constexpr int B_LOADS = B_BYTES / (1024 * WAVES);
    static constexpr int LOADS = A_LOADS + B_LOADS;
    static_assert(BM % WM == 0 && BN % WN == 0, "waves must split the tile");
    static_assert(MF == 16 || MF == 32, "MFMA blocks are 16x16 or 32x32");
    static_assert(TM % MF == 0 && TN % MF == 0, "wave sub-tiles are made of MFMA blocks");
    static_assert(BK == 32 || BK == 64, "block_K must be 32 or 64");
    static_assert(A_BYTES % (1024 * WAVES) == 0 && B_BYTES % (1024 * WAVES) == 0,
                  "each wave must copy a whole number of 1 KiB pieces of each tile");
    static_assert(LOADS >= 1, "at least one copy per wave");
    static_assert(BN >= 128, "the N-contiguous B tile swizzle needs 16 chunks per row");
};

// ---------------------------------------------------------------------------
// Small device helpers.

// s_waitcnt vmcnt(n) with every other counter left free (gfx9 encoding:
// vmcnt[3:0] bits 3:0, vmcnt[5:4] bits 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most `tiles` tiles' worth of this wave's copies are in flight.
template <int LOADS>
__device__ __forceinline__ void wait_tiles(int tiles)
{
    switch (tiles) {
#define PG_WAIT_CASE(i) \
    case i:             \
        if constexpr (i * LOADS <= 63) wait_vmcnt<i * LOADS>(); else wait_vmcnt<0>(); \
        break;
        PG_WAIT_CASE(1) PG_WAIT_CASE(2) PG_WAIT_CASE(3) PG_WAIT_CASE(4)
        PG_WAIT_CASE(5) PG_WAIT_CASE(6) PG_WAIT_CASE(7) PG_WAIT_CASE(8)
#undef PG_WAIT_CASE
    default:
        wait_vmcnt<0>();
        break;
    }
}

// s_waitcnt lgkmcnt(0): every LDS read this wave issued has returned.
__device__ __forceinline__ void wait_lds()
{
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

// Workgroup barrier.  Every LDS read this wave issued before it has returned
// when it is passed (so a slot it read may be overwritten afterwards), and the
// compiler may not move memory accesses across it.
__device__ __forceinline__ void barrier()
{
    asm volatile("" ::: "memory");
    wait_lds();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One 16-byte-per-lane direct-to-LDS load: lane i's chunk lands at dst + 16 i.
__device__ __forceinline__ void copy_1k(__amdgpu_buffer_rsrc_t rsrc, char *dst, uint32_t voffset)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void *)dst, 16, voffset, 0, 0, 0);
}

// An offset that is out of range for every buffer resource this kernel builds
// (their num_records are all below 2^31), so the load returns zero.
constexpr uint32_t kOOB = 0x80000000u;

// Calls f(std::integral_constant<int, i>()) for i = 0 .. N-1, so the body can
// use i in constant expressions (template arguments of scheduling hints).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>()), ...);
}

template <int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>());
}

// Scheduling hint for one stretch of NM MFMAs: LDS reads (NR) go out as early
// as possible, RPM per MFMA, and global loads (NL) are spread evenly after
// them, so both issue while the matrix core is busy.  RPM is 2 for the
// 32-cycle 32x32x16 MFMA and 1 for the 16-cycle 16x16x32 one: one 1 KiB read
// per 16 cycles per wave is what the LDS command queue sustains with two waves
// per SIMD (twice that rate fills it and stalls the issuing wave).
template <int NM, int NR, int NL, int RPM, int... I>
__device__ __forceinline__ void interleave_impl(std::integer_sequence<int, I...>)
{
    ((__builtin_amdgcn_sched_group_barrier(0x008, 1, 0),
      (RPM * I < NR ? __builtin_amdgcn_sched_group_barrier(0x100, (NR - RPM * I) < RPM ? (NR - RPM * I) : RPM, 0)
                    : (void)0),
      ((I + 1) * NL / NM - I * NL / NM > 0
           ? __builtin_amdgcn_sched_group_barrier(0x020, (I + 1) * NL / NM - I * NL / NM, 0)
           : (void)0)),
     ...);
}

template <int NM, int NR, int NL, int RPM = 2>
__device__ __forceinline__ void interleave()
{
    interleave_impl<NM, NR, NL, RPM>(std::make_integer_sequence<int, NM>());
}

// ---------------------------------------------------------------------------
// NN form: MFMA operand from the N-contiguous B tile, two transposed reads
// (see nn_tr_offset for the lane mapping).
//
// The reads are issued through inline assembly: for the ds_read_tr builtin the
// compiler's wait insertion adds s_waitcnt vmcnt(0) before every read (it
// cannot tell the read from the in-flight direct-to-LDS copies), which would
// wait for every copy of the ring at every k-step.  The kernel orders copies
// and reads itself (vmcnt waits and barriers); sync_nn_operands() supplies the
// one thing the compiler no longer sees, the wait for the reads' data.
__device__ __forceinline__ i16x4 ds_read_tr16_b64(const char *addr)
{
    i16x4 v;
    const uint32_t lds_addr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)addr;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(lds_addr) : "memory");
    return v;
}

// `slot` is the B tile's slot.
template <class T, class Cfg>
__device__ __forceinline__ typename Elem<T>::frag load_b_nn(const char *slot, int kk, int ncol0, int lane)
{
    i16x8 out;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int off = Cfg::MF == 32 ? nn_tr_offset<Cfg::BN>(lane, kk, ncol0, h)
                                      : nn_tr_offset16<Cfg::BN>(lane, kk, ncol0, h);
        const i16x4 v = ds_read_tr16_b64(slot + off);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            out[4 * h + e] = v[e];
    }
    return __builtin_bit_cast(typename Elem<T>::frag, out);
}

// Wait for every LDS read this wave issued (including the transposed reads
// the compiler does not track) and make the B fragments depend on that wait,
// so no MFMA reading them can be scheduled before it.
template <class Frag, int FN>
__device__ __forceinline__ void sync_nn_operands(Frag (&fb)[FN])
{
    // the builtin (not inline assembly), so the compiler's own wait
    // bookkeeping also knows every earlier LDS read has completed
    wait_lds();
#pragma unroll
    for (int g = 0; g < FN; ++g)
        asm volatile("" : "+v"(fb[g]));
}

// ---------------------------------------------------------------------------
// The kernel.
// KCHECK: K is not a multiple of BK, so the last K tile is ragged.
template <class T, bool NN, class Cfg, bool KCHECK>
__global__ __launch_bounds__(Cfg::THREADS, 1) void gemm_kernel(const KernelArgs p)
{
    using E = Elem<T>;
    using frag = typename E::frag;
    using MM = Mfma<T, Cfg::MF>;
    using accv = typename MM::acc;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, MF = Cfg::MF;
    constexpr int WAVES = Cfg::WAVES, FM = Cfg::FM, FN = Cfg::FN;
    constexpr int NACC = MF == 32 ? 16 : 4;  // accumulators per lane per block

    extern __shared__ __attribute__((aligned(1024))) char smem[];
    // clock stamps (scalar reads of the cycle and real-time counters; written
    // out at the end only when p.stamps is set)
    const unsigned long long st_c0 = __builtin_amdgcn_s_memtime(), st_t0 = __builtin_amdgcn_s_memrealtime();
    unsigned long long st_c1 = 0, st_c2 = 0;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % Cfg::WM, wn = wave / Cfg::WM;

    int tm, tn;
    map_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int K = p.K, N = p.N, nk = p.nk;

    // The A panel (rows m0..) and the B panel (rows n0.. of the NT form, columns
    // n0.. of the NN form), as byte ranges.  Each K tile is copied through a
    // buffer resource of its panel shifted to the tile's first K position: a
    // resource is four scalar registers, so the shift costs a few scalar
    // instructions per tile and every lane's offset is the same in every tile.
    // Bytes at or beyond the end of the panel read as zero, so in the NN form
    // rows of B past K, and tiles past the end of K, land as zeros.  In the
    // K-contiguous tiles a chunk past K in the ragged last tile would read the
    // next row instead: with KCHECK those chunks get an out-of-range offset.
    const int a_rows = min(BM, p.M - m0);
    const char *const a_panel = (const char *)p.A + (size_t)m0 * K * 2;
    const int a_bytes = a_rows * K * 2;
    const char *b_panel;
    int b_bytes;
    if constexpr (!NN) {
        b_panel = (const char *)p.B + (size_t)n0 * K * 2;
        b_bytes = min(BN, N - n0) * K * 2;
    } else {
        b_panel = (const char *)p.B + (size_t)n0 * 2;
        b_bytes = (K * N - n0) * 2;
    }
    auto tile_rsrc = [](const char *panel, int bytes, int64_t shift) {
        const int64_t left = (int64_t)bytes - shift;
        return __builtin_amdgcn_make_buffer_rsrc((void *)(panel + shift), 0, left > 0 ? (int)left : 0, 0x00020000);
    };

    // Per-lane source offsets of this wave's copies within a tile and the K
    // position of each chunk within a tile (for the K bound).
    uint32_t a_off[Cfg::A_LOADS];
    int a_kc[Cfg::A_LOADS];
#pragma unroll
    for (int t = 0; t < Cfg::A_LOADS; ++t) {
        int r, c;
        k_tile_unit<BK, MF>((t * WAVES + wave) * 64 + lane, r, c);
        a_off[t] = (uint32_t)(r * K * 2 + c * 16);
        a_kc[t] = c * 8;
    }
    uint32_t b_off[Cfg::B_LOADS];
    int b_kc[Cfg::B_LOADS];
#pragma unroll
    for (int t = 0; t < Cfg::B_LOADS; ++t) {
        const int u = (t * WAVES + wave) * 64 + lane;
        if constexpr (!NN) {
            int r, c;
            k_tile_unit<BK, MF>(u, r, c);
            b_off[t] = (uint32_t)(r * K * 2 + c * 16);
            b_kc[t] = c * 8;
        } else {
            int k, c;
            n_tile_unit<BN>(u, k, c);
            b_off[t] = (n0 + c * 8 < N) ? (uint32_t)(k * N * 2 + c * 16) : kOOB;
            b_kc[t] = 0;
        }
    }

    // Issue this wave's copies [first, last) of the A tile (B tile) of K tile
    // kt into the slot at `dst`.
    auto issue_a = [&](int kt, char *dst, int first, int last) {
        const int kbase = kt * BK;
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(a_panel, a_bytes, (int64_t)kbase * 2);
#pragma unroll
        for (int t = 0; t < Cfg::A_LOADS; ++t) {
            if (t < first || t >= last)
                continue;
            uint32_t off = a_off[t];
            if constexpr (KCHECK)
                off = kbase + a_kc[t] < K ? off : kOOB;
            copy_1k(rs, dst + (t * WAVES + wave) * 1024, off);
        }
    };
    auto issue_b = [&](int kt, char *dst, int first, int last) {
        const int kbase = kt * BK;
        const __amdgpu_buffer_rsrc_t rs =
            tile_rsrc(b_panel, b_bytes, NN ? (int64_t)kbase * N * 2 : (int64_t)kbase * 2);
#pragma unroll
        for (int t = 0; t < Cfg::B_LOADS; ++t) {
            if (t < first || t >= last)
                continue;
            uint32_t off = b_off[t];
            if constexpr (KCHECK && !NN)
                off = kbase + b_kc[t] < K ? off : kOOB;
            copy_1k(rs, dst + (t * WAVES + wave) * 1024, off);
        }
    };

    // Per-lane LDS read offsets of the MFMA operands, per k-step: lane l reads
    // row l mod MF of a block, chunk (KPS / 8) kk + l / MF.
    const int lr = lane % MF, lh = lane / MF;
    int a_rd[Cfg::KSTEPS], b_rd[Cfg::KSTEPS];
#pragma unroll
    for (int kk = 0; kk < Cfg::KSTEPS; ++kk) {
        // kswz is periodic in 16 rows, so the f-th / g-th block adds f * MF * BK * 2
        a_rd[kk] = k_tile_offset<BK, MF>(wm * Cfg::TM + lr, (Cfg::KPS / 8) * kk + lh);
        if constexpr (!NN)
            b_rd[kk] = k_tile_offset<BK, MF>(wn * Cfg::TN + lr, (Cfg::KPS / 8) * kk + lh);
        else
            b_rd[kk] = 0;
    }

    accv acc[FM][FN];
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int g = 0; g < FN; ++g)
#pragma unroll
            for (int v = 0; v < NACC; ++v)
                acc[f][g][v] = 0.0f;

    // MFMA operands, double-buffered: k-step kk computes from buffer kk & 1
    // while the reads of k-step kk+1 fill the other one.
    frag fa[2][FM], fb[2][FN];
    auto read_operands = [&](const char *as, const char *bs, int kk, int buf) {
#pragma unroll
        for (int f = 0; f < FM; ++f)
            fa[buf][f] = *(const frag *)(as + a_rd[kk] + f * MF * BK * 2);
#pragma unroll
        for (int g = 0; g < FN; ++g) {
            if constexpr (!NN)
                fb[buf][g] = *(const frag *)(bs + b_rd[kk] + g * MF * BK * 2);
            else
                fb[buf][g] = load_b_nn<T, Cfg>(bs, kk, wn * Cfg::TN + g * MF, lane);
        }
    };
    // NN form: the operands in buffer `buf` have arrived before any MFMA uses
    // them (called before the next k-step's reads are issued, so those stay
    // in flight).
    auto sync_operands = [&](int buf) {
        if constexpr (NN)
            sync_nn_operands(fb[buf]);
    };
    // MFMAs [first, last) of one k-step, in row-major block order.
    auto mfmas = [&](int buf, int first, int last) {
#pragma unroll
        for (int i = 0; i < FM * FN; ++i)
            if (i >= first && i < last)
                acc[i / FN][i % FN] = MM::run(fb[buf][i % FN], fa[buf][i / FN], acc[i / FN][i % FN]);
    };
    // One operand fragment j (A fragments first, then B; an NN B fragment is
    // two transposed reads) of k-step kk into buffer buf.
    auto read_one = [&](const char *as_, const char *bs_, auto kk_c, int buf, auto j_c) __attribute__((always_inline)) {
        constexpr int kk = decltype(kk_c)::value, j = decltype(j_c)::value;
        if constexpr (j < FM)
            fa[buf][j] = *(const frag *)(as_ + a_rd[kk] + j * MF * BK * 2);
        else if constexpr (!NN)
            fb[buf][j - FM] = *(const frag *)(bs_ + b_rd[kk] + (j - FM) * MF * BK * 2);
        else
            fb[buf][j - FM] = load_b_nn<T, Cfg>(bs_, kk, wn * Cfg::TN + (j - FM) * MF, lane);
    };
    // MFMAs [M0, M0 + NM) of buffer buf in an explicit issue order: after the
    // i-th MFMA the i-th of NR operand reads (rd), and the NC copies (cp)
    // spread evenly after the reads; a scheduling barrier after every MFMA
    // keeps that order.
    auto stretch = [&](auto nm_c, auto m0_c, int buf, auto nr_c, auto rd, auto nc_c, auto cp) __attribute__((always_inline)) {
        constexpr int NM = decltype(nm_c)::value, M0 = decltype(m0_c)::value;
        constexpr int NR = decltype(nr_c)::value, NC = decltype(nc_c)::value;
        constexpr int R0 = NR < NM ? NR : 0;
        static_for<NM>([&](auto i_c) __attribute__((always_inline)) {
            constexpr int i = decltype(i_c)::value;
            mfmas(buf, M0 + i, M0 + i + 1);
            if constexpr (i < NR)
                rd(i_c);
            static_for<NC>([&](auto c_c) __attribute__((always_inline)) {
                constexpr int c = decltype(c_c)::value;
                if constexpr (R0 + c * (NM - R0) / NC == i)
                    cp(c_c);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    constexpr int kMfma = FM * FN;
    constexpr int kRpm = MF == 32 ? 2 : 1;  // LDS reads issued per MFMA
    constexpr int kReads = FM + FN * (NN ? 2 : 1);
    constexpr int kLast = Cfg::KSTEPS - 1;

    constexpr int kLA = Cfg::A_LOADS, kLB = Cfg::B_LOADS, kS = Cfg::KSTEPS;
    // Wave priority in the steady loop (two waves share each SIMD): a wave
    // runs at priority 1 from the barrier until its last k-step, and drops to
    // 0 for that k-step's first half, where it waits for the next tile; the
    // other wave of the SIMD, still in its MFMA stretch, then gets the issue
    // slots.  Measured on the 8-wave 256 x 256 tiles (4096^3, 84.7 -> 77.6 us
    // with zero operands at 256 x 256 x 64), and with random operands on the
    // 8-wave 128 x 256 x 64 tile: +1.5 % at S = 3 (NT), and +11 % (NT) and
    // +15 % (NN) at S = 2 with a_lead, where it also brings the early B
    // copies (ring_early_b); the 256 x 128 x 32 tile is unchanged.  No gain
    // on the 128 x 128 ones.
    constexpr bool kPrio = Cfg::WAVES == 8 && Cfg::BM * Cfg::BN >= 128 * 256;
    auto set_prio = [](auto level_c) __attribute__((always_inline)) {
        if constexpr (kPrio)
            __builtin_amdgcn_s_setprio(decltype(level_c)::value);
    };

    // The K loop for a B ring of S slots and an A ring of S + LEAD slots
    // (A slots first in LDS, then B slots); S and LEAD are compile-time
    // constants inside, so every wait count is an immediate.
    auto pipeline = [&](auto stages_c, auto lead_c) {
        constexpr int S = decltype(stages_c)::value;
        constexpr int LEAD = decltype(lead_c)::value;
        constexpr int SA = S + LEAD;
        // early B (measured on the 8-wave 256 x 256 NT tile: same warm time,
        // 4-6 % less with the caches scrubbed at 4096^3)
        constexpr bool kEarlyB = ring_early_b(S, LEAD, kPrio);
        char *const ring_a = smem;
        char *const ring_b = smem + SA * Cfg::A_BYTES;
        if constexpr (S == 1) {
            // one slot: the copy of round kt+1 may start only after every wave
            // has finished computing round kt; copy and compute never overlap
            st_c1 = __builtin_amdgcn_s_memtime();
            for (int kt = 0; kt < nk; ++kt) {
                issue_a(kt, ring_a, 0, kLA);
                issue_b(kt, ring_b, 0, kLB);
                wait_vmcnt<0>();
                barrier();
#pragma unroll
                for (int kk = 0; kk < Cfg::KSTEPS; ++kk) {
                    read_operands(ring_a, ring_b, kk, 0);
                    sync_operands(0);
                    mfmas(0, 0, kMfma);
                }
                barrier();
            }
        } else {
            constexpr bool spread = ring_spread(S, LEAD);
            // prologue (tiles past the end of K are all-zero copies, so every
            // iteration below is identical and every wait is one immediate)
#pragma unroll
            for (int t = 0; t < ring_prologue(S, LEAD); ++t) {
                issue_a(t, ring_a + ring_slot(t, SA) * Cfg::A_BYTES, 0, kLA);
                issue_b(t, ring_b + ring_slot(t, S) * Cfg::B_BYTES, 0, kLB);
            }
            if constexpr (LEAD)
                issue_a(S - 1, ring_a + ring_slot(S - 1, SA) * Cfg::A_BYTES, 0, kLA);
            wait_vmcnt<ring_wait_first(S, LEAD, kLA, kLB)>();
            barrier();
            st_c1 = __builtin_amdgcn_s_memtime();
            read_operands(ring_a, ring_b, 0, 0);
            if constexpr (kEarlyB) {
                // the B copies iteration 0 would issue, into the slot no tile used yet
                constexpr int t = ring_issue_tile_b(0, S, LEAD);
                issue_b(t, ring_b + ring_slot(t, S) * Cfg::B_BYTES, 0, kLB);
            }
            int ra = 0, rb = 0;  // A and B slots of tile kt
            // One K tile.  Its k-step kk computes from operand buffer (kk + P) & 1;
            // with an odd number of k-steps per tile the parity P alternates
            // from tile to tile, so the loop below runs tiles in pairs.
            auto tile = [&](int kt, auto parity_c) __attribute__((always_inline)) {
                constexpr int P = decltype(parity_c)::value;
                const int na = ra + 1 == SA ? 0 : ra + 1, nb = rb + 1 == S ? 0 : rb + 1;
                const char *as = ring_a + ra * Cfg::A_BYTES, *bs = ring_b + rb * Cfg::B_BYTES;
                // spread copies go to the slots freed at the previous barrier
                char *cas = ring_a + (ra == 0 ? SA - 1 : ra - 1) * Cfg::A_BYTES;
                char *cbs = ring_b + (rb == 0 ? S - 1 : rb - 1) * Cfg::B_BYTES;
                const int ta = ring_issue_tile_a(kt, S, LEAD), tb = ring_issue_tile_b(kt, S, LEAD);
                // the copies k-step kk issues (before its wait, in the last one)
                auto copies = [&](auto kk_c, auto kk_end_c) __attribute__((always_inline)) {
                    constexpr int k0 = decltype(kk_c)::value, k1 = decltype(kk_end_c)::value;
                    constexpr int a0 = copy_a_before(k0, kS, kLA, kLB, LEAD), a1 = copy_a_before(k1, kS, kLA, kLB, LEAD);
                    constexpr int b0 = copy_b_before(k0, kS, kLA, kLB, LEAD), b1 = copy_b_before(k1, kS, kLA, kLB, LEAD);
                    if constexpr (spread) {
                        if constexpr (LEAD) {
                            if constexpr (!kEarlyB)
                                issue_b(tb, cbs, b0, b1);
                            issue_a(ta, cas, a0, a1);
                        } else {
                            issue_a(ta, cas, a0, a1);
                            issue_b(tb, cbs, b0, b1);
                        }
                    }
                    return std::integral_constant<int, spread ? (a1 - a0) + (kEarlyB ? 0 : b1 - b0) : 0>();
                };
                // every k-step but the last
                static_for<kLast>([&](auto kk_c) __attribute__((always_inline)) {
                    constexpr int kk = decltype(kk_c)::value;
                    sync_operands((kk + P) & 1);
                    set_prio(std::integral_constant<int, 1>());
                    read_operands(as, bs, kk + 1, (kk + 1 + P) & 1);
                    auto nl = copies(kk_c, std::integral_constant<int, kk + 1>());
                    mfmas((kk + P) & 1, 0, kMfma);
                    interleave<kMfma, kReads, decltype(nl)::value, kRpm>();
                    __builtin_amdgcn_sched_barrier(0);
                    set_prio(std::integral_constant<int, 0>());
                });
                // last k-step: its operands are in registers; once they have
                // arrived this wave no longer reads tile kt's slots
                constexpr int last = (kLast + P) & 1, next = (kS + P) & 1;
                wait_lds();
                sync_operands(last);
                __builtin_amdgcn_sched_barrier(0);
                auto nl = copies(std::integral_constant<int, kLast>(), std::integral_constant<int, kS>());
                mfmas(last, 0, kMfma / 2);
                interleave<kMfma / 2, 0, decltype(nl)::value, kRpm>();
                __builtin_amdgcn_sched_barrier(0);
                // tile kt+1 has landed once only the copies issued after its
                // last B copy may be in flight; after the barrier every wave is
                // done with tile kt's slots and sees tile kt+1
                wait_vmcnt<ring_wait_steady(S, LEAD, kLA, kLB)>();
                barrier();
                set_prio(std::integral_constant<int, 1>());
                if constexpr (kEarlyB) {
                    // the next tile's first operands, one read per MFMA, then
                    // the B copies of tile kt+S+1 into the slot tile kt freed
                    const char *nas = ring_a + na * Cfg::A_BYTES, *nbs = ring_b + nb * Cfg::B_BYTES;
                    auto rd = [&](auto j_c) __attribute__((always_inline)) {
                        read_one(nas, nbs, std::integral_constant<int, 0>(), next, j_c);
                    };
                    auto cp = [&](auto c_c) __attribute__((always_inline)) {
                        constexpr int c = decltype(c_c)::value;
                        issue_b(tb + 1, (char *)bs, c, c + 1);
                    };
                    stretch(std::integral_constant<int, kMfma - kMfma / 2>(), std::integral_constant<int, kMfma / 2>(), last,
                            std::integral_constant<int, FM + FN>(), rd, std::integral_constant<int, kLB>(), cp);
                    set_prio(std::integral_constant<int, 0>());
                    ra = na;
                    rb = nb;
                    return;
                }
                read_operands(ring_a + na * Cfg::A_BYTES, ring_b + nb * Cfg::B_BYTES, 0, next);
                if constexpr (!spread) {
                    // burst: tile kt+S into the slots tile kt just freed
                    issue_a(tb, (char *)as, 0, kLA);
                    issue_b(tb, (char *)bs, 0, kLB);
                }
                mfmas(last, kMfma / 2, kMfma);
                interleave<kMfma - kMfma / 2, kReads, spread ? 0 : kLA + kLB, kRpm>();
                __builtin_amdgcn_sched_barrier(0);
                set_prio(std::integral_constant<int, 0>());
                ra = na;
                rb = nb;
            };
            if constexpr (kS % 2 == 0) {
                for (int kt = 0; kt < nk; ++kt)
                    tile(kt, std::integral_constant<int, 0>());
            } else {
                for (int kt = 0; kt < nk; kt += 2) {
                    tile(kt, std::integral_constant<int, 0>());
                    if (kt + 1 < nk)
                        tile(kt + 1, std::integral_constant<int, 1>());
                }
            }
            // no copy may still be writing LDS when the workgroup ends
            wait_vmcnt<0>();
            // the last iteration's reads of the next (padding) tile are never
            // used; with the NN form's untracked transposed reads, keep their
            // destination registers live until the reads have returned, so
            // the compiler cannot hand them to other values meanwhile
            sync_operands(0);
            sync_operands(1);
        }
    };
    // Instantiated rings: the B ring fits in 160 KiB with the A ring, and the
    // copies in flight fit the 6-bit vmcnt.
#define PG_RING_OK(i, l)                                                                                \
    ((i) >= 1 && ((l) == 0 || ((i) >= 2 && (i) <= kMaxLeadStages)) &&                                   \
     ring_fits_vmcnt((i), (l), Cfg::A_LOADS, Cfg::B_LOADS) &&                                            \
     ring_lds_bytes((i), (l), Cfg::A_BYTES, Cfg::B_BYTES) <= 160 * 1024)
    // K == 0: no K tile, C = 0 (the accumulators as cleared)
    if (nk > 0) switch (p.stages) {
#define PG_STAGES_CASE(i)                                                          \
    case i:                                                                        \
        if (p.a_lead) {                                                            \
            if constexpr (PG_RING_OK(i, 1))                                        \
                pipeline(std::integral_constant<int, i>(), std::integral_constant<int, 1>()); \
        } else {                                                                   \
            if constexpr (PG_RING_OK(i, 0))                                        \
                pipeline(std::integral_constant<int, i>(), std::integral_constant<int, 0>()); \
        }                                                                          \
        break;
        PG_STAGES_CASE(1) PG_STAGES_CASE(2) PG_STAGES_CASE(3) PG_STAGES_CASE(4)
        PG_STAGES_CASE(5) PG_STAGES_CASE(6) PG_STAGES_CASE(7) PG_STAGES_CASE(8)
        PG_STAGES_CASE(9) PG_STAGES_CASE(10)
#undef PG_STAGES_CASE
#undef PG_RING_OK
    default:
        break;  // rejected on the host
    }

    // Epilogue.  The ring is free once every copy has landed and every wave
    // is past its last LDS read; each wave then stages its output through
    // its own LDS strip so that every global store writes 16 contiguous bytes
    // per lane and whole row segments per instruction, instead of 8 bytes in
    // each of 16 or 32 rows.
    st_c2 = __builtin_amdgcn_s_memtime();
    wait_vmcnt<0>();
    barrier();
    // ReLU once over the accumulators, under one uniform branch
    if (p.relu) {
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int g = 0; g < FN; ++g)
#pragma unroll
                for (int v = 0; v < NACC; ++v)
                    acc[f][g][v] = acc[f][g][v] > 0.f ? acc[f][g][v] : 0.f;
    }
    T *C = (T *)p.C;
    const int M = p.M;
    const int mw = m0 + wm * Cfg::TM, nw = n0 + wn * Cfg::TN;
    auto out_value = [&](int f, int g, int v) { return (T)acc[f][g][v]; };
    // The workgroup's rows of C as one buffer resource (below 2 GiB, checked
    // on the host), so a 16-byte store needs one 32-bit offset per lane; a
    // store to a row past M falls outside it and is dropped.
    const __amdgpu_buffer_rsrc_t c_rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(C + (size_t)m0 * N), 0, min(BM, M - m0) * N * 2, 0x00020000);
    // 16 bytes (8 columns from n) of row m of C; columns past N are skipped
    auto store_row = [&](int m, int n, i16x8 x) {
        if (p.c_vec) {
            // N % 8 == 0: a 16-byte chunk is wholly inside or outside the row.
            // C is written once and is far larger than the L2s: streaming
            // (nt) at system scope (sc1), so the L2 keeps none of it.
            // Measured at 4096^3 against a plain store: -1.6 us for nt,
            // another -1 us for sc1.
            if (n < N)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), c_rs, ((m - m0) * N + n) * 2, 0,
                                                       kStoreNtSc1);
        } else if (m < M) {
            short *crow = (short *)(C + (size_t)m * N);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < N)
                    crow[n + e] = x[e];
        }
    };
    if constexpr (MF == 16) {
        // one strip of 16 rows x TN columns per block row f: lane holds row
        // lr, columns 16 g + 4 lh .. +3 of block g.  NF block rows go through
        // LDS per batch (as many as one ring slot holds for every wave), so a
        // batch costs one LDS round trip instead of one per block row.
        constexpr int TN = Cfg::TN, CH = TN / 8, STRIP = 32 * TN;
        constexpr int NF = epi_batch(FM, Cfg::SLOT_BYTES / (WAVES * STRIP));
        static_assert(NF >= 1 && FM % NF == 0 && NF * STRIP * WAVES <= Cfg::SLOT_BYTES,
                      "strips must fit in one ring slot");
        static_assert((16 * CH) % 64 == 0, "whole strip reads");
        char *strip = smem + wave * NF * STRIP;
#pragma unroll
        for (int f0 = 0; f0 < FM; f0 += NF) {
#pragma unroll
            for (int fl = 0; fl < NF; ++fl)
#pragma unroll
                for (int g = 0; g < FN; ++g) {
                    typename E::quad v;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] = out_value(f0 + fl, g, r);
                    *(typename E::quad *)(strip + fl * STRIP + strip_half_offset<TN>(lr, 2 * g + (lh >> 1), lh & 1)) =
                        v;
                }
#pragma unroll
            for (int fl = 0; fl < NF; ++fl)
#pragma unroll
                for (int i = 0; i < CH / 4; ++i) {
                    const int idx = i * 64 + lane;
                    const int r = idx / CH, c = idx % CH;
                    i16x8 x = *(const i16x8 *)(strip + fl * STRIP + strip_offset<TN>(r, c));
                    if (r & 1)
                        x = __builtin_shufflevector(x, x, 4, 5, 6, 7, 0, 1, 2, 3);
                    store_row(mw + (f0 + fl) * 16 + r, nw + c * 8, x);
                }
        }
    } else {
        // G blocks of 32 x 32 at a time (one 32-row strip, 32 G columns)
        constexpr int G = cbuf_blocks(FN, Cfg::SLOT_BYTES / WAVES);
        constexpr int CH = 4 * G;  // 16-byte chunks per strip row
        static_assert(2048 * G * WAVES <= Cfg::SLOT_BYTES, "strips must fit in one ring slot");
        char *strip = smem + wave * 2048 * G;
#pragma unroll
        for (int f = 0; f < FM; ++f) {
#pragma unroll
            for (int gp = 0; gp < FN / G; ++gp) {
                // MFMA layout -> strip: lane holds row lr, columns 32 gb + 8 q + 4 lh .. +3
#pragma unroll
                for (int gb = 0; gb < G; ++gb)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        typename E::quad v;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            v[r] = out_value(f, gp * G + gb, 4 * q + r);
                        *(typename E::quad *)(strip + cbuf_half_offset(lr, 4 * gb + q, lh, G)) = v;
                    }
                // strip -> C: lane takes 16 bytes (8 columns) of one row
#pragma unroll
                for (int i = 0; i < 2 * G; ++i) {
                    const int idx = i * 64 + lane;
                    const int r = idx / CH, c = idx % CH;
                    i16x8 x = *(const i16x8 *)(strip + cbuf_chunk_offset(r, c, G));
                    if (hswz(r))
                        x = __builtin_shufflevector(x, x, 4, 5, 6, 7, 0, 1, 2, 3);
                    store_row(mw + f * 32 + r, nw + (gp * G) * 32 + c * 8, x);
                }
            }
        }
    }
    if (p.stamps && threadIdx.x == 0) {
        const unsigned long long c3 = __builtin_amdgcn_s_memtime(), t3 = __builtin_amdgcn_s_memrealtime();
        unsigned long long *q = p.stamps + stamp_index(blockIdx.x, 0);
        q[0] = st_c0;
        q[1] = st_c1;
        q[2] = st_c2;
        q[3] = c3;
        q[4] = st_t0;
        q[5] = t3;
    }
}

}  // namespace pipegemm
