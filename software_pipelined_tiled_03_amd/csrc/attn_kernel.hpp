// Device code of the pipelined attention forward pass (gfx950 / MI355X).
//
// O = softmax(scale * Q K^T [causal mask]) V for one (batch, head) and a block
// of BM = 32 * QB * WAVES queries per workgroup (QB blocks of 32 per wave).  The KV-length loop is the long
// reduction loop the TileLang tutorial pipelines exactly like the GEMM K loop
// (chapter 11, section 1.4): the K and V tiles of BN keys stream from HBM into
// a ring of S LDS slots with direct-to-LDS loads, copies of later tiles in
// flight while the matrix cores work on the current one (section 2.3: versioned
// buffers; section 5.2: a slot is refilled only after its last reader is done).
//
// Per wave (QB blocks of 32 queries; every K and V fragment read from LDS feeds
// QB MFMAs, so a second block halves the LDS reads per flop) and K/V tile:
//   S^T = K Q^T        v_mfma_f32_32x32x16 with the K fragment first, so each
//                      lane ends with one query's scores for 16 of every 32
//                      keys (its partner lane l ^ 32 holds the other 16);
//   online softmax     reference max m and sum l per query, in fp32,
//                      lane-local plus one exchange with the partner lane;
//                      m lags the running max by up to 8 in the base-2
//                      exponent (any reference gives the same quotient), so
//                      O is rescaled only when it moves; l sums the P values
//                      after rounding, as the second product sees them;
//   O^T += V^T P^T     P goes from the S^T accumulator to the second MFMA
//                      operand with no exchange: the key order it is left in
//                      is the order the V^T fragment is read in (any common
//                      order gives the same contraction); O^T's lane layout
//                      again puts one query in each lane, so the softmax
//                      rescale of O is lane-local.
// Q stays in registers for the whole loop; the output goes through the same
// LDS strip epilogue as the GEMM.
#pragma once

#include <math.h>

#include "attn_map.hpp"
#include "pipegemm_kernel.hpp"

namespace pipegemm {

// Kernel parameters, passed by value.
struct AttnArgs {
    const void *Q;  // [B, H, Sq, D]
    const void *K;  // [B, Hkv, Skv, D]
    const void *V;  // [B, Hkv, Skv, D]
    void *O;        // [B, H, Sq, D]
    int B, H, Hkv, Sq, Skv;
    int groups;        // H / Hkv: query heads per KV head
    int causal;        // key j visible to query i iff j <= i
    float scale_log2;  // softmax scale x log2(e)
    int stages;        // LDS ring slots, >= 1
    int nq;            // ceil(Sq / BM)
};

template <int BN_, int WAVES_, int QB_ = 1, int D_ = 128>
struct AttnTile {
    static constexpr int D = D_, BN = BN_, WAVES = WAVES_, QB = QB_, BM = 32 * QB * WAVES, THREADS = 64 * WAVES;
    static constexpr int K_BYTES = BN * D * 2, V_BYTES = BN * D * 2, SLOT_BYTES = K_BYTES + V_BYTES;
    static constexpr int K_LOADS = K_BYTES / (1024 * WAVES), V_LOADS = V_BYTES / (1024 * WAVES);
    static constexpr int LOADS = K_LOADS + V_LOADS;
    static constexpr int KB = BN / 32;  // 32-key blocks of S^T
    static constexpr int DS = D / 16;   // 16-wide d steps of S^T
    static constexpr int DB = D / 32;   // 32-wide d blocks of O^T
    static constexpr int KS = BN / 16;  // 16-key steps of O^T
    static_assert(BN == 64 || BN == 128, "block_N must be 64 or 128");
    static_assert(D == 64 || D == 128, "head dimension 64 or 128");
    static_assert(QB == 1 || QB == 2, "one or two 32-query blocks per wave");
    static_assert(K_BYTES % (1024 * WAVES) == 0 && K_LOADS >= 1, "whole 1 KiB copies per wave");
};

// ds_read_b64_tr_b16 at addr + OFF, with OFF in the instruction's 16-bit
// offset field.  The read is inline assembly for the reason ds_read_tr16_b64
// gives (the builtin would make the compiler wait for every copy in flight),
// and the compiler cannot fold constants into an inline-assembly address:
// without the field every read costs one more vector add (measured 4 % of
// the attention loop's time at 4096 keys).
template <int OFF>
__device__ __forceinline__ i16x4 ds_read_tr16_b64_at(const char *addr)
{
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field is 16 bits");
    i16x4 v;
    const uint32_t lds_addr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)addr;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(lds_addr), "i"(OFF) : "memory");
    return v;
}

// s_waitcnt lgkmcnt(N): all but the N most recent LDS reads of this wave
// have returned (LDS reads return in issue order).
template <int N>
__device__ __forceinline__ void wait_lds_keep()
{
    static_assert(N >= 0 && N < 16, "lgkmcnt is 4 bits");
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (N << 8));
}

// c + a + b with a, b in the input dtype (v_dot2c_f32_{f16,bf16} against
// (1, 1): exact products, fp32 accumulation)
__device__ __forceinline__ float dot2_ones(_Float16 a, _Float16 b, float c)
{
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2(h2{a, b}, h2{(_Float16)1.0f, (_Float16)1.0f}, c, false);
}
__device__ __forceinline__ float dot2_ones(__bf16 a, __bf16 b, float c)
{
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(b2{a, b}, b2{(__bf16)1.0f, (__bf16)1.0f}, c, false);
}

template <class T, class Cfg>
__global__ __launch_bounds__(Cfg::THREADS, 1) void attn_kernel(const AttnArgs p)
{
    using E = Elem<T>;
    using frag = typename E::frag;
    constexpr int D = Cfg::D, BN = Cfg::BN, BM = Cfg::BM, WAVES = Cfg::WAVES;
    constexpr int KB = Cfg::KB, DS = Cfg::DS, DB = Cfg::DB, KS = Cfg::KS, QB = Cfg::QB;

    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 31, lh = lane >> 5;

    // Work item (attn_work_item): longest query blocks first with the causal
    // mask, a head's blocks together on one XCD without it.
    int bh, qblk;
    attn_work_item((int)blockIdx.x, p.B * p.H, p.nq, p.causal != 0, bh, qblk);
    const int b = bh / p.H, h = bh % p.H;
    const int hk = h / p.groups;
    const int q0 = qblk * BM;
    const int q0w = q0 + wave * 32 * QB;  // this wave's first query
    // this lane's query in block qb (column of S^T and O^T): q0w + 32 qb + lr
    const int Skv = p.Skv;

    // key tiles: all of them, or up to the block's last query with the mask
    const int kv_end = p.causal ? min(Skv, q0 + BM) : Skv;
    const int nt = (kv_end + BN - 1) / BN;

    const char *qbase = (const char *)p.Q + (size_t)(b * p.H + h) * p.Sq * (D * 2);
    const char *kbase = (const char *)p.K + (size_t)(b * p.Hkv + hk) * Skv * (D * 2);
    const char *vbase = (const char *)p.V + (size_t)(b * p.Hkv + hk) * Skv * (D * 2);
    const int kv_bytes = Skv * D * 2;

    // Q fragments, second operand of S^T = K Q^T: lane l holds query
    // q0w + 32 qb + lr, d = 16 ds + 8 lh .. +7.  Queries past Sq read as zero.
    frag qf[QB][DS];
    {
        const __amdgpu_buffer_rsrc_t rq =
            __builtin_amdgcn_make_buffer_rsrc((void *)qbase, 0, p.Sq * D * 2, 0x00020000);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int ds = 0; ds < DS; ++ds)
                qf[qb][ds] = __builtin_bit_cast(
                    frag, __builtin_amdgcn_raw_buffer_load_b128(
                              rq, (uint32_t)((q0w + 32 * qb + lr) * D * 2 + (16 * ds + 8 * lh) * 2), 0, 0));
    }

    // Copies: per-lane offsets within a tile; each tile goes through a buffer
    // resource shifted to its first key (keys past Skv read as zero).
    uint32_t k_off[Cfg::K_LOADS], v_off[Cfg::V_LOADS];
#pragma unroll
    for (int t = 0; t < Cfg::K_LOADS; ++t) {
        int r, c;
        attn_k_unit<BN>((t * WAVES + wave) * 64 + lane, r, c);
        k_off[t] = (uint32_t)(r * D * 2 + c * 16);
    }
#pragma unroll
    for (int t = 0; t < Cfg::V_LOADS; ++t) {
        int k, c;
        n_tile_unit<D>((t * WAVES + wave) * 64 + lane, k, c);
        v_off[t] = (uint32_t)(k * D * 2 + c * 16);
    }
    auto tile_rsrc = [&](const char *base, int j) __attribute__((always_inline)) {
        const int64_t shift = (int64_t)j * BN * D * 2;
        const int64_t left = (int64_t)kv_bytes - shift;
        return __builtin_amdgcn_make_buffer_rsrc((void *)(base + shift), 0, left > 0 ? (int)left : 0, 0x00020000);
    };
    auto issue_k = [&](int j, char *slot, int first, int last) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(kbase, j);
#pragma unroll
        for (int t = 0; t < Cfg::K_LOADS; ++t)
            if (t >= first && t < last)
                copy_1k(rs, slot + (t * WAVES + wave) * 1024, k_off[t]);
    };
    auto issue_v = [&](int j, char *slot, int first, int last) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(vbase, j);
#pragma unroll
        for (int t = 0; t < Cfg::V_LOADS; ++t)
            if (t >= first && t < last)
                copy_1k(rs, slot + Cfg::K_BYTES + (t * WAVES + wave) * 1024, v_off[t]);
    };

    // Operand reads.  K fragment (first operand of S^T): key 32 kb + lr,
    // d chunk 2 ds + lh; the swizzle repeats every 32 rows, so block kb adds
    // 32 rows of 128 bytes within a half.
    int k_rd[DS];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
        k_rd[ds] = attn_k_offset<BN>(lr, 2 * ds + lh);
    auto read_k = [&](const char *slot, int ds, frag (&kf)[KB]) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            kf[kb] = *(const frag *)(slot + k_rd[ds] + kb * 32 * 128);
    };
    // V^T fragment (first operand of O^T): column d = 32 db + lr, keys in the
    // order P is held in (two transposed reads).  The k-step ks moves every
    // read by 32 D ks bytes (v_tr_offset), which goes into the instruction's
    // offset field with the K part of the slot; the lane part is computed
    // once per slot.
    int v_rd[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 2; ++r)
            v_rd[db][r] = v_tr_offset<D>(lane, 0, 32 * db, r);
    auto read_v = [&](const char *slot, auto ks_c, frag (&vf)[DB]) __attribute__((always_inline)) {
        constexpr int OFF = Cfg::K_BYTES + 32 * D * decltype(ks_c)::value;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            i16x8 out;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const i16x4 v = ds_read_tr16_b64_at<OFF>(slot + v_rd[db][r]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    out[4 * r + e] = v[e];
            }
            vf[db] = __builtin_bit_cast(frag, out);
        }
    };

    // Accumulators and softmax state (per query block; the partner lane holds the same).
    f32x16 oacc[DB][QB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                oacc[db][qb][v] = 0.0f;
    float m_run[QB], l_run[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.0f;
    }
    const float sl2 = p.scale_log2;

    // The three phases of one key tile j: S^T = K Q^T into `sacc`, the
    // online softmax of `sacc` into `pf`, O^T += V^T P^T.  The copies of tile
    // cj into `cslot` (if any) are spread over the two MFMA phases: K pieces
    // among the S^T k-steps, V pieces among the O^T k-steps.
    using SAcc = f32x16[KB][QB];
    using PFrag = frag[KS][QB];
    auto s_phase = [&](SAcc &sacc, const char *slot, int cj, char *cslot, auto copies_c) __attribute__((always_inline)) {
        constexpr bool copies = decltype(copies_c)::value;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    sacc[kb][qb][v] = 0.0f;
        frag kf[2][KB];
        read_k(slot, 0, kf[0]);
        static_for<DS>([&](auto ds_c) __attribute__((always_inline)) {
            constexpr int ds = decltype(ds_c)::value;
            if constexpr (ds + 1 < DS)
                read_k(slot, ds + 1, kf[(ds + 1) & 1]);
            constexpr int c0 = ds * Cfg::K_LOADS / DS, c1 = (ds + 1) * Cfg::K_LOADS / DS;
            if constexpr (copies && c1 > c0)
                issue_k(cj, cslot, c0, c1);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    sacc[kb][qb] = E::mfma(kf[ds & 1][kb], qf[qb][ds], sacc[kb][qb]);
        });
    };
    auto softmax = [&](SAcc &sacc, PFrag &pf, int j) __attribute__((always_inline)) {
        // mask: keys past the query (causal) or past Skv
        const int key0 = j * BN;
        if ((p.causal && key0 + BN - 1 > q0w) || key0 + BN > Skv) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                // the last visible key, relative to this lane's first key of
                // the tile: element v of block kb is key key0 + 4 lh + 32 kb +
                // 8 (v / 4) + v % 4.  A score is kept by min(s, +inf) and masked
                // by min(s, -inf), the infinity's sign taken from last - offset:
                // no compares, branches or lane masks.  The IEEE 754-2019
                // minimum (v_minimum_f32) needs no quieting of its inputs,
                // which the IEEE-mode minNum would spend two instructions on
                // per score; the scores and the infinities are never NaN.
                const int last = (p.causal ? min(q0w + 32 * qb + lr, Skv - 1) : Skv - 1) - key0 - 4 * lh;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int d = last - (32 * kb + 8 * (v >> 2) + (v & 3));
                        const float lim = __builtin_bit_cast(float, ((unsigned)d & 0x80000000u) | 0x7f800000u);
                        sacc[kb][qb][v] = __builtin_elementwise_minimum(sacc[kb][qb][v], lim);
                    }
            }
        }
        // online softmax per query block (base-2 exponentials of
        // scale x log2(e) x score)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float mx = sacc[0][qb][0];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    mx = fmaxf(mx, sacc[kb][qb][v]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            // the reference max moves only when some query's max has grown by
            // more than 8 in the base-2 exponent: the exponentials then stay
            // at most 256, far inside the input dtype's range, and O and l
            // are rescaled on few tiles (measured: 2-7 % faster at 4096 keys)
            if (__any((mx - m_run[qb]) * sl2 > 8.0f)) {
                const float m_new = fmaxf(m_run[qb], mx);  // finite: every query sees key 0 in tile 0
                const float alpha = __builtin_amdgcn_exp2f((m_run[qb] - m_new) * sl2);
                l_run[qb] *= alpha;
                m_run[qb] = m_new;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        oacc[db][qb][v] *= alpha;
            }
            const float mb = m_run[qb] * sl2;
            float rs = 0.0f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const float e = __builtin_amdgcn_exp2f(fmaf(sacc[ks >> 1][qb][8 * (ks & 1) + jj], sl2, -mb));
                    pf[ks][qb][jj] = (T)e;
                }
            // the row sum of the rounded P, two at a time (exact products, fp32 sum)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int jj = 0; jj < 8; jj += 2)
                    rs = dot2_ones(pf[ks][qb][jj], pf[ks][qb][jj + 1], rs);
            rs += __shfl_xor(rs, 32);
            l_run[qb] += rs;
        }
    };
    auto o_phase = [&](const PFrag &pf, const char *slot, int cj, char *cslot, auto copies_c) __attribute__((always_inline)) {
        constexpr bool copies = decltype(copies_c)::value;
        // V^T fragments are read two k-steps ahead (three buffers): the wait
        // before step ks lets the 2 DB transposed reads of step ks + 1 stay in
        // flight, and LDS reads return in issue order.
        frag vf[3][DB];
        read_v(slot, std::integral_constant<int, 0>(), vf[0]);
        read_v(slot, std::integral_constant<int, 1>(), vf[1]);
        static_for<KS>([&](auto ks_c) __attribute__((always_inline)) {
            constexpr int ks = decltype(ks_c)::value;
            if constexpr (ks + 1 < KS) {
                wait_lds_keep<2 * DB>();
#pragma unroll
                for (int g = 0; g < DB; ++g)
                    asm volatile("" : "+v"(vf[ks % 3][g]));
            } else {
                sync_nn_operands(vf[ks % 3]);
            }
            if constexpr (ks + 2 < KS)
                read_v(slot, std::integral_constant<int, ks + 2>(), vf[(ks + 2) % 3]);
            constexpr int c0 = ks * Cfg::V_LOADS / KS, c1 = (ks + 1) * Cfg::V_LOADS / KS;
            if constexpr (copies && c1 > c0)
                issue_v(cj, cslot, c0, c1);
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    oacc[db][qb] = E::mfma(vf[ks % 3][db], pf[ks][qb], oacc[db][qb]);
        });
        // every LDS read of this slot has returned
        wait_lds();
    };
    auto compute_tile = [&](int j, const char *slot, int cj, char *cslot, auto copies_c) __attribute__((always_inline)) {
        SAcc sacc;
        s_phase(sacc, slot, cj, cslot, copies_c);
        PFrag pf;
        softmax(sacc, pf, j);
        o_phase(pf, slot, cj, cslot, copies_c);
    };

    // With the causal mask the tiles whose first key lies past this wave's
    // last query are the workgroup's last ones, and the wave has nothing to
    // add in them: every score is masked, P is zero, and m, l and O stay as
    // they are, bit for bit.  The wave computes only the tiles before them
    // (nt_w); in the rest it issues its share of the copies and passes the
    // same waits and barriers as the other waves, whose SIMD partner then has
    // the matrix core to itself.  Not on the two-block 128-key 8-wave tile,
    // which is at 256 registers and would spill.
    constexpr bool kSkipIdle = !(WAVES == 8 && QB == 2 && BN == 128);
    const int nt_w = (kSkipIdle && p.causal) ? min(nt, (q0w + 32 * QB - 1) / BN + 1) : nt;
    auto pipeline = [&](auto stages_c) __attribute__((always_inline)) {
        constexpr int S = decltype(stages_c)::value;
        constexpr int L = Cfg::LOADS;
        if constexpr (S == 1) {
            for (int j = 0; j < nt_w; ++j) {
                issue_k(j, smem, 0, Cfg::K_LOADS);
                issue_v(j, smem, 0, Cfg::V_LOADS);
                wait_vmcnt<0>();
                barrier();
                compute_tile(j, smem, 0, smem, std::false_type());
                barrier();
            }
            for (int j = nt_w; j < nt; ++j) {
                issue_k(j, smem, 0, Cfg::K_LOADS);
                issue_v(j, smem, 0, Cfg::V_LOADS);
                wait_vmcnt<0>();
                barrier();
                barrier();
            }
        } else {
            // prologue: tiles 0 .. S-2 (tiles past the last are all-zero copies)
#pragma unroll
            for (int t = 0; t < S - 1; ++t) {
                issue_k(t, smem + t * Cfg::SLOT_BYTES, 0, Cfg::K_LOADS);
                issue_v(t, smem + t * Cfg::SLOT_BYTES, 0, Cfg::V_LOADS);
            }
            wait_vmcnt<(S - 2) * L>();
            barrier();
            int rs_ = 0;  // slot of tile j
            for (int j = 0; j < nt_w; ++j) {
                const int cs = rs_ == 0 ? S - 1 : rs_ - 1;  // freed at the previous barrier
                compute_tile(j, smem + rs_ * Cfg::SLOT_BYTES, j + S - 1, smem + cs * Cfg::SLOT_BYTES,
                             std::true_type());
                // tile j+1 has landed once only the S-2 tiles issued after it
                // may be in flight; after the barrier every wave is done with
                // slot j and sees tile j+1
                wait_vmcnt<(S - 2) * L>();
                barrier();
                rs_ = rs_ + 1 == S ? 0 : rs_ + 1;
            }
            // past this wave's diagonal: the same copies (K then V of tile
            // j+S-1 into the slot the last barrier freed), waits and barriers
            for (int j = nt_w; j < nt; ++j) {
                const int cs = rs_ == 0 ? S - 1 : rs_ - 1;
                issue_k(j + S - 1, smem + cs * Cfg::SLOT_BYTES, 0, Cfg::K_LOADS);
                issue_v(j + S - 1, smem + cs * Cfg::SLOT_BYTES, 0, Cfg::V_LOADS);
                wait_vmcnt<(S - 2) * L>();
                barrier();
                rs_ = rs_ + 1 == S ? 0 : rs_ + 1;
            }
        }
    };
    switch (p.stages) {
#define PG_ATTN_CASE(i)                                                                   \
    case i:                                                                               \
        if constexpr ((i - 1) * Cfg::LOADS <= 63 && i * Cfg::SLOT_BYTES <= 160 * 1024)   \
            pipeline(std::integral_constant<int, i>());                                   \
        break;
        PG_ATTN_CASE(1) PG_ATTN_CASE(2) PG_ATTN_CASE(3) PG_ATTN_CASE(4)
#undef PG_ATTN_CASE
    default:
        break;  // rejected on the host
    }

    // Epilogue: O = O^T / l through a per-wave LDS strip (the GEMM's), whole
    // 16-byte row segments per lane.  The ring is free once every copy has
    // landed and every wave is past its last read.
    constexpr int G = cbuf_blocks(DB, Cfg::SLOT_BYTES / WAVES);
    constexpr int CH = 4 * G;
    static_assert(2048 * G * WAVES <= Cfg::SLOT_BYTES, "strips must fit in one ring slot");
    wait_vmcnt<0>();
    barrier();
    char *strip = smem + wave * 2048 * G;
    short *obase = (short *)((char *)p.O + (size_t)(b * p.H + h) * p.Sq * (D * 2));
    // this head's rows of O as one buffer resource: a row past Sq falls
    // outside it and its store is dropped.  O is written once: streaming
    // (nt) at system scope (sc1), as the GEMM's C (measured 2-3 % faster than
    // plain stores at 4096 keys)
    const __amdgpu_buffer_rsrc_t o_rs = __builtin_amdgcn_make_buffer_rsrc((void *)obase, 0, p.Sq * D * 2, 0x00020000);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float inv_l = 1.0f / l_run[qb];
#pragma unroll
        for (int gp = 0; gp < DB / G; ++gp) {
#pragma unroll
            for (int gb = 0; gb < G; ++gb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    typename E::quad v;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] = (T)(oacc[gp * G + gb][qb][4 * q + r] * inv_l);
                    *(typename E::quad *)(strip + cbuf_half_offset(lr, 4 * gb + q, lh, G)) = v;
                }
#pragma unroll
            for (int i = 0; i < 2 * G; ++i) {
                const int idx = i * 64 + lane;
                const int r = idx / CH, c = idx % CH;
                i16x8 x = *(const i16x8 *)(strip + cbuf_chunk_offset(r, c, G));
                if (hswz(r))
                    x = __builtin_shufflevector(x, x, 4, 5, 6, 7, 0, 1, 2, 3);
                const int query = q0w + 32 * qb + r;
                // unsigned: a padding row's offset may pass 2^31 (Sq D 2 < 2^31 is checked on the host)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), o_rs,
                                                       (uint32_t)(query * D + (gp * G) * 32 + c * 8) * 2u, 0,
                                                       kStoreNtSc1);
            }
        }
    }
}

}  // namespace pipegemm
