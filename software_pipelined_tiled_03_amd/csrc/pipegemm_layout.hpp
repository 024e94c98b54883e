// LDS tile layouts and the pipeline's slot/wait schedule, as host+device
// functions: the kernel uses them, and tests/layout_check.cpp enumerates them
// on the CPU (write/read consistency, bank-conflict freedom, slot safety).
#pragma once

#if defined(__HIPCC__)
#define PG_HD __host__ __device__
#else
#define PG_HD
#endif

namespace pipegemm {

// ---------------------------------------------------------------------------
// K-contiguous tiles (A always; B in the NT form).  Row r holds BK elements,
// i.e. BK/8 16-byte chunks; logical chunk c of row r is stored at physical
// chunk c ^ kswz(r).
//
// MFMA operand reads have 32 consecutive lanes read one logical chunk of 32
// consecutive rows (rows 32q .. 32q+31).  The swizzle maps any 8 consecutive
// rows of such a block to 8 distinct 16-byte bank groups, and any 16
// consecutive rows to 16 distinct positions modulo 16 chunks, so ds_read_b128
// is conflict-free whether the LDS serves 8 or 16 lanes' 16 bytes per cycle.
// It depends only on r mod 32, so a lane's swizzle is the same in every
// 32-row block and block offsets become immediates.
template <int BK>
PG_HD constexpr int kswz(int r)
{
    static_assert(BK == 32 || BK == 64, "block_K must be 32 or 64");
    return BK == 64 ? ((r & 7) ^ ((r >> 3) & 1)) : (((r >> 1) ^ (r >> 3)) & 3);
}

// Byte offset, within a K-contiguous tile, of logical chunk c of row r.
template <int BK>
PG_HD constexpr int k_tile_offset(int r, int c)
{
    return (r * (BK / 8) + (c ^ kswz<BK>(r))) * 16;
}

// The (row, logical chunk) that 16-byte unit u of a K-contiguous tile holds:
// the direct-to-LDS copy writes unit u = 64 * load + lane, so this picks the
// global chunk each lane fetches.
template <int BK>
PG_HD constexpr void k_tile_unit(int u, int &r, int &c)
{
    r = u / (BK / 8);
    c = (u % (BK / 8)) ^ kswz<BK>(r);
}

// ---------------------------------------------------------------------------
// N-contiguous B tile (NN form): row k holds BN elements, BN/8 chunks; logical
// chunk c of row k is stored at physical chunk c ^ nswz(k).  A transposed read
// by 16 lanes touches 4 consecutive rows x 2 adjacent chunks (32 bytes each);
// nswz puts the 4 rows' chunk pairs on 8 distinct 16-byte bank groups.
PG_HD constexpr int nswz(int k)
{
    return ((k & 3) << 1) ^ ((k >> 2) & 1);
}

template <int BN>
PG_HD constexpr int n_tile_offset(int k, int c)
{
    return (k * (BN / 8) + (c ^ nswz(k))) * 16;
}

template <int BN>
PG_HD constexpr void n_tile_unit(int u, int &k, int &c)
{
    k = u / (BN / 8);
    c = (u % (BN / 8)) ^ nswz(k);
}

// Transposed read (ds_read_b64_tr_b16) feeding the 32x32x16 MFMA operand from
// the N-contiguous tile: lane l must end up with k = 16 kk + 8 (l / 32) + e,
// e = 0..7, of column ncol0 + (l mod 32).  Within each group of 16 lanes the
// instruction hands lane i element (i mod 4) of the 8 bytes lane 4 e + i / 4
// loaded, for e = 0..3; so lane L of group G loads row L / 4 (of the 4-row
// block), columns 4 (L mod 4) .. +3 of the group's 16 columns.  Returns the
// byte offset within the tile of read h (h = 0: e 0..3, h = 1: e 4..7).
template <int BN>
PG_HD constexpr int nn_tr_offset(int lane, int kk, int ncol0, int h)
{
    const int G = lane >> 4, L = lane & 15;
    const int n = ncol0 + 16 * (G & 1) + 4 * (L & 3);
    const int k = 16 * kk + 8 * (G >> 1) + 4 * h + (L >> 2);
    return n_tile_offset<BN>(k, n >> 3) + (n & 7) * 2;
}

// ---------------------------------------------------------------------------
// Pipeline schedule over a ring of S slots (S >= 2), nk K tiles.
//   prologue: tile t (t < min(S-1, nk)) into slot t
//   iteration kt: wait until at most ring_inflight(...) tiles issued after kt
//   are outstanding, barrier, issue tile kt+S-1 (if any) into its slot,
//   compute slot kt mod S.
PG_HD constexpr int ring_slot(int tile, int S) { return tile % S; }

PG_HD constexpr int ring_prologue(int S, int nk) { return S - 1 < nk ? S - 1 : nk; }

// Tiles issued after tile kt that may still be in flight at iteration kt's wait.
PG_HD constexpr int ring_inflight(int kt, int S, int nk)
{
    return (S - 2) < (nk - 1 - kt) ? (S - 2) : (nk - 1 - kt);
}

}  // namespace pipegemm
