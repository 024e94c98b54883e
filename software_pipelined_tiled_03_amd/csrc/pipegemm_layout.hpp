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
// Workgroup -> C tile.  Workgroups are dispatched round-robin over the 8 XCDs
// (id mod 8), each with its own L2: the id is renumbered so that the ids one
// XCD receives are consecutive, and tiles are walked in groups of group_m
// tile rows (column by column within a group) so that the workgroups sharing
// an XCD share A panels and B panels.  A bijection from 0 .. tiles_m tiles_n
// - 1 onto the tiles (the grid is ceil(N / block_N) x ceil(M / block_M)
// workgroups, chapter 11, section 1.1); enumerated on the CPU.
PG_HD constexpr void map_tile(int bid, int tiles_m, int tiles_n, int group_m, int &tm, int &tn)
{
    const int nwg = tiles_m * tiles_n;
    const int xcd = bid & 7, idx = bid >> 3;
    const int per = nwg >> 3, rem = nwg & 7;
    const int id = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    const int width = group_m * tiles_n;
    const int first_m = (id / width) * group_m;
    const int gsize = tiles_m - first_m < group_m ? tiles_m - first_m : group_m;
    const int in_group = id % width;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

// Index of counter i (0..5) of workgroup bid in the clock-stamp array.
PG_HD constexpr int stamp_index(int bid, int i) { return 6 * bid + i; }

// ---------------------------------------------------------------------------
// K-contiguous tiles (A always; B in the NT form).  Row r holds BK elements,
// i.e. BK/8 16-byte chunks; logical chunk c of row r is stored at physical
// chunk c ^ kswz(r).
//
// MFMA operand reads: with the 32x32x16 MFMA (MF = 32), 32 consecutive lanes
// read one logical chunk of 32 consecutive rows (lanes 32..63 the next chunk);
// with the 16x16x32 MFMA (MF = 16), 16 consecutive lanes read one chunk of 16
// rows (each further group of 16 lanes the next chunk).  Without a swizzle,
// rows 128 or 64 bytes apart fall on the same LDS banks.
//
// Bank rule of ds_read_b128 on gfx950, fitted to rocprofv3
// SQ_LDS_BANK_CONFLICT measurements of a few hundred per-lane address tables
// (it predicts every one of them): within each half-wave, the 16 lanes whose
// quad index (lane >> 2) & 7 has even parity are served together, and so are
// the 16 with odd parity; a group is conflict-free when its 16 addresses fall
// on 16 different 16-byte positions of a 256-byte bank row.
//  - MF = 32: (r & 7) ^ ((r >> 3) & 1) for BK = 64 and (r >> 2) & 3 for
//    BK = 32 (these measure conflict-free; e.g. r & 7 for BK = 64 costs 2x);
//  - MF = 16: a group holds rows {0-3, 12-15} of one chunk and rows 4..11 of
//    the next, i.e. chunk c ^ t(r) with t(r) = ((r >> 2) ^ (r >> 3)) & 1, so
//    the swizzle is a bijection onto positions once t is folded in:
//    ((r >> 1) & 7) ^ t(r) for BK = 64, ((r >> 2) & 3) ^ t(r) for BK = 32.
//    (The MF = 32 swizzles give a 2-way conflict on this pattern.)
// All depend only on r mod 16 (MF = 16) or r mod 32 (MF = 32), so a lane's
// swizzle is the same in every block of MF rows and block offsets become
// immediates.
template <int BK, int MF = 32>
PG_HD constexpr int kswz(int r)
{
    static_assert(BK == 32 || BK == 64, "block_K must be 32 or 64");
    static_assert(MF == 16 || MF == 32, "MFMA blocks are 16x16 or 32x32");
    if (MF == 16) {
        const int t = ((r >> 2) ^ (r >> 3)) & 1;
        return BK == 64 ? (((r >> 1) & 7) ^ t) : (((r >> 2) & 3) ^ t);
    }
    return BK == 64 ? ((r & 7) ^ ((r >> 3) & 1)) : ((r >> 2) & 3);
}

// Byte offset, within a K-contiguous tile, of logical chunk c of row r.
template <int BK, int MF = 32>
PG_HD constexpr int k_tile_offset(int r, int c)
{
    return (r * (BK / 8) + (c ^ kswz<BK, MF>(r))) * 16;
}

// The (row, logical chunk) that 16-byte unit u of a K-contiguous tile holds:
// the direct-to-LDS copy writes unit u = 64 * load + lane, so this picks the
// global chunk each lane fetches.
template <int BK, int MF = 32>
PG_HD constexpr void k_tile_unit(int u, int &r, int &c)
{
    r = u / (BK / 8);
    c = (u % (BK / 8)) ^ kswz<BK, MF>(r);
}

// ---------------------------------------------------------------------------
// N-contiguous B tile (NN form): row k holds BN elements, BN/8 chunks; logical
// chunk c of row k is stored at physical chunk c ^ nswz(k).  Rows are 256 or
// 512 bytes apart, so unswizzled they share banks.  A transposed read for the
// 32x32x16 MFMA has its two 16-lane groups read 4 consecutive rows x 64
// bytes; for the 16x16x32 MFMA they read rows k .. k+3 and k+8 .. k+11 x 32
// bytes.  nswz moves the 4 rows to the four different 64-byte quarters of a
// 256-byte bank row (bits 2-3), and rows k and k+8 to different 32-byte halves
// of a quarter (bit 1), so both patterns hit 32 distinct 8-byte bank pairs.
// The quarters measure conflict-free on gfx950 (the rate of a contiguous
// ds_read_b64_tr_b16); permuting chunks within 128 bytes only, e.g.
// (k & 3) << 1, measures 1.8x slower.  Needs BN >= 128 (16 chunks per row).
PG_HD constexpr int nswz(int k)
{
    return ((k & 3) << 2) | (((k >> 3) & 1) << 1);
}
// The same for rows of 64 elements (128 bytes, 8 chunks: the V tile of a
// 64-dimension attention head).  Two rows share a 256-byte bank row, so rows
// k and k+2 meet on the same banks; a transposed read's half-wave reads rows
// k .. k+3 x 64 bytes at the same logical chunks, and flipping the chunk's
// 64-byte half on every second pair of rows gives those 256 bytes 32
// distinct 8-byte bank pairs.  Checked on the CPU.
PG_HD constexpr int nswz64(int k) { return ((k >> 1) & 1) << 2; }
template <int W>
PG_HD constexpr int nswz_w(int k)
{
    static_assert(W == 64 || W >= 128, "N-contiguous rows of 64 or >= 128 elements");
    return W == 64 ? nswz64(k) : nswz(k);
}

template <int BN>
PG_HD constexpr int n_tile_offset(int k, int c)
{
    return (k * (BN / 8) + (c ^ nswz_w<BN>(k))) * 16;
}

template <int BN>
PG_HD constexpr void n_tile_unit(int u, int &k, int &c)
{
    k = u / (BN / 8);
    c = (u % (BN / 8)) ^ nswz_w<BN>(k);
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

// The same for the 16x16x32 MFMA operand: lane l must end up with k = 32 kk +
// 8 (l / 16) + e, e = 0..7, of column ncol0 + (l mod 16); so lane L of group G
// loads row 8 G + 4 h + L / 4 of k-step kk, columns 4 (L mod 4) .. +3 of the
// 16 columns.
template <int BN>
PG_HD constexpr int nn_tr_offset16(int lane, int kk, int ncol0, int h)
{
    const int G = lane >> 4, L = lane & 15;
    const int n = ncol0 + 4 * (L & 3);
    const int k = 32 * kk + 8 * G + 4 * h + (L >> 2);
    return n_tile_offset<BN>(k, n >> 3) + (n & 7) * 2;
}

// ---------------------------------------------------------------------------
// Attention tiles (head dimension D = 64 or 128).
//
// The K tile (BN keys x D, D contiguous) is stored as K-contiguous halves of
// 64 columns (one for D = 64, two for D = 128), each laid out like a BK = 64
// GEMM tile (so its operand reads reuse the measured kswz<64> swizzle): half
// hf holds columns 64 hf .. +63.
template <int BN>
PG_HD constexpr int attn_k_offset(int r, int c)  // c: 16-byte chunk 0..15 of row r
{
    return (c >> 3) * (BN * 128) + k_tile_offset<64>(r, c & 7);
}
template <int BN>
PG_HD constexpr void attn_k_unit(int u, int &r, int &c)
{
    int c8 = 0;
    k_tile_unit<64>(u % (BN * 8), r, c8);
    c = (u / (BN * 8)) * 8 + c8;
}

// The V tile (BN keys x D) is stored like the N-contiguous B tile of the NN
// form with D columns.  O^T = V^T P^T takes V^T as its first MFMA operand:
// lane l needs column d = dcol0 + (l mod 32) and, in slot j of k-step ks, the
// key attn_key_of_slot(l, ks, j) -- the order in which the S^T = K Q^T
// accumulator leaves P in the lane (so P goes to the second operand with no
// exchange; any order works as long as both operands use the same one).
PG_HD constexpr int attn_key_of_slot(int lane, int ks, int j)
{
    return 16 * ks + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
}
// Byte offset of transposed read r (slots 4r .. 4r+3) of that fragment: lane L
// of 16-lane group G loads row 16 ks + 8 r + 4 (G / 2) + L / 4, columns
// 4 (L mod 4) .. +3 of the group's 16 (see nn_tr_offset for the exchange).
template <int D>
PG_HD constexpr int v_tr_offset(int lane, int ks, int dcol0, int r)
{
    const int G = lane >> 4, L = lane & 15;
    const int n = dcol0 + 16 * (G & 1) + 4 * (L & 3);
    const int k = 16 * ks + 8 * r + 4 * (G >> 1) + (L >> 2);
    return n_tile_offset<D>(k, n >> 3) + (n & 7) * 2;
}

// ---------------------------------------------------------------------------
// Epilogue staging buffer: each wave turns G of its 32 x 32 output blocks at a
// time (one 32-row strip, 32 G columns, 2 bytes each) from the MFMA layout
// into row-major order, so the global stores write whole row segments.
//
// Row r of the strip has 4 G 16-byte chunks.  The MFMA layout gives lane l
// (l < 64) 4 consecutive columns of row l mod 32 (an 8-byte "half" of a
// chunk); lanes 0..15 (and each further group of 16) write 16 different rows
// at the same logical position, so both the chunk and the half are swizzled
// by the row: chunk c goes to c ^ cswz(r) and half h to h ^ hswz(r).  Reading
// back, lane i takes logical chunk i mod 4G of row i / 4G (16 bytes) and swaps
// its halves when hswz(r) is 1.
PG_HD constexpr int cswz(int r, int G)
{
    return G == 1 ? ((r >> 1) & 3) : (r & 7);
}
PG_HD constexpr int hswz(int r) { return (r >> 3) & 1; }

// Byte offset of the 8-byte half h of logical chunk c in row r.
PG_HD constexpr int cbuf_half_offset(int r, int c, int h, int G)
{
    return r * 64 * G + ((c ^ cswz(r, G)) << 4) + ((h ^ hswz(r)) << 3);
}

// Byte offset of the 16-byte physical chunk holding logical chunk c of row r.
PG_HD constexpr int cbuf_chunk_offset(int r, int c, int G)
{
    return r * 64 * G + ((c ^ cswz(r, G)) << 4);
}

// Output blocks per strip: the largest power of two dividing FN whose strip
// (2 KiB per block) fits in `region` bytes.
PG_HD constexpr int cbuf_blocks(int FN, int region)
{
    int g = 1;
    while (g * 2 <= FN && FN % (g * 2) == 0 && 2048 * g * 2 <= region)
        g *= 2;
    return g;
}

// Epilogue staging strip of the 16x16x32 layout: 16 rows x TN columns of one
// wave, row-major (2 TN bytes a row, TN / 8 16-byte chunks).  The MFMA layout
// gives lane l 4 consecutive columns of row l mod 16 (an 8-byte write);
// reading back, lane i takes 16 bytes of consecutive chunks.  Logical chunk c
// of row r sits at physical chunk c ^ sswz(r), and its two 8-byte halves are
// swapped in odd rows; this measures conflict-free on gfx950 for both the
// writes and the reads at TN = 64 and 128 (TN = 32 keeps a 2-way conflict on
// the writes, which are a few instructions per tile).
template <int TN>
PG_HD constexpr int sswz(int r)
{
    return (r >> 1) & (TN / 8 - 1);
}
template <int TN>
PG_HD constexpr int strip_offset(int r, int c)
{
    return r * TN * 2 + ((c ^ sswz<TN>(r)) << 4);
}
// Byte offset of the 8-byte half h of logical chunk c of row r.
template <int TN>
PG_HD constexpr int strip_half_offset(int r, int c, int h)
{
    return strip_offset<TN>(r, c) + ((h ^ (r & 1)) << 3);
}

// Block rows of the 16x16x32 epilogue staged through LDS per batch: the
// largest divisor of FM that is at most `fit` (the strips one wave's share of
// a ring slot holds), and at least 1.
PG_HD constexpr int epi_batch(int FM, int fit)
{
    int nf = 1;
    for (int d = 1; d <= FM; ++d)
        if (FM % d == 0 && d <= fit)
            nf = d;
    return nf;
}

// ---------------------------------------------------------------------------
// Pipeline schedule.  The A tiles live in a ring of S + lead slots and the B
// tiles in a ring of S slots (lead = 0 or 1); tile t uses A slot t mod (S +
// lead) and B slot t mod S.  Tiles with index >= nk are "padding" copies whose
// every chunk is out of range: they write zeros and read no memory, and they
// make every iteration identical.
//
// Iteration j computes tile j, each k-step reading the next k-step's operands
// into registers.  Once every LDS read of tile j has returned (during its last
// k-step) the wave waits until tile j+1 has landed, passes a barrier (every
// wave is done with tile j's slots and sees tile j+1), reads tile j+1's first
// operands and finishes tile j's last k-step from registers.  A slot is
// refilled only after that barrier (chapter 11, section 5.2: write a slot only
// after its last reader is done).
//
// Three ways to place the copies:
//  - burst (S = 2, lead 0): right after the barrier of iteration j, all copies
//    of tile j+S into the slots of tile j; the prologue issues tiles 0 .. S-1.
//  - spread (S >= 3, lead 0): during iteration j, before its wait, the copies
//    of tile j+S-1 into the slots of tile j-1 (freed at the previous barrier),
//    spread evenly over the k-steps (A pieces first) so the address unit takes
//    them while the matrix cores run; the prologue issues tiles 0 .. S-2.
//  - lead (S >= 2, lead 1): the A tile runs one tile further ahead.  During
//    iteration j the B copies of tile j+S-1 go out over the first half of the
//    k-steps and the A copies of tile j+S over the second half, each into the
//    slot its ring freed at the previous barrier; the prologue issues tiles
//    0 .. S-2 and the A tile of tile S-1.  The B tile then has one iteration
//    from its first copy to its wait, the A tile two.
// In every mode the copies go out in the order A(t), B(t), A(t+1), B(t+1), ...
// and the copy of a tile is issued one slot-turn after the tile its ring slot
// held has been read, which is the pages' rule that copy i may start once
// compute i-S has finished (with S + lead for the A ring).
PG_HD constexpr int ring_slot(int tile, int slots) { return tile % slots; }
PG_HD constexpr bool ring_spread(int S, int lead) { return lead ? S >= 2 : S >= 3; }
// whole tiles the prologue issues (lead adds the A tile of the next one)
PG_HD constexpr int ring_prologue(int S, int lead) { return ring_spread(S, lead) ? S - 1 : S; }
// tile whose B copies iteration j issues, and tile whose A copies it issues
PG_HD constexpr int ring_issue_tile_b(int j, int S, int lead)
{
    return ring_spread(S, lead) ? j + S - 1 : j + S;
}
PG_HD constexpr int ring_issue_tile_a(int j, int S, int lead)
{
    return ring_issue_tile_b(j, S, lead) + lead;
}
// copies (per wave) allowed in flight at the wait for tile 0, and at iteration
// j's wait for tile j+1 (everything issued after that tile's last B copy)
PG_HD constexpr int ring_wait_first(int S, int lead, int la, int lb)
{
    return ring_spread(S, lead) ? (S - 2) * (la + lb) + lead * la : (S - 1) * (la + lb);
}
PG_HD constexpr int ring_wait_steady(int S, int lead, int la, int lb)
{
    return (S - 2) * (la + lb) + lead * la;
}
// Copies one wave can have in flight at most (S-1 tiles and the leading A
// tile); the 6-bit vmcnt bounds it at 63.
PG_HD constexpr bool ring_fits_vmcnt(int S, int lead, int la, int lb)
{
    return (S - 1) * (la + lb) + lead * la <= 63;
}
// Deepest B ring built with lead (each lead ring is one more kernel variant).
constexpr int kMaxLeadStages = 4;

// Deepest ring without lead whose waits fit the 6-bit vmcnt, for `loads`
// copies per tile per wave.
PG_HD constexpr int ring_max_stages(int loads) { return 1 + 63 / loads; }
// LDS bytes of the two rings.
PG_HD constexpr int ring_lds_bytes(int S, int lead, int a_bytes, int b_bytes)
{
    return (S + lead) * a_bytes + S * b_bytes;
}

// Spread placement of one iteration's copies over its ks k-steps: the A (B)
// pieces issued before k-step kk, of la (lb) per wave.  Without lead the
// sequence A pieces then B pieces is cut evenly over all k-steps; with lead the
// B pieces are cut over the first half and the A pieces over the second half.
PG_HD constexpr int spread_part(int kk, int k0, int k1, int n)
{
    return kk <= k0 ? 0 : (kk >= k1 ? n : (kk - k0) * n / (k1 - k0));
}
// Early B (lead rings with S = 2, on the tiles that select it): iteration j
// issues the B copies of tile j+S right after its barrier, into the slot tile
// j has just freed, instead of over the first half of iteration j+1's k-steps.
// The copies go out in the same order (A(t), B(t), A(t+1), ...) and every
// wait allows the same count; only B's copies leave earlier, which shortens
// the exposed copy latency when A and B come from HBM.
PG_HD constexpr bool ring_early_b(int S, int lead, bool wanted) { return wanted && lead == 1 && S == 2; }
PG_HD constexpr int copy_a_before(int kk, int ks, int la, int lb, int lead)
{
    return lead ? spread_part(kk, ks / 2, ks, la)
                : (spread_part(kk, 0, ks, la + lb) < la ? spread_part(kk, 0, ks, la + lb) : la);
}
PG_HD constexpr int copy_b_before(int kk, int ks, int la, int lb, int lead)
{
    return lead ? spread_part(kk, 0, ks / 2, lb)
                : (spread_part(kk, 0, ks, la + lb) > la ? spread_part(kk, 0, ks, la + lb) - la : 0);
}

}  // namespace pipegemm
