// Host-side check of the LDS layouts and the ring schedule the GPU kernel uses
// (software_pipelined_tiled_03_amd/csrc/pipegemm_layout.hpp), by enumeration:
//  1. every 16-byte unit the direct-to-LDS copy writes lands where the MFMA
//     operand reads look for it (K-contiguous and N-contiguous tiles);
//  2. the transposed reads of the NN form deliver, lane by lane, exactly the
//     k / n elements the 32x32x16 and 16x16x32 MFMA operands need;
//  3. the operand reads are free of LDS bank conflicts;
//  4. over a ring of S slots, each tile's wait covers its own copy exactly, and
//     no slot is overwritten while a tile in it is still to be read.
// Prints one line per failure and exits non-zero on any.
#include <cstdio>
#include <set>
#include <vector>
#include <algorithm>

#include "pipegemm_layout.hpp"
#include "attn_map.hpp"

using namespace pipegemm;

static int failures = 0;
#define CHECK(cond, ...)                       \
    do {                                       \
        if (!(cond)) {                         \
            if (failures < 40) {               \
                std::printf("FAIL: " __VA_ARGS__); \
                std::printf("\n");             \
            }                                  \
            ++failures;                        \
        }                                      \
    } while (0)

// The measured bank rule of ds_read_b128 on gfx950: within each half-wave,
// the lanes whose quad index (lane >> 2) & 7 has even parity form one group of
// 16 and the odd ones another; a group is conflict-free when its distinct
// addresses fall on distinct 16-byte positions of a 256-byte bank row.
static bool b128_conflict_free(const int *addr)
{
    for (int half = 0; half < 64; half += 32)
        for (int p = 0; p < 2; ++p) {
            int seen[16];
            for (int i = 0; i < 16; ++i)
                seen[i] = -1;
            for (int l = half; l < half + 32; ++l) {
                const int q = (l >> 2) & 7;
                if (((q ^ (q >> 1) ^ (q >> 2)) & 1) != p)
                    continue;
                const int pos = (addr[l] >> 4) & 15;
                if (seen[pos] >= 0 && seen[pos] != addr[l])
                    return false;
                seen[pos] = addr[l];
            }
        }
    return true;
}

template <int BK>
void check_k_tile(int rows)
{
    const int cpr = BK / 8;
    for (int u = 0; u < rows * cpr; ++u) {
        int r = 0, c = 0;
        k_tile_unit<BK>(u, r, c);
        CHECK(c >= 0 && c < cpr, "BK=%d unit %d: chunk %d out of row", BK, u, c);
        CHECK(k_tile_offset<BK>(r, c) == u * 16, "BK=%d unit %d: written (%d,%d) read elsewhere", BK, u, r, c);
    }
    for (int r = 0; r < rows; ++r) {
        CHECK(kswz<BK>(r) == kswz<BK>(r % 32), "BK=%d: swizzle of row %d differs from row %d", BK, r, r % 32);
        for (int c = 0; c < cpr; ++c)
            CHECK(k_tile_offset<BK>(r + 32, c) == k_tile_offset<BK>(r, c) + 32 * BK * 2,
                  "BK=%d: 32-row blocks are not a fixed stride apart", BK);
    }
    // MFMA operand read: lane l reads row base + l%32, chunk 2kk + l/32.  The
    // bank behaviour of these reads was measured on the GPU (the swizzle is the
    // measured conflict-free choice); here: every lane reads a distinct 16-byte
    // unit, and within each 16-lane group the 16 units cover all 16 positions of
    // a 256-byte LDS row (a necessary condition for a conflict-free cycle).
    for (int base = 0; base < rows; base += 32)
        for (int kk = 0; kk < BK / 16; ++kk) {
            std::set<int> all;
            for (int g = 0; g < 64; g += 16) {
                std::set<int> pos;
                for (int l = g; l < g + 16; ++l) {
                    const int off = k_tile_offset<BK>(base + l % 32, 2 * kk + l / 32);
                    all.insert(off);
                    pos.insert((off / 16) % 16);
                }
                CHECK(pos.size() == 16, "BK=%d rows %d kk %d lanes %d..: 16-byte units repeat in a 256-byte row", BK,
                      base, kk, g);
            }
            CHECK(all.size() == 64, "BK=%d: operand reads overlap", BK);
            int addr[64];
            for (int l = 0; l < 64; ++l)
                addr[l] = k_tile_offset<BK>(base + l % 32, 2 * kk + l / 32);
            CHECK(b128_conflict_free(addr), "BK=%d MF=32 rows %d kk %d: bank conflict", BK, base, kk);
        }
    // the 16x16x32 tile layout: copies land where the reads look
    for (int u = 0; u < rows * cpr; ++u) {
        int r = 0, c = 0;
        k_tile_unit<BK, 16>(u, r, c);
        CHECK(c >= 0 && c < cpr, "BK=%d MF=16 unit %d: chunk %d out of row", BK, u, c);
        CHECK((k_tile_offset<BK, 16>(r, c) == u * 16), "BK=%d MF=16 unit %d: written (%d,%d) read elsewhere", BK, u, r,
              c);
    }
    // 16x16x32 operand read: lane l reads row base + l%16, chunk 4kk + l/16;
    // the swizzle is periodic in 16 rows, so 16-row blocks are a fixed stride
    // apart, and each 16-lane group covers the 16 positions of a 256-byte row.
    for (int r = 0; r < rows; ++r) {
        CHECK((kswz<BK, 16>(r) == kswz<BK, 16>(r % 16)), "BK=%d: swizzle of row %d differs from row %d", BK, r,
              r % 16);
        if (r + 16 < rows)
            for (int c = 0; c < cpr; ++c)
                CHECK((k_tile_offset<BK, 16>(r + 16, c) == k_tile_offset<BK, 16>(r, c) + 16 * BK * 2),
                      "BK=%d: 16-row blocks are not a fixed stride apart", BK);
    }
    for (int base = 0; base < rows; base += 16)
        for (int kk = 0; kk < BK / 32; ++kk) {
            std::set<int> all;
            int addr[64];
            for (int l = 0; l < 64; ++l) {
                addr[l] = k_tile_offset<BK, 16>(base + l % 16, 4 * kk + l / 16);
                all.insert(addr[l]);
            }
            CHECK(all.size() == 64, "BK=%d MF=16: operand reads overlap", BK);
            CHECK(b128_conflict_free(addr), "BK=%d MF=16 rows %d kk %d: bank conflict", BK, base, kk);
        }
}

template <int BN>
void check_n_tile(int bk)
{
    const int cpr = BN / 8;
    for (int u = 0; u < bk * cpr; ++u) {
        int k = 0, c = 0;
        n_tile_unit<BN>(u, k, c);
        CHECK(c >= 0 && c < cpr, "BN=%d unit %d: chunk out of row", BN, u);
        CHECK(n_tile_offset<BN>(k, c) == u * 16, "BN=%d unit %d: written (%d,%d) read elsewhere", BN, u, k, c);
    }
    // transposed reads: decode which (k, n) each loaded element is, apply the
    // instruction's lane exchange, compare with what the MFMA operand needs
    for (int kk = 0; kk < bk / 16; ++kk)
        for (int ncol0 = 0; ncol0 < BN; ncol0 += 32)
            for (int h = 0; h < 2; ++h) {
                int lk[64][4], ln[64][4], word[64];
                for (int l = 0; l < 64; ++l) {
                    const int off = nn_tr_offset<BN>(l, kk, ncol0, h);
                    CHECK(off % 8 == 0 && off >= 0 && off + 8 <= bk * BN * 2, "BN=%d: tr read offset %d", BN, off);
                    word[l] = off / 4;
                    const int k = off / (BN * 2);
                    const int phys = (off % (BN * 2)) / 16;
                    const int c = phys ^ nswz(k);
                    for (int j = 0; j < 4; ++j) {
                        lk[l][j] = k;
                        ln[l][j] = c * 8 + (off % 16) / 2 + j;
                    }
                }
                for (int l = 0; l < 64; ++l) {
                    const int G = l / 16, i = l % 16;
                    for (int e = 0; e < 4; ++e) {
                        const int src = 16 * G + 4 * e + i / 4;
                        const int k = lk[src][i % 4], n = ln[src][i % 4];
                        CHECK(k == 16 * kk + 8 * (l / 32) + 4 * h + e && n == ncol0 + l % 32,
                              "BN=%d kk=%d ncol0=%d h=%d lane %d elem %d: got (k=%d,n=%d)", BN, kk, ncol0, h, l, e,
                              k, n);
                    }
                }
                // the 4 rows of each 16-lane group put their 64-byte pieces in the
                // 4 different quarters of a 256-byte LDS row (the property that
                // separated conflict-free from conflicting swizzles on the GPU)
                for (int g = 0; g < 64; g += 16) {
                    std::set<int> quarters;
                    for (int l = g; l < g + 16; ++l)
                        quarters.insert((word[l] * 4 / 64) % 4);
                    CHECK(quarters.size() == 4, "BN=%d kk=%d h=%d lanes %d..: rows share a 64-byte bank quarter", BN,
                          kk, h, g);
                }
            }
}

// Transposed reads for the 16x16x32 MFMA operand: lane l must get k = 32 kk +
// 8 (l / 16) + 4 h + e of column ncol0 + l % 16; each half-wave's 32 8-byte
// reads fall on 32 different 8-byte positions of a 256-byte LDS row.
template <int BN>
void check_n_tile16(int bk)
{
    for (int kk = 0; kk < bk / 32; ++kk)
        for (int ncol0 = 0; ncol0 < BN; ncol0 += 16)
            for (int h = 0; h < 2; ++h) {
                int lk[64], ln[64], off8[64];
                for (int l = 0; l < 64; ++l) {
                    const int off = nn_tr_offset16<BN>(l, kk, ncol0, h);
                    CHECK(off % 8 == 0 && off >= 0 && off + 8 <= bk * BN * 2, "BN=%d: tr16 read offset %d", BN, off);
                    off8[l] = (off / 8) % 32;
                    lk[l] = off / (BN * 2);
                    ln[l] = (((off % (BN * 2)) / 16) ^ nswz(lk[l])) * 8 + (off % 16) / 2;
                }
                for (int l = 0; l < 64; ++l) {
                    const int G = l / 16, i = l % 16;
                    for (int e = 0; e < 4; ++e) {
                        const int src = 16 * G + 4 * e + i / 4;
                        const int k = lk[src], n = ln[src] + i % 4;
                        CHECK(k == 32 * kk + 8 * G + 4 * h + e && n == ncol0 + i,
                              "BN=%d MF=16 kk=%d ncol0=%d h=%d lane %d elem %d: got (k=%d,n=%d)", BN, kk, ncol0, h, l,
                              e, k, n);
                    }
                }
                for (int g = 0; g < 64; g += 32) {
                    std::set<int> pos(off8 + g, off8 + g + 32);
                    CHECK(pos.size() == 32, "BN=%d MF=16 kk=%d ncol0=%d h=%d lanes %d..: 8-byte positions repeat", BN,
                          kk, ncol0, h, g);
                }
            }
}

// Epilogue strip of the 16x16x32 layout (16 rows x TN columns): the write of
// block g by lane l (row l % 16, columns 16 g + 4 (l / 16) .. +3) and the
// read-back (lane i of read j: chunk (64 j + i) % CH of row (64 j + i) / CH,
// halves swapped in odd rows) address the same bytes; the reads follow the
// bank rule (the writes' bank behaviour was measured on the GPU).
template <int TN>
void check_strip()
{
    const int CH = TN / 8;
    std::set<int> offs;
    for (int r = 0; r < 16; ++r)
        for (int c = 0; c < CH; ++c) {
            const int off = strip_offset<TN>(r, c);
            CHECK(off >= 0 && off + 16 <= 32 * TN && off % 16 == 0, "TN=%d strip offset", TN);
            offs.insert(off);
        }
    CHECK((int)offs.size() == 16 * CH, "TN=%d: strip chunks overlap", TN);
    for (int g = 0; g < TN / 16; ++g)
        for (int half = 0; half < 64; half += 32) {
            std::set<int> pos;
            for (int l = half; l < half + 32; ++l) {
                const int lr = l % 16, lh = l / 16;
                const int off = strip_half_offset<TN>(lr, 2 * g + (lh >> 1), lh & 1);
                // the read of logical chunk (16 g + 4 lh) / 8 of row lr finds these 8
                // bytes in its half (lh & 1) after the odd-row half swap
                const int col = 16 * g + 4 * lh;
                const int h_read = ((col % 8) / 4) ^ (lr & 1);
                CHECK(strip_offset<TN>(lr, col / 8) + 8 * h_read == off, "TN=%d: write/read mismatch", TN);
                pos.insert(off);
            }
            CHECK(pos.size() == 32, "TN=%d g=%d lanes %d..: strip writes overlap", TN, g, half);
        }
    for (int j = 0; j < CH / 4; ++j) {
        int addr[64];
        for (int l = 0; l < 64; ++l) {
            const int idx = 64 * j + l;
            addr[l] = strip_offset<TN>(idx / CH, idx % CH);
        }
        CHECK(b128_conflict_free(addr), "TN=%d read %d: bank conflict", TN, j);
    }
}

// Attention tiles: the copies' destinations match the reads; the V^T
// transposed reads deliver to lane l, slot j, the key attn_key_of_slot and
// column dcol0 + l mod 32; the S^T accumulator holds P in that same key order.
template <int BN, int D>
void check_attn()
{
    // K: every copied unit is where the operand reads look for it
    std::set<int> seen;
    for (int u = 0; u < BN * (D / 8); ++u) {
        int r = 0, c = 0;
        attn_k_unit<BN>(u, r, c);
        CHECK(r >= 0 && r < BN && c >= 0 && c < D / 8, "attn K unit %d: (%d,%d) outside the tile", u, r, c);
        CHECK(attn_k_offset<BN>(r, c) == u * 16, "attn K unit %d: written (%d,%d) read elsewhere", u, r, c);
        seen.insert(r * (D / 8) + c);
    }
    CHECK((int)seen.size() == BN * (D / 8), "attn K: units do not cover the tile");
    // V^T transposed reads
    for (int ks = 0; ks < BN / 16; ++ks)
        for (int dcol0 = 0; dcol0 < D; dcol0 += 32)
            for (int rr = 0; rr < 2; ++rr) {
                int lk[64], ln[64], word[64];
                for (int l = 0; l < 64; ++l) {
                    const int off = v_tr_offset<D>(l, ks, dcol0, rr);
                    CHECK(off % 8 == 0 && off >= 0 && off + 8 <= BN * D * 2, "attn V: tr read offset %d", off);
                    // the kernel puts the k-step's part in the read's offset field
                    CHECK(off == v_tr_offset<D>(l, 0, dcol0, rr) + 32 * D * ks,
                          "attn V: k-step %d does not move lane %d's read by 32 D ks bytes", ks, l);
                    word[l] = off / 4;
                    lk[l] = off / (D * 2);
                    ln[l] = (((off % (D * 2)) / 16) ^ nswz_w<D>(lk[l])) * 8 + (off % 16) / 2;
                }
                for (int l = 0; l < 64; ++l) {
                    const int G = l / 16, i = l % 16;
                    for (int e = 0; e < 4; ++e) {
                        const int src = 16 * G + 4 * e + i / 4;
                        const int k = lk[src], n = ln[src] + i % 4;
                        CHECK(k == attn_key_of_slot(l, ks, 4 * rr + e) && n == dcol0 + l % 32,
                              "attn V ks=%d dcol0=%d r=%d lane %d elem %d: got (k=%d,n=%d)", ks, dcol0, rr, l, e, k,
                              n);
                    }
                }
                // each half-wave's 32 reads of 8 bytes hit 32 distinct 8-byte bank pairs
                for (int g = 0; g < 64; g += 32) {
                    std::set<int> pairs;
                    for (int l = g; l < g + 32; ++l)
                        pairs.insert((word[l] / 2) % 32);
                    CHECK(pairs.size() == 32, "attn V D=%d ks=%d r=%d lanes %d..: %d of 32 bank pairs", D, ks, rr, g,
                          (int)pairs.size());
                }
            }
    // P: S^T accumulator element (kb, v) of lane l holds key 32 kb + 8 (v/4) + 4 (l/32) + v%4;
    // slot j of P fragment ks takes element v = 8 (ks % 2) + j of block kb = ks / 2
    for (int l = 0; l < 64; ++l)
        for (int ks = 0; ks < BN / 16; ++ks)
            for (int j = 0; j < 8; ++j) {
                const int kb = ks / 2, v = 8 * (ks % 2) + j;
                CHECK(32 * kb + 8 * (v / 4) + 4 * (l / 32) + v % 4 == attn_key_of_slot(l, ks, j),
                      "attn P lane %d ks %d slot %d", l, ks, j);
            }
}

// Epilogue staging buffer for strips of G output blocks.
void check_cbuf(int G)
{
    const int chunks = 4 * G, bytes = 32 * 64 * G;
    std::set<int> written;
    // every (row, column quad) lands in a distinct 8-byte slot inside the strip
    for (int r = 0; r < 32; ++r)
        for (int c = 0; c < chunks; ++c)
            for (int h = 0; h < 2; ++h) {
                const int off = cbuf_half_offset(r, c, h, G);
                CHECK(off >= 0 && off + 8 <= bytes && off % 8 == 0, "G=%d: half offset %d", G, off);
                CHECK(written.insert(off).second, "G=%d: (%d,%d,%d) overlaps", G, r, c, h);
                // the read of logical chunk c of row r finds this half at 8 (h ^ hswz(r))
                CHECK(cbuf_chunk_offset(r, c, G) + 8 * (h ^ hswz(r)) == off, "G=%d: read/write mismatch", G);
            }
    // writes: lane l of a 16-lane group writes row (l mod 32) at one logical
    // (chunk, half); 16 lanes x 8 bytes must hit 16 distinct 8-byte bank pairs
    for (int c = 0; c < chunks; ++c)
        for (int h = 0; h < 2; ++h)
            for (int g = 0; g < 64; g += 16) {
                std::set<int> slots;
                for (int l = g; l < g + 16; ++l)
                    slots.insert((cbuf_half_offset(l % 32, c, (l / 32) ^ h, G) / 8) % 16);
                CHECK(slots.size() == 16, "G=%d c=%d h=%d lanes %d..: epilogue write bank conflict", G, c, h, g);
            }
    // reads: lane i reads 16 bytes of row i / chunks; 8 lanes per LDS cycle
    for (int base = 0; base < 32 * chunks; base += 64)
        for (int g = 0; g < 64; g += 8) {
            std::set<int> units;
            for (int i = base + g; i < base + g + 8; ++i)
                units.insert((cbuf_chunk_offset(i / chunks, i % chunks, G) / 16) % 8);
            CHECK(units.size() == 8, "G=%d lanes %d..: epilogue read bank conflict", G, base + g);
        }
    // block choice
    CHECK(cbuf_blocks(4, 8192) == 4 && cbuf_blocks(4, 6144) == 2 && cbuf_blocks(1, 2048) == 1 &&
              cbuf_blocks(2, 16384) == 2,
          "cbuf_blocks");
}

// Simulates the kernel's copy schedule piece by piece (every 1 KiB copy of a
// wave, in issue order) for the three placements, and checks that a slot is
// refilled only after its tile was read, that every wait leaves exactly the
// copies issued after the awaited tile in flight, that each tile is read from
// the slots its copies went to, and the 63-copy vmcnt bound.
void check_ring_case(int S, int lead, int la, int lb, int ks, int nk, bool early_wanted)
{
    const bool early = ring_early_b(S, lead, early_wanted);
    const int SA = S + lead;
    struct Slot {
        int tile = -1;
        bool read = true;
    };
    std::vector<Slot> a_slots(SA), b_slots(S);
    std::vector<int> last_a(nk + 2 * S + 4, -1), last_b(nk + 2 * S + 4, -1);  // index of a tile's last piece
    int issued = 0, completed = 0, max_flight = 0;
    int next_a = 0, next_b = 0;  // copies go out in tile order per operand
    auto put = [&](std::vector<Slot> &ring, int t, bool is_a) {
        Slot &sl = ring[ring_slot(t, is_a ? SA : S)];
        if (sl.tile != t) {
            CHECK(sl.tile < 0 || sl.tile >= nk || sl.read, "S=%d lead=%d nk=%d: %s tile %d overwrites unread tile %d",
                  S, lead, nk, is_a ? "A" : "B", t, sl.tile);
            sl.tile = t;
            sl.read = false;
        }
        (is_a ? last_a : last_b)[t] = issued++;
        max_flight = std::max(max_flight, issued - completed);
    };
    auto issue_a = [&](int t, int first, int last) {
        for (int i = first; i < last; ++i) {
            if (i == 0) {
                CHECK(t == next_a, "S=%d lead=%d: A tile %d issued out of order", S, lead, t);
                ++next_a;
            }
            put(a_slots, t, true);
        }
    };
    auto issue_b = [&](int t, int first, int last) {
        for (int i = first; i < last; ++i) {
            if (i == 0) {
                CHECK(t == next_b, "S=%d lead=%d: B tile %d issued out of order", S, lead, t);
                ++next_b;
            }
            put(b_slots, t, false);
        }
    };
    auto wait_for = [&](int j, int allowed) {
        const int last = std::max(last_a[j], last_b[j]);
        CHECK(last >= 0, "S=%d lead=%d nk=%d: tile %d never issued", S, lead, nk, j);
        CHECK(allowed == issued - 1 - last, "S=%d lead=%d la=%d lb=%d nk=%d: wait for tile %d allows %d, %d after it",
              S, lead, la, lb, nk, j, allowed, issued - 1 - last);
        completed = std::max(completed, issued - allowed);
        CHECK(a_slots[ring_slot(j, SA)].tile == j && b_slots[ring_slot(j, S)].tile == j,
              "S=%d lead=%d nk=%d: tile %d not in its slots", S, lead, nk, j);
    };
    const bool spread = ring_spread(S, lead);
    for (int t = 0; t < ring_prologue(S, lead); ++t) {
        issue_a(t, 0, la);
        issue_b(t, 0, lb);
    }
    if (lead)
        issue_a(S - 1, 0, la);
    wait_for(0, ring_wait_first(S, lead, la, lb));
    if (early)  // after the first barrier: the B copies iteration 0 would issue
        issue_b(ring_issue_tile_b(0, S, lead), 0, lb);
    for (int j = 0; j < nk; ++j) {
        const int ta = ring_issue_tile_a(j, S, lead), tb = ring_issue_tile_b(j, S, lead);
        for (int kk = 0; kk < ks; ++kk) {
            if (spread) {
                const int a0 = copy_a_before(kk, ks, la, lb, lead), a1 = copy_a_before(kk + 1, ks, la, lb, lead);
                const int b0 = copy_b_before(kk, ks, la, lb, lead), b1 = copy_b_before(kk + 1, ks, la, lb, lead);
                CHECK(a0 <= a1 && b0 <= b1, "plan not monotone");
                if (lead) {
                    if (!early)
                        issue_b(tb, b0, b1);
                    issue_a(ta, a0, a1);
                } else {
                    issue_a(ta, a0, a1);
                    issue_b(tb, b0, b1);
                }
            }
            if (kk == ks - 1) {
                // every LDS read of tile j has returned
                a_slots[ring_slot(j, SA)].read = true;
                b_slots[ring_slot(j, S)].read = true;
            }
        }
        if (spread)
            CHECK(copy_a_before(ks, ks, la, lb, lead) == la && copy_b_before(ks, ks, la, lb, lead) == lb &&
                      copy_a_before(0, ks, la, lb, lead) == 0 && copy_b_before(0, ks, la, lb, lead) == 0,
                  "plan does not cover the tile");
        wait_for(j + 1, ring_wait_steady(S, lead, la, lb));
        // barrier
        if (early)  // B of the tile iteration j+1 would issue, into tile j's freed slot
            issue_b(tb + 1, 0, lb);
        if (!spread) {
            CHECK(ta == tb && ring_slot(ta, SA) == ring_slot(j, SA), "burst refills the freed slots");
            issue_a(ta, 0, la);
            issue_b(tb, 0, lb);
        }
    }
    if (ring_fits_vmcnt(S, lead, la, lb))
        CHECK(max_flight <= 63, "S=%d lead=%d la=%d lb=%d: %d copies in flight", S, lead, la, lb, max_flight);
}

void check_ring()
{
    const int loads[][2] = {{1, 1}, {2, 2}, {4, 4}, {8, 8}, {4, 8}, {8, 4}, {2, 6}, {3, 5}};
    for (int S = 2; S <= 10; ++S)
        for (int lead = 0; lead <= 1; ++lead)
            for (auto &l : loads)
                for (int ks : {1, 2, 4})  // k-steps per tile: BK / 16 (32x32x16) or BK / 32 (16x16x32)
                    for (int nk = 0; nk <= 24; ++nk)
                        for (bool early : {false, true})
                            check_ring_case(S, lead, l[0], l[1], ks, nk, early);
    for (int n = 1; n <= 32; ++n)
        CHECK((ring_max_stages(n) - 1) * n <= 63 && ring_max_stages(n) * n > 63, "ring_max_stages(%d)", n);
    // the ring depths the kernel builds: B ring S, A ring S + lead
    CHECK(ring_lds_bytes(2, 1, 32768, 32768) == 160 * 1024, "256x256x64 S=2 lead fills 160 KiB");
    CHECK(ring_lds_bytes(3, 0, 16384, 16384) == 3 * 32768, "no-lead ring is S stages");
}

// The workgroup -> C tile map is a bijection of 0 .. tiles_m tiles_n - 1 onto
// the grid, for every grid up to 64 x 64 tiles (group_m = min(tiles_m, 4), as
// the host sets it), which covers the 4096^3 grids at 256 x 256 (16 x 16) and
// 128 x 128 (32 x 32) and the 4000 x 5000 grids (16 x 20, 32 x 40).  Also:
// each XCD (id mod 8) receives consecutive renumbered ids, so with the
// 4096^3 grid at 256 x 256 an XCD's 32 tiles form a 4 x 8 block (4 A panels,
// 8 B panels).
void check_map_tile()
{
    std::vector<int> seen;
    for (int tm_n = 1; tm_n <= 64; ++tm_n)
        for (int tn_n = 1; tn_n <= 64; ++tn_n) {
            const int gm = tm_n < 4 ? tm_n : 4;
            seen.assign(tm_n * tn_n, 0);
            for (int bid = 0; bid < tm_n * tn_n; ++bid) {
                int tm = -1, tn = -1;
                map_tile(bid, tm_n, tn_n, gm, tm, tn);
                if (tm < 0 || tm >= tm_n || tn < 0 || tn >= tn_n) {
                    CHECK(false, "map_tile %dx%d: workgroup %d -> (%d,%d) outside the grid", tm_n, tn_n, bid, tm, tn);
                    continue;
                }
                ++seen[tm * tn_n + tn];
            }
            for (int t = 0; t < tm_n * tn_n; ++t)
                CHECK(seen[t] == 1, "map_tile %dx%d: tile (%d,%d) owned by %d workgroups", tm_n, tn_n, t / tn_n,
                      t % tn_n, seen[t]);
        }
    // the XCD blocks of the 4096^3 grid at 256 x 256
    for (int x = 0; x < 8; ++x) {
        std::set<int> rows, cols;
        for (int bid = x; bid < 256; bid += 8) {
            int tm = 0, tn = 0;
            map_tile(bid, 16, 16, 4, tm, tn);
            rows.insert(tm);
            cols.insert(tn);
        }
        CHECK(rows.size() == 4 && cols.size() == 8, "XCD %d of the 16x16 grid spans %zu tile rows and %zu tile "
              "columns, not 4 x 8", x, rows.size(), cols.size());
    }
}

// Attention work items: every (head row, query block) goes to exactly one
// workgroup, with and without the mask.  Causal: the first B H ids take the
// last query block of every head.  Without the mask, when B H is a multiple
// of 8, all blocks of a head land on one XCD (id mod 8), e.g. 16 whole heads
// per XCD at 4 x 32 heads and 16 query blocks.
void check_attn_map()
{
    std::vector<int> seen;
    for (int bhs = 1; bhs <= 48; ++bhs)
        for (int nq = 1; nq <= 40; ++nq)
            for (int causal = 0; causal < 2; ++causal) {
                seen.assign(bhs * nq, 0);
                for (int bid = 0; bid < bhs * nq; ++bid) {
                    int bh = -1, qb = -1;
                    attn_work_item(bid, bhs, nq, causal != 0, bh, qb);
                    if (bh < 0 || bh >= bhs || qb < 0 || qb >= nq) {
                        CHECK(false, "attn_work_item(%d, %d, %d, %d) -> (%d,%d) outside", bid, bhs, nq, causal, bh, qb);
                        continue;
                    }
                    ++seen[bh * nq + qb];
                    if (causal && bid < bhs)
                        CHECK(qb == nq - 1, "causal id %d of %d x %d does not take a last query block", bid, bhs, nq);
                }
                for (int t = 0; t < bhs * nq; ++t)
                    CHECK(seen[t] == 1, "attn work item (%d,%d) of %d x %d (causal %d) owned by %d workgroups",
                          t / nq, t % nq, bhs, nq, causal, seen[t]);
                if (!causal && bhs % 8 == 0)
                    for (int bh = 0; bh < bhs; ++bh) {
                        std::set<int> xcds;
                        for (int bid = 0; bid < bhs * nq; ++bid) {
                            int b2 = 0, q2 = 0;
                            attn_work_item(bid, bhs, nq, false, b2, q2);
                            if (b2 == bh)
                                xcds.insert(bid % 8);
                        }
                        CHECK(xcds.size() == 1, "head row %d of %d x %d spans %zu XCDs", bh, bhs, nq, xcds.size());
                    }
            }
}

// Epilogue batches: a divisor of FM that fits, and the largest such.
void check_epi_batch()
{
    for (int fm = 1; fm <= 16; ++fm)
        for (int fit = 0; fit <= 20; ++fit) {
            const int nf = epi_batch(fm, fit);
            CHECK(nf >= 1 && fm % nf == 0, "epi_batch(%d,%d) = %d does not divide", fm, fit, nf);
            CHECK(nf == 1 || nf <= fit, "epi_batch(%d,%d) = %d does not fit", fm, fit, nf);
            for (int d = nf + 1; d <= fm && d <= fit; ++d)
                CHECK(fm % d != 0, "epi_batch(%d,%d) = %d, but %d also fits", fm, fit, nf, d);
        }
}

int main()
{
    check_map_tile();
    check_attn_map();
    check_epi_batch();
    check_k_tile<32>(256);
    check_k_tile<64>(256);
    check_k_tile<64>(64);
    check_n_tile<128>(32);
    check_n_tile<128>(64);
    check_n_tile<256>(32);
    check_n_tile<256>(64);
    check_n_tile16<128>(32);
    check_n_tile16<128>(64);
    check_n_tile16<256>(32);
    check_n_tile16<256>(64);
    check_strip<32>();
    check_strip<64>();
    check_strip<128>();
    check_ring();
    check_attn<64, 128>();
    check_attn<128, 128>();
    check_attn<64, 64>();
    check_attn<128, 64>();
    check_cbuf(1);
    check_cbuf(2);
    check_cbuf(4);
    if (failures) {
        std::printf("%d failures\n", failures);
        return 1;
    }
    std::printf("layout and schedule invariants: OK\n");
    return 0;
}
