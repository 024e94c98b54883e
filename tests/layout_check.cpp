// Host-side check of the LDS layouts and the ring schedule the GPU kernel uses
// (software_pipelined_tiled_03_amd/csrc/pipegemm_layout.hpp), by enumeration:
//  1. every 16-byte unit the direct-to-LDS copy writes lands where the MFMA
//     operand reads look for it (K-contiguous and N-contiguous tiles);
//  2. the transposed reads of the NN form deliver, lane by lane, exactly the
//     k / n elements the 32x32x16 MFMA operand needs;
//  3. the operand reads are free of LDS bank conflicts;
//  4. over a ring of S slots, each tile's wait covers its own copy exactly, and
//     no slot is overwritten while a tile in it is still to be read.
// Prints one line per failure and exits non-zero on any.
#include <cstdio>
#include <set>

#include "pipegemm_layout.hpp"

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

void check_ring()
{
    for (int S = 2; S <= 10; ++S)
        for (int nk = 0; nk <= 40; ++nk) {
            int slot_tile[16];
            bool slot_read[16];
            for (int s = 0; s < 16; ++s) {
                slot_tile[s] = -1;
                slot_read[s] = true;
            }
            int issued = 0, real = 0;
            auto issue = [&](int t) {
                const int s = ring_slot(t, S);
                // a slot holding a real tile is refilled only after it was read
                CHECK(slot_tile[s] < 0 || slot_tile[s] >= nk || slot_read[s],
                      "S=%d nk=%d: tile %d overwrites unread tile %d", S, nk, t, slot_tile[s]);
                CHECK(t == issued, "S=%d nk=%d: tiles issued out of order (%d, expected %d)", S, nk, t, issued);
                slot_tile[s] = t;
                slot_read[s] = false;
                ++issued;
                real += t < nk;
            };
            // the wait for tile j is exact: it lets precisely the tiles issued
            // after j stay in flight (copies complete in issue order)
            auto wait_for = [&](int j, int allowed) {
                CHECK(allowed == issued - 1 - j, "S=%d nk=%d: wait for tile %d allows %d, issued after it %d", S, nk,
                      j, allowed, issued - 1 - j);
                CHECK(slot_tile[ring_slot(j, S)] == j, "S=%d nk=%d: slot of tile %d holds %d", S, nk, j,
                      slot_tile[ring_slot(j, S)]);
            };
            for (int t = 0; t < ring_prologue(S); ++t)
                issue(t);
            wait_for(0, ring_wait_first(S));
            for (int j = 0; j < nk; ++j) {
                CHECK(slot_tile[ring_slot(j, S)] == j, "S=%d nk=%d: tile %d not in its slot", S, nk, j);
                if (ring_spread(S)) {
                    // spread copies go out during iteration j, before its wait,
                    // into the slot the previous barrier freed
                    CHECK(ring_slot(ring_issue_tile(j, S), S) == ring_slot(j + S - 1, S), "spread slot");
                    issue(ring_issue_tile(j, S));
                }
                slot_read[ring_slot(j, S)] = true;  // every LDS read of tile j has returned
                wait_for(j + 1, ring_wait_steady(S));
                // barrier
                if (!ring_spread(S)) {
                    CHECK(ring_slot(ring_issue_tile(j, S), S) == ring_slot(j, S), "burst refills the freed slot");
                    issue(ring_issue_tile(j, S));
                }
            }
            CHECK(real == nk, "S=%d nk=%d: %d real tiles issued", S, nk, real);
        }
    for (int loads = 1; loads <= 32; ++loads)
        CHECK((ring_max_stages(loads) - 1) * loads <= 63 && ring_max_stages(loads) * loads > 63,
              "ring_max_stages(%d)", loads);
}

int main()
{
    check_k_tile<32>(256);
    check_k_tile<64>(256);
    check_n_tile<128>(32);
    check_n_tile<128>(64);
    check_n_tile<256>(32);
    check_n_tile<256>(64);
    check_ring();
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
