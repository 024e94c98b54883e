// Which (batch x head, query block) an attention workgroup computes, from its
// id in the launch.  Shared by the kernel and the host-side layout checks.
#pragma once

#include "pipegemm_layout.hpp"  // PG_HD

namespace pipegemm {

// bhs = batch x heads work rows, nq query blocks per head; bid < bhs nq.
//
// With the causal mask, query block q sees q + 1 key tiles of block_M keys at
// most, so the blocks differ in work by up to nq times.  The ids then go out
// longest first over every head (ids 0 .. bhs - 1 take the last query block
// of each head, the next bhs the one before, and so on), and the short blocks
// fill the compute units at the end.
//
// Without a mask every block costs the same.  Workgroup ids are dealt to the
// 8 XCDs round-robin (id mod 8), so the ids are renumbered to give each XCD a
// contiguous run of the head-major work list: all query blocks of a head then
// run on one XCD at about the same time and read the head's K and V tiles
// through that XCD's L2, instead of every XCD streaming every head.  Query
// heads that share a KV head are adjacent in the list, so they share too.
PG_HD inline void attn_work_item(int bid, int bhs, int nq, bool causal, int &bh, int &qblk)
{
    if (causal) {
        qblk = nq - 1 - bid / bhs;
        bh = bid % bhs;
        return;
    }
    const int n = bhs * nq, x = bid % 8, per = n / 8, rem = n % 8;
    const int item = x * per + (x < rem ? x : rem) + bid / 8;
    bh = item / nq;
    qblk = nq - 1 - item % nq;
}

}  // namespace pipegemm
