// Interface between the host table (pipegemm.hip) and the kernel translation
// units (pipegemm_kernels.hip, compiled once per dtype and B layout).
#pragma once

#include <hip/hip_runtime.h>

namespace pipegemm {

struct KernelArgs;

// Deepest LDS ring any built kernel accepts.  The smallest built stage is
// 128 x 128 x 32 (16 KiB), so no deeper ring fits gfx950's 160 KiB anyway.
constexpr int kMaxStages = 10;

// Launch gemm_kernel<T, NN, Tile<BM, BN, BK, WM, WN>, KCHECK> on `stream` with
// `grid` workgroups and `lds_bytes` of dynamic LDS.  KCHECK: K is not a
// multiple of BK.
template <class T, bool NN, int BM, int BN, int BK, int WM, int WN, bool KCHECK>
hipError_t launch(const KernelArgs &args, int grid, int lds_bytes, hipStream_t stream);

// 1 KiB copies each wave issues per K tile (bounds the copy wait, 63 loads);
// loads_per_wave(bm, 0, bk, w) counts the A tile's alone, (0, bn, bk, w) B's.
constexpr int loads_per_wave(int bm, int bn, int bk, int waves)
{
    return (bm + bn) * bk * 2 / (1024 * waves);
}

// The built tile shapes: X(block_M, block_N, block_K, waves along M, waves along N).
#define PG_TILE_LIST(X)            \
    X(64, 128, 64, 2, 2)           \
    X(128, 128, 32, 2, 1)          \
    X(128, 128, 32, 2, 2)          \
    X(128, 128, 32, 2, 4)          \
    X(128, 128, 64, 2, 2)          \
    X(128, 128, 64, 2, 4)          \
    X(128, 256, 32, 2, 2)          \
    X(128, 256, 64, 2, 2)          \
    X(128, 256, 64, 2, 4)          \
    X(256, 128, 32, 2, 2)          \
    X(256, 128, 32, 4, 2)          \
    X(256, 128, 64, 2, 2)          \
    X(256, 256, 32, 2, 2)          \
    X(256, 256, 32, 2, 4)          \
    X(256, 256, 64, 2, 2)          \
    X(256, 256, 64, 2, 4)

}  // namespace pipegemm
