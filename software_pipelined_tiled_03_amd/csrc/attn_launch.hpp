// Interface between the host code (pipegemm.hip) and the attention kernel
// translation units (attn_kernels.hip, compiled once per dtype).
#pragma once

#include <hip/hip_runtime.h>

namespace pipegemm {

struct AttnArgs;

// Launch attn_kernel<T, AttnTile<BN, WAVES, QB, D>> on `stream`.
template <class T, int BN, int WAVES, int QB, int D>
hipError_t attn_launch(const AttnArgs &args, int grid, int lds_bytes, hipStream_t stream);

constexpr int kAttnMaxStages = 4;

// The built attention tiles: X(block_N, waves, 32-query blocks per wave, head
// dimension); block_M = 32 x blocks x waves.
#define PG_ATTN_TILE_LIST(X) \
    X(64, 4, 1, 128)         \
    X(64, 8, 1, 128)         \
    X(128, 4, 1, 128)        \
    X(128, 8, 1, 128)        \
    X(64, 4, 2, 128)         \
    X(64, 4, 1, 64)          \
    X(64, 8, 1, 64)          \
    X(128, 4, 1, 64)         \
    X(128, 8, 1, 64)         \
    X(64, 4, 2, 64)          \
    X(64, 8, 2, 64)          \
    X(128, 8, 2, 64)

}  // namespace pipegemm
