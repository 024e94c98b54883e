// Interface between the host code (pipegemm.hip) and the attention kernel
// translation units (attn_kernels.hip, compiled once per dtype).
#pragma once

#include <hip/hip_runtime.h>

namespace pipegemm {

struct AttnArgs;

// Launch attn_kernel<T, AttnTile<BN, WAVES>> on `stream`.
template <class T, int BN, int WAVES>
hipError_t attn_launch(const AttnArgs &args, int grid, int lds_bytes, hipStream_t stream);

constexpr int kAttnMaxStages = 4;

// The built attention tiles: X(block_N, waves).
#define PG_ATTN_TILE_LIST(X) \
    X(64, 4)                 \
    X(64, 8)                 \
    X(128, 4)

}  // namespace pipegemm
