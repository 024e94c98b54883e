// Attention kernel instantiations for one element type (PG_ELEM).
#include "attn_kernel.hpp"
#include "attn_launch.hpp"
#include "launch_util.hpp"

#ifndef PG_ELEM
#error "PG_ELEM must name the element type"
#endif

namespace pipegemm {

template <class T, int BN, int WAVES, int QB, int D>
hipError_t attn_launch(const AttnArgs &args, int grid, int lds_bytes, hipStream_t stream)
{
    using Cfg = AttnTile<BN, WAVES, QB, D>;
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t attr_err = allow_full_lds((const void *)&attn_kernel<T, Cfg>, lds_set);
    if (attr_err != hipSuccess)
        return attr_err;
    hipLaunchKernelGGL((attn_kernel<T, Cfg>), dim3(grid), dim3(Cfg::THREADS), lds_bytes, stream, args);
    return hipGetLastError();
}

#define PG_ATTN_INSTANTIATE(BN, W, QB, D) \
    template hipError_t attn_launch<PG_ELEM, BN, W, QB, D>(const AttnArgs &, int, int, hipStream_t);
PG_ATTN_TILE_LIST(PG_ATTN_INSTANTIATE)
#undef PG_ATTN_INSTANTIATE

}  // namespace pipegemm
