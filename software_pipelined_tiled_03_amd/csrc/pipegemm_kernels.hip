// Kernel instantiations for one (element type, B layout, K bound) triple,
// selected by PG_ELEM (_Float16 or __bf16), PG_NN (0 = NT, 1 = NN) and
// PG_KCHECK (1 = the per-chunk K bound of a ragged last K tile) at compile time.
#include "pipegemm_kernel.hpp"
#include "launch_util.hpp"
#include "pipegemm_launch.hpp"

#ifndef PG_ELEM
#error "PG_ELEM must name the element type"
#endif
#ifndef PG_NN
#error "PG_NN must be 0 or 1"
#endif
#ifndef PG_KCHECK
#error "PG_KCHECK must be 0 or 1"
#endif

namespace pipegemm {

template <class T, bool NN, int BM, int BN, int BK, int WM, int WN, bool KCHECK>
hipError_t launch(const KernelArgs &args, int grid, int lds_bytes, hipStream_t stream)
{
    using Cfg = Tile<BM, BN, BK, WM, WN>;
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t attr_err = allow_full_lds((const void *)&gemm_kernel<T, NN, Cfg, KCHECK>, lds_set);
    if (attr_err != hipSuccess)
        return attr_err;
    hipLaunchKernelGGL((gemm_kernel<T, NN, Cfg, KCHECK>), dim3(grid), dim3(Cfg::THREADS), lds_bytes, stream, args);
    return hipGetLastError();
}

#define PG_INSTANTIATE(BM, BN, BK, WM, WN)                                                                   \
    template hipError_t launch<PG_ELEM, (PG_NN != 0), BM, BN, BK, WM, WN, (PG_KCHECK != 0)>(const KernelArgs &, \
                                                                                            int, int, hipStream_t);
PG_TILE_LIST(PG_INSTANTIATE)
#undef PG_INSTANTIATE

}  // namespace pipegemm
