// misc_grouped.hip -- launches of the grouped per-expert GEMM kernels.
#include "kernels_fp.h"

namespace qg {

template <int FMT, int DT, int XL>
hipError_t launch_grouped_t(const Plan &pl, const Args &a, hipStream_t s)
{
    if (pl.rung == GROUPED_SHARED) {
        if (pl.pn != 2 || pl.waves != 4 || (pl.rb != 2 && pl.rb != 5)) return hipErrorInvalidValue;
        if (pl.rb == 2) hipLaunchKernelGGL((k_grouped_shared<FMT, DT, 2, 2, 4, XL>), pl.grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_grouped_shared<FMT, DT, 5, 2, 4, XL>), pl.grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    if (pl.pn != 4 || (pl.rb != 1 && pl.rb != 2)) return hipErrorInvalidValue;
    if (pl.rb == 1) hipLaunchKernelGGL((k_direct_grouped<FMT, DT, 1, 4, XL>), pl.grid, dim3(64 * pl.kw), pl.lds, s, a);
    else hipLaunchKernelGGL((k_direct_grouped<FMT, DT, 2, 4, XL>), pl.grid, dim3(64 * pl.kw), pl.lds, s, a);
    return hipGetLastError();
}

template <int FMT, int DT>
hipError_t launch_grouped_l(int xl, const Plan &pl, const Args &a, hipStream_t s)
{
    return xl == X_FRAG ? launch_grouped_t<FMT, DT, X_FRAG>(pl, a, s) : launch_grouped_t<FMT, DT, X_ROW>(pl, a, s);
}

hipError_t launch_grouped(int fmt, int dtype, int xl, const Plan &pl, const Args &a, hipStream_t s)
{
    if (fmt == FMT_Q4K)
        return dtype == DT_F16 ? launch_grouped_l<FMT_Q4K, DT_F16>(xl, pl, a, s)
                               : launch_grouped_l<FMT_Q4K, DT_BF16>(xl, pl, a, s);
    if (fmt == FMT_Q6K)
        return dtype == DT_F16 ? launch_grouped_l<FMT_Q6K, DT_F16>(xl, pl, a, s)
                               : launch_grouped_l<FMT_Q6K, DT_BF16>(xl, pl, a, s);
    return dtype == DT_F16 ? launch_grouped_l<FMT_W4, DT_F16>(xl, pl, a, s) : launch_grouped_l<FMT_W4, DT_BF16>(xl, pl, a, s);
}

}  // namespace qg
