// misc_grouped.hip -- launches of the grouped per-expert GEMM kernels.
#include "kernels_fp.h"

namespace qg {

template <int FMT, int DT, int XL>
hipError_t launch_grouped_fd(const Plan &pl, const Args &a, hipStream_t s)
{
    if (pl.rb == 1) hipLaunchKernelGGL((k_direct_grouped<FMT, DT, 1, 4, XL>), pl.grid, dim3(64 * pl.kw), pl.lds, s, a);
    else hipLaunchKernelGGL((k_direct_grouped<FMT, DT, 2, 4, XL>), pl.grid, dim3(64 * pl.kw), pl.lds, s, a);
    return hipGetLastError();
}

// 64x64 streaming tiles, two waves per workgroup over all of K (splitting K
// inside the workgroup measured slower: too few chunks per group at an
// expert's K, 98-103 against 80-81 us); row slots dealt to the XCDs in turn.
template <int FMT, int DT, int XL>
hipError_t launch_grouped_stream(const Args &a, long long T, long long E, hipStream_t s)
{
    const long long tn = (a.np + 3) / 4, slots = (T + 63) / 64 + E;
    const dim3 grid((unsigned)(tn * ((slots + 7) / 8) * 8));
    hipLaunchKernelGGL((k_stream32_grouped<FMT, DT, 1, XL>), grid, dim3(128), 0, s, a);
    return hipGetLastError();
}

template <int FMT, int DT>
hipError_t launch_grouped_t(int xl, bool stream_tiles, const Plan &pl, const Args &a, long long T, long long E,
                            hipStream_t s)
{
    if (xl == X_FRAG)
        return stream_tiles ? launch_grouped_stream<FMT, DT, X_FRAG>(a, T, E, s) : launch_grouped_fd<FMT, DT, X_FRAG>(pl, a, s);
    return stream_tiles ? launch_grouped_stream<FMT, DT, X_ROW>(a, T, E, s) : launch_grouped_fd<FMT, DT, X_ROW>(pl, a, s);
}

hipError_t launch_grouped(int fmt, int dtype, int xl, bool stream_tiles, const Plan &pl, const Args &a, long long T,
                          long long E, hipStream_t s)
{
    if (fmt == FMT_Q4K)
        return dtype == DT_F16 ? launch_grouped_t<FMT_Q4K, DT_F16>(xl, stream_tiles, pl, a, T, E, s)
                               : launch_grouped_t<FMT_Q4K, DT_BF16>(xl, stream_tiles, pl, a, T, E, s);
    if (fmt == FMT_Q6K)
        return dtype == DT_F16 ? launch_grouped_t<FMT_Q6K, DT_F16>(xl, stream_tiles, pl, a, T, E, s)
                               : launch_grouped_t<FMT_Q6K, DT_BF16>(xl, stream_tiles, pl, a, T, E, s);
    return dtype == DT_F16 ? launch_grouped_t<FMT_W4, DT_F16>(xl, stream_tiles, pl, a, T, E, s)
                           : launch_grouped_t<FMT_W4, DT_BF16>(xl, stream_tiles, pl, a, T, E, s);
}

}  // namespace qg
