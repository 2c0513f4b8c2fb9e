// misc_i8.hip -- launches of the int8 path's row quantizer, per-column
// factors and split-K epilogue.
#include "kernels_i8.h"

namespace qg {

hipError_t launch_i8_reduce(int dtype, const int *part, const float *sx, const float *sw, uint16_t *Y, int M, int N,
                            long long stride, int S, hipStream_t s)
{
    const long long MN = (long long)M * N;
    const dim3 grid((unsigned)(((MN + 3) / 4 + 255) / 256));
    if (dtype == DT_F16)
        hipLaunchKernelGGL((k_i8_splitk_reduce<DT_F16>), grid, dim3(256), 0, s, part, sx, sw, Y, M, N, stride, S);
    else
        hipLaunchKernelGGL((k_i8_splitk_reduce<DT_BF16>), grid, dim3(256), 0, s, part, sx, sw, Y, M, N, stride, S);
    return hipGetLastError();
}

hipError_t launch_i8_quant(int dtype, const uint16_t *X, uint8_t *Xq, float *sx, int M, int K, hipStream_t s)
{
    const unsigned groups = (unsigned)(((long long)M + 31) / 32 * 8);  // four padded rows per workgroup
    if (dtype == DT_F16) hipLaunchKernelGGL((k_i8_quant<DT_F16>), dim3(groups), dim3(256), 0, s, X, Xq, sx, M, K);
    else hipLaunchKernelGGL((k_i8_quant<DT_BF16>), dim3(groups), dim3(256), 0, s, X, Xq, sx, M, K);
    return hipGetLastError();
}

hipError_t launch_i8_colscale(int fmt, const Args &a, float *rw, float *sw, hipStream_t s)
{
    const dim3 grid((unsigned)a.np);
    if (fmt == FMT_Q4K) hipLaunchKernelGGL((k_i8_colscale<FMT_Q4K>), grid, dim3(64), 0, s, a, rw, sw);
    else if (fmt == FMT_Q6K) hipLaunchKernelGGL((k_i8_colscale<FMT_Q6K>), grid, dim3(64), 0, s, a, rw, sw);
    else hipLaunchKernelGGL((k_i8_colscale<FMT_W4>), grid, dim3(64), 0, s, a, rw, sw);
    return hipGetLastError();
}

}  // namespace qg
