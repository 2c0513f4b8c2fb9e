// misc.hip -- the single-purpose kernels around the GEMM: the split-K
// reduction, the logical dequant, the staged arm (unpack pass + the 128x128
// streaming kernel on its scratch) and the fragment-major copy of X.
#include "kernels_fp.h"

namespace qg {

// ---------------------------------------------------------------------------
// Logical dequant: the same unpack, written out as W[K][N] (row-major).
// One thread per (panel, chunk, run, column).
// ---------------------------------------------------------------------------
template <int FMT, int DT>
__global__ void __launch_bounds__(256) k_dequant(Args a, uint16_t *Wout)
{
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int nch = a.K / kChunk;
    const long long total = (long long)a.np * nch * 64;
    if (idx >= total) return;
    const int lane = (int)(idx & 63), col = lane & 15, g = lane >> 4;
    const long long pc = idx >> 6;
    const int c = (int)(pc % nch), p = (int)(pc / nch);
    const int n = 16 * p + col;
    RunSrc<FMT> src;
    src.init(a, p, g, col);
    RunRaw<FMT> raw;
    src.load(c, raw);
    u32x4 f[4];
    unpack_run<FMT, DT>(raw, src, c, f);
    if (n >= a.N) return;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const long long k = (long long)kChunk * c + 32 * g + 8 * i + 2 * j;
            Wout[k * a.N + n] = (uint16_t)(f[i][j] & 0xFFFFu);
            Wout[(k + 1) * a.N + n] = (uint16_t)(f[i][j] >> 16);
        }
}

// ---------------------------------------------------------------------------
// Staged arm, step one: the same unpack, written to a scratch buffer in the
// order the streaming kernel reads it (the FMT_DENSE layout): one thread per
// (panel, chunk, run); a wave's four 16-byte stores are four contiguous
// kilobytes.  Step two is k_stream32<FMT_DENSE, ...> on that scratch.
// ---------------------------------------------------------------------------
template <int FMT, int DT>
__global__ void __launch_bounds__(256) k_stage(Args a, uint8_t *Ws)
{
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int nch = a.K / kChunk;
    const long long total = (long long)a.np * nch * 64;
    if (idx >= total) return;
    const int run = (int)(idx & 63), col = run & 15, g = run >> 4;
    const long long pc = idx >> 6;  // = panel * nch + chunk
    const int c = (int)(pc % nch), p = (int)(pc / nch);
    RunSrc<FMT> src;
    src.init(a, p, g, col);
    RunRaw<FMT> raw;
    src.load(c, raw);
    u32x4 f[4];
    unpack_run<FMT, DT>(raw, src, c, f);
    u32x4 *dst = reinterpret_cast<u32x4 *>(Ws + pc * 4096) + run;
#pragma unroll
    for (int i = 0; i < 4; i++) dst[64 * i] = f[i];
}

// ---------------------------------------------------------------------------
// Fragment-major copy of X (layout X_FRAG).  One workgroup per (32-row block,
// 128-wide chunk), which is 8 KB in both layouts; each thread moves two
// 16-byte units (8 consecutive k of one row), read row-major, 16 lanes per
// row, and written to their fragment slot.  Rows at or past M become zeros.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_x_to_xf(const uint16_t *X, uint16_t *Xf, int M, int K)
{
    const int nch = K / kChunk;
    const int tile = blockIdx.x, blk = tile / nch, c = tile % nch;
    uint16_t *dst = Xf + (long long)tile * (32 * kChunk);
#pragma unroll
    for (int half = 0; half < 2; half++) {
        const int t = threadIdx.x + 256 * half;  // unit of the tile: row r, k group kq
        const int r = t >> 4, kq = t & 15;
        const int m = 32 * blk + r;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (m < M) v = *(const u32x4 *)(X + (long long)m * K + kChunk * c + 8 * kq);
        // k-step kq/2, half kq%2, row r
        *(u32x4 *)(dst + ((kq >> 1) * 64 + (kq & 1) * 32 + r) * 8) = v;
    }
}

hipError_t launch_splitk_reduce(int dtype, const float *part, uint16_t *Y, long long MN, long long stride, int S,
                                hipStream_t s)
{
    const dim3 grid((unsigned)(((MN + 3) / 4 + 255) / 256));
    if (dtype == DT_F16) hipLaunchKernelGGL((k_splitk_reduce<DT_F16>), grid, dim3(256), 0, s, part, Y, MN, stride, S);
    else hipLaunchKernelGGL((k_splitk_reduce<DT_BF16>), grid, dim3(256), 0, s, part, Y, MN, stride, S);
    return hipGetLastError();
}

hipError_t launch_dequant(int fmt, int dtype, const Args &a, uint16_t *o, hipStream_t s)
{
    const long long total = (long long)a.np * (a.K / kChunk) * 64;
    const dim3 grid((unsigned)((total + 255) / 256));
#define QG_DQ(F, D) hipLaunchKernelGGL((k_dequant<F, D>), grid, dim3(256), 0, s, a, o)
    if (fmt == FMT_Q4K) { if (dtype == DT_F16) QG_DQ(FMT_Q4K, DT_F16); else QG_DQ(FMT_Q4K, DT_BF16); }
    else if (fmt == FMT_Q6K) { if (dtype == DT_F16) QG_DQ(FMT_Q6K, DT_F16); else QG_DQ(FMT_Q6K, DT_BF16); }
    else { if (dtype == DT_F16) QG_DQ(FMT_W4, DT_F16); else QG_DQ(FMT_W4, DT_BF16); }
#undef QG_DQ
    return hipGetLastError();
}

hipError_t launch_x_to_xf(const uint16_t *X, uint16_t *Xf, int M, int K, hipStream_t s)
{
    const long long tiles = ((long long)(M + 31) / 32) * (K / kChunk);
    hipLaunchKernelGGL(k_x_to_xf, dim3((unsigned)tiles), dim3(256), 0, s, X, Xf, M, K);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_staged_dt(int fmt, const Args &a, uint8_t *scratch, const Plan &pl, hipStream_t s)
{
    const long long work = (long long)a.np * (a.K / kChunk) * 64;
    const dim3 grid((unsigned)((work + 255) / 256));
    if (fmt == FMT_Q4K) hipLaunchKernelGGL((k_stage<FMT_Q4K, DT>), grid, dim3(256), 0, s, a, scratch);
    else if (fmt == FMT_Q6K) hipLaunchKernelGGL((k_stage<FMT_Q6K, DT>), grid, dim3(256), 0, s, a, scratch);
    else hipLaunchKernelGGL((k_stage<FMT_W4, DT>), grid, dim3(256), 0, s, a, scratch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.M == 0) return e;
    Args b = a;
    b.W = scratch;
    hipLaunchKernelGGL((k_stream32<FMT_DENSE, DT, 32, 8, 4, 1, 1, X_ROW>), pl.grid, dim3(256), 0, s, b);
    return hipGetLastError();
}

hipError_t launch_staged(int fmt, int dtype, const Args &a, uint8_t *scratch, const Plan &pl, hipStream_t s)
{
    return dtype == DT_F16 ? launch_staged_dt<DT_F16>(fmt, a, scratch, pl, s) : launch_staged_dt<DT_BF16>(fmt, a, scratch, pl, s);
}

}  // namespace qg
