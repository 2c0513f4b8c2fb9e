// plan.h -- host-side launch plans of the fused-dequant GEMM and the launch
// functions each kernel translation unit provides.  The M-ladder and the C
// ABI (api.hip) fill a Plan and call these; the kernels and their template
// instantiations live in the inst_*.hip and misc*.hip units, compiled apart
// so that the library builds in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "common.h"

namespace qg {

enum Rung {
    RUNG_SMALL_M = 0,     // direct, one panel per wave, up to 64 rows per wave
    RUNG_SKINNY_N = 1,    // direct, up to four panels per wave, 16 rows per wave
    RUNG_WIDE = 2,        // direct, four panels and up to 48 rows per wave
    RUNG_M16_256 = 3,     // 16x16x32 MFMA: 256x128, 8 waves of 32x128
    RUNG_M128 = 4,        // 32x32x16 MFMA: 128x128, 4 waves of 32x128
    RUNG_M128_K2 = 5,     // 32x32x16 MFMA: 128x128, K split over two 4-wave groups
    RUNG_M128N160 = 6,    // 32x32x16 MFMA: 128x160, 4 waves of 32x160
    RUNG_M64_K4 = 7,      // 32x32x16 MFMA: 64x64, 2 waves of 32x64, K split over four groups
    RUNG_M352N96 = 8,     // 32x32x16 MFMA: 352x96, 11 waves of 32x96
    RUNG_M192N96_K2 = 9,  // 32x32x16 MFMA: 192x96, K split over two 6-wave groups (three waves per SIMD)
    RUNG_M192N64_K2 = 10, // 32x32x16 MFMA: 192x64, K split over two 6-wave groups
    RUNG_M64_SK = 11,     // 32x32x16 MFMA: 64x64, K split over four groups and across workgroups
    RUNG_M64N32_K4 = 12,  // 32x32x16 MFMA: 64x32, 2 waves of 32x32, K split over four groups
    RUNG_M128N64_K2 = 13, // 32x32x16 MFMA: 128x64, 4 waves of 32x64, K split over two groups
    RUNG_M96N32_K4 = 14,  // 32x32x16 MFMA: 96x32, 3 waves of 32x32, K split over four groups
    RUNG_M768N96 = 15,    // 32x32x16 MFMA: 768x96, 8 waves of 96x96 (two per SIMD)
    RUNG_M512N128 = 16,   // 32x32x16 MFMA: 512x128, 8 waves of 64x128
    RUNG_M512N96 = 17,    // 32x32x16 MFMA: 512x96, 8 waves of 64x96
    RUNG_M768N64_SK = 18, // 32x32x16 MFMA: 768x64, 8 waves of 96x64, K split across workgroups
    RUNG_COUNT = 19
};

enum I8Rung {
    I8_M128 = 0,        // 128x128, 4 waves of 32x128
    I8_M256 = 1,        // 256x128, 8 waves of 32x128: each weight unpacked once for 256 rows
    I8_M128_K2 = 2,     // 128x128, K split over two 4-wave groups
    I8_M256N96 = 3,     // 256x96, 8 waves of 32x96
    I8_M512N96 = 4,     // 512x96, 8 waves of 64x96: each weight unpacked once for 512 rows
    I8_M352N96 = 5,     // 352x96, 11 waves of 32x96 (three per SIMD)
    I8_M192N96_K2 = 6,  // 192x96, K split over two 6-wave groups (three waves per SIMD)
    I8_M192N64_K2 = 7,  // 192x64, K split over two 6-wave groups
    I8_M64_SK = 8,      // 64x64, K split over four groups and across workgroups
    I8_M768N96 = 9,     // 768x96, 8 waves of 96x96: each weight unpacked once for 768 rows
    I8_RUNG_COUNT = 10
};

struct Plan {
    int rung;
    int tiles_n, tiles_m;  // output tiles along N and along M
    int rows, cols;        // output tile
    int waves, kw;         // waves per workgroup, K-split ways inside one workgroup
    int split;             // K slices across workgroups (1: none)
    int rb, pn;            // direct kernel: row blocks / panels per wave
    dim3 grid;
    size_t lds;            // dynamic LDS bytes
};

// fp16/bf16 path, one instantiation per (format, dtype, activation layout)
// in inst_fp.hip: the direct and streaming rungs of a Plan.
template <int FMT, int DT, int XL>
hipError_t launch_fd(const Plan &pl, const Args &a, hipStream_t s);

// misc.hip
hipError_t launch_splitk_reduce(int dtype, const float *part, uint16_t *Y, long long MN, long long stride, int S,
                                hipStream_t s);
hipError_t launch_dequant(int fmt, int dtype, const Args &a, uint16_t *out, hipStream_t s);
hipError_t launch_x_to_xf(const uint16_t *X, uint16_t *Xf, int M, int K, hipStream_t s);
hipError_t launch_staged(int fmt, int dtype, const Args &a, uint8_t *scratch, const Plan &pl, hipStream_t s);
// Grouped plans: Plan.rung names the kernel, Plan.rb its 16-row blocks.
enum GroupedKernel {
    GROUPED_DIRECT = 0,  // k_direct_grouped: 4 panels per wave, rb 1 or 2, K split over kw waves
    GROUPED_SHARED = 1   // k_grouped_shared: 4 waves of 2 panels sharing X through LDS, rb 2 or 5
};
// misc_grouped.hip: the Plan's grouped kernel on activations of layout xl
// (X_ROW or X_FRAG)
hipError_t launch_grouped(int fmt, int dtype, int xl, const Plan &pl, const Args &a, hipStream_t s);

// api.hip: the checked fp16/bf16 GEMM of qgemm_gemm_rung (layout X_ROW) and
// qgemm_gemm_xf (X_FRAG) with an explicit workspace, and the workspace it
// needs; for the entry points that bring their own workspace (noalloc.hip).
int gemm_entry(int fmt, int rung, const void *X, const void *W, void *Y, long long M, long long N, long long K,
               long long group, int has_zp, int dtype, void *ws, size_t ws_bytes, void *stream, int xl);
// Every argument check of gemm_entry but the workspace's: QGEMM_OK (M == 0
// included) with the workspace bytes the call needs, or the first error.
int gemm_check(int fmt, int rung, const void *X, const void *W, void *Y, long long M, long long N, long long K,
               long long group, int dtype, int xl, size_t *ws_need);

// int8 path: one instantiation per (format, dtype) in inst_i8.hip, the rest in
// misc_i8.hip
template <int FMT, int DT>
hipError_t launch_i8_fd(const Plan &pl, const Args &a, hipStream_t s);
hipError_t launch_i8_reduce(int dtype, const int *part, const float *sx, const float *sw, uint16_t *Y, int M, int N,
                            long long stride, int S, hipStream_t s);
hipError_t launch_i8_quant(int dtype, const uint16_t *X, uint8_t *Xq, float *sx, int M, int K, hipStream_t s);
hipError_t launch_i8_colscale(int fmt, const Args &a, float *rw, float *sw, hipStream_t s);

}  // namespace qg
