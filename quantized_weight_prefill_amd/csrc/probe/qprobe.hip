// Measurement aids (libqprobe.so), not part of the GEMM library.  The MFMA probe gives the
// sustained rate of the 32x32x16 MFMA on operands the caller supplies; the
// read probe gives the rate of a plain streaming read.  MI355X lowers its clock
// under dense MFMA load by an amount that depends on the operand bits (random
// fp16 data draws more power than zeros or constants), so the rate a real
// GEMM can reach sits below the 2.5 PFLOP/s dense fp16 figure, which assumes
// the full clock.  The probe reports that ceiling for a given operand set.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "qprobe.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Every wave runs `iters` rounds of four independent 32x32x16 MFMAs; lane l
// of thread t takes its A operands from ops[8t .. 8t+3] and its B operands,
// rotating, from ops[8t+4 .. 8t+7] (one 32 KiB operand block for all waves).
template <int DT>
__global__ void __launch_bounds__(256) k_probe(const u32x4 *ops, float *out, int iters)
{
    u32x4 a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        a[j] = ops[threadIdx.x * 8 + j];
        b[j] = ops[threadIdx.x * 8 + 4 + j];
    }
    f32x16 c[4];
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
        for (int e = 0; e < 16; e++) c[j][e] = 0.f;
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            if constexpr (DT == QPROBE_F16)
                c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[j]),
                                                              __builtin_bit_cast(f16x8, b[(j + it) & 3]), c[j], 0, 0, 0);
            else
                c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[j]),
                                                               __builtin_bit_cast(bf16x8, b[(j + it) & 3]), c[j], 0, 0, 0);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; j++) s += c[j][0] + c[j][15];
    out[blockIdx.x * 256 + threadIdx.x] = s;  // keeps the MFMAs live
}

// Streaming read: each thread loads 16-byte vectors at a grid stride, four
// in flight per step, and folds them into one word so the loads stay live.
__global__ void __launch_bounds__(256) k_read(const u32x4 *buf, long long nvec, uint32_t *out)
{
    const long long stride = (long long)gridDim.x * blockDim.x;
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < nvec; i += 4 * stride) {
        const u32x4 a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
    }
    for (; i < nvec; i += stride) {
        const u32x4 a = buf[i];
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    out[(long long)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" int qprobe_read(const void *buf, int64_t bytes, void *out, int blocks, void *stream)
{
    if (!buf || !out) return QPROBE_ERR_NULL;
    if (((uintptr_t)buf & 15u) != 0) return QPROBE_ERR_ALIGN;
    if (bytes < 16 || bytes % 16 != 0 || blocks < 1) return QPROBE_ERR_SHAPE;
    hipLaunchKernelGGL(k_read, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const u32x4 *)buf, (long long)(bytes / 16),
                       (uint32_t *)out);
    return hipGetLastError() == hipSuccess ? QPROBE_OK : QPROBE_ERR_HIP;
}

extern "C" int qprobe_mfma(const void *operands, float *out, int blocks, int iters, int dtype, void *stream)
{
    if (!operands || !out) return QPROBE_ERR_NULL;
    if (((uintptr_t)operands & 15u) != 0) return QPROBE_ERR_ALIGN;
    if (blocks < 1 || iters < 1) return QPROBE_ERR_SHAPE;
    if (dtype != QPROBE_F16 && dtype != QPROBE_BF16) return QPROBE_ERR_DTYPE;
    hipStream_t s = (hipStream_t)stream;
    if (dtype == QPROBE_F16)
        hipLaunchKernelGGL(k_probe<QPROBE_F16>, dim3(blocks), dim3(256), 0, s, (const u32x4 *)operands, out, iters);
    else
        hipLaunchKernelGGL(k_probe<QPROBE_BF16>, dim3(blocks), dim3(256), 0, s, (const u32x4 *)operands, out, iters);
    return hipGetLastError() == hipSuccess ? QPROBE_OK : QPROBE_ERR_HIP;
}
