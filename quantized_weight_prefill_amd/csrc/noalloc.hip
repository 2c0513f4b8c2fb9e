// noalloc.hip -- qgemm_gemm_xf_noalloc: qgemm_gemm_xf for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The one kernel family that needs memory
// beyond its inputs and outputs is the K split across workgroups (fp32
// partial sums of every slice); here that memory is `scratch`, a fixed
// device array of this file, instead of a workspace argument.
//
// Each GPU the library runs on holds its own copy of `scratch` (16 MiB)
// until the process ends.  In host code the name `scratch` is only a stand-in
// for the symbol: its device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is ever
// handed to a kernel.  Every call on one GPU shares the array: calls that
// overlap on one GPU (two streams, or two host threads) race on it, so
// callers order them, e.g. on one stream.  Nothing in it needs clearing
// between calls: every slice of partial sums is written whole (each output
// of the M x N tile grid by exactly one workgroup of that slice) before the
// reduction reads it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>

#include "plan.h"
#include "qgemm.h"

namespace {

static __device__ __align__(256) unsigned char scratch[QGEMM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device, taken on the first
// call there (two threads racing on that first call both store the same
// address).  Returns QGEMM_OK or QGEMM_ERR_HIP.
int scratch_address(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        fprintf(stderr, "qgemm_gemm_xf_noalloc: no usable current device (%s)\n", hipGetErrorString(e));
        return QGEMM_ERR_HIP;
    }
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            fprintf(stderr, "qgemm_gemm_xf_noalloc: hipGetSymbolAddress failed: %s\n", hipGetErrorString(e));
            return QGEMM_ERR_HIP;
        }
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return QGEMM_OK;
}

}  // namespace

extern "C" int qgemm_gemm_xf_noalloc(int format, int rung, const void *Xf, const void *Wpacked, void *Y, int64_t M,
                                     int64_t N, int64_t K, int64_t group_size, int has_zp, int dtype, void *stream)
{
    // every argument error first, as qgemm_gemm_xf reports it (no launch, no lookup)
    size_t need = 0;
    const int st = qg::gemm_check(format, rung, Xf, Wpacked, Y, M, N, K, group_size, dtype, qg::X_FRAG, &need);
    if (st != QGEMM_OK || M == 0) return st;
    if (need > (size_t)QGEMM_NOALLOC_SCRATCH_BYTES) {
        fprintf(stderr,
                "qgemm_gemm_xf_noalloc: this call needs %zu bytes of split-K partial sums, more than the %d-byte "
                "fixed scratch; use qgemm_gemm_xf with a workspace\n",
                need, QGEMM_NOALLOC_SCRATCH_BYTES);
        return QGEMM_ERR_SIZE;
    }
    void *ws = nullptr;
    if (need > 0) {
        const int sa = scratch_address(&ws);
        if (sa != QGEMM_OK) return sa;
    }
    return qg::gemm_entry(format, rung, Xf, Wpacked, Y, M, N, K, group_size, has_zp, dtype, ws,
                          ws ? (size_t)QGEMM_NOALLOC_SCRATCH_BYTES : 0, stream, qg::X_FRAG);
}
