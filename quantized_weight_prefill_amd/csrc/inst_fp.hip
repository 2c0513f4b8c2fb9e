// inst_fp.hip -- one (format, dtype, activation layout) instantiation of
// the fp16/bf16 kernels; the build compiles this file once per combination
// with QG_FMT, QG_DT and QG_XL defined.
#include "kernels_fp.h"

#if !defined(QG_FMT) || !defined(QG_DT) || !defined(QG_XL)
#error "inst_fp.hip is compiled with -DQG_FMT=<format> -DQG_DT=<dtype> -DQG_XL=<layout>"
#endif

namespace qg {
template hipError_t launch_fd<QG_FMT, QG_DT, QG_XL>(const Plan &, const Args &, hipStream_t);
}  // namespace qg
