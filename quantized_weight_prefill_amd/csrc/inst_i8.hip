// inst_i8.hip -- one (format, dtype) instantiation of the int8-path GEMM
// kernels; the build compiles this file once per combination with QG_FMT
// and QG_DT defined.
#include "kernels_i8.h"

#if !defined(QG_FMT) || !defined(QG_DT)
#error "inst_i8.hip is compiled with -DQG_FMT=<format> -DQG_DT=<dtype>"
#endif

namespace qg {
template hipError_t launch_i8_fd<QG_FMT, QG_DT>(const Plan &, const Args &, hipStream_t);
}  // namespace qg
