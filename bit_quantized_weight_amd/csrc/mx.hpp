// Internal interface between the dense and MX sources.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {
// fp32 dump of MXFP8 / MXFP4 packed weights (qgemv_dequant for those formats)
int mx_dequant(int fmt, const void* wq, const void* ws, int64_t M, int64_t K, float* w_out, hipStream_t stream);
}  // namespace qg
