// ss_scan_fwd.hip -- prefill launches with the first-order input term dt B u and u given (the
// default), the dispatch to the exact zero-order-hold and convolution front-end instances, and
// the empty-sequence state copy.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ss_launch.h"
#include "ss_scan_kernel.h"

namespace ss {
namespace {

__global__ void __launch_bounds__(256) copy_state_kernel(float* dst, const float* src, int64_t n) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = src ? src[i] : 0.0f;
}

}  // namespace

hipError_t launch_scan(const ScanArgs& a, bool bf16, bool summary, hipStream_t stream) {
  if (a.conv_w)
    return a.zoh ? launch_scan_conv_zoh(a, bf16, summary, stream)
                 : launch_scan_conv(a, bf16, summary, stream);
  if (a.zoh) return launch_scan_zoh(a, bf16, summary, stream);
  return launch_scan_instances<false, false>(a, bf16, summary, stream);
}

hipError_t launch_copy_state(float* dst, const float* src, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(copy_state_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, dst, src, n);
  return hipGetLastError();
}

}  // namespace ss
