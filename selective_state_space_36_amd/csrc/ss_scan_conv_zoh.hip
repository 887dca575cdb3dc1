// ss_scan_conv_zoh.hip -- prefill instances with the convolution + SiLU front end on x and the
// exact zero-order-hold input term (reading guide, "Método").
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ss_launch.h"
#include "ss_scan_kernel.h"

namespace ss {

hipError_t launch_scan_conv_zoh(const ScanArgs& a, bool bf16, bool summary, hipStream_t stream) {
  return launch_scan_instances<true, true>(a, bf16, summary, stream);
}

}  // namespace ss
