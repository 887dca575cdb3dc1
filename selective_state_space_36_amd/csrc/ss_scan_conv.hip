// ss_scan_conv.hip -- prefill instances with the convolution + SiLU front end on x (the Mamba
// block's SSM input, IBM explainer, Mamba-block walk-through) and the first-order input term.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ss_launch.h"
#include "ss_scan_kernel.h"

namespace ss {

hipError_t launch_scan_conv(const ScanArgs& a, bool bf16, bool summary, hipStream_t stream) {
  return launch_scan_instances<false, true>(a, bf16, summary, stream);
}

}  // namespace ss
