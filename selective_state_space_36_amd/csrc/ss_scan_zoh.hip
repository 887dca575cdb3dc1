// ss_scan_zoh.hip -- prefill instances with the exact zero-order-hold input term
// (exp(dt A) - 1) / A * B u (reading guide, "Método"); a translation unit of its own so that
// the two sets of instances compile in parallel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ss_launch.h"
#include "ss_scan_kernel.h"

namespace ss {

hipError_t launch_scan_zoh(const ScanArgs& a, bool bf16, bool summary, hipStream_t stream) {
  return launch_scan_instances<true, false>(a, bf16, summary, stream);
}

}  // namespace ss
