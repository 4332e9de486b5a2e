// scan_time.hip -- instantiations of the time-parallel scan (scan_time.hpp): dstate 16, Delta B,
// blocks of K = 4 or 8 steps per lane (chunks of 256 or 512 steps).
#include <hip/hip_runtime.h>

#include "scan_time.hpp"
#include "scan_time_table.hpp"

namespace ssm {

TimeKernel time_kernel(bool bf16, int k) {
  if (k == 4) return bf16 ? scan_time_kernel<true, 4> : scan_time_kernel<false, 4>;
  if (k == 8) return bf16 ? scan_time_kernel<true, 8> : scan_time_kernel<false, 8>;
  return nullptr;
}

}  // namespace ssm
