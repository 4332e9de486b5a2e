// scan_time_table.hpp -- lookup of the time-parallel scan kernels (scan_time.hip).
#pragma once

#include "scan_fwd.hpp"

namespace ssm {

constexpr int kTimeThreads = 256;  // four waves: one (batch row, channel) per workgroup
using TimeKernel = void (*)(const ScanArgs);
// K = steps per lane: 4 or 8 (NULL otherwise)
TimeKernel time_kernel(bool bf16, int k);

}  // namespace ssm
