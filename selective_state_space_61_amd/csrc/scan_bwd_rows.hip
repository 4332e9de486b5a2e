// scan_bwd_rows.hip -- instantiations of the state-row backward (scan_bwd_rows.hpp): dstate 16,
// Delta B input term, bf16; S scan waves (16 S channels) per workgroup.
#include <hip/hip_runtime.h>

#include "scan_bwd_rows.hpp"

namespace ssm {

BwdRowsKernel bwd_rows_kernel(int S) {
  switch (S) {
    case 1: return scan_bwd_rows_kernel<1>;
    case 2: return scan_bwd_rows_kernel<2>;
    case 3: return scan_bwd_rows_kernel<3>;
    default: return nullptr;
  }
}

}  // namespace ssm
