// scan_f32.hip -- scan kernels for fp32 x / delta / B / C / z / y.
#include <hip/hip_runtime.h>
#define SSM_SCAN_TABLE_DEFINE
#include "scan_table.hpp"

namespace ssm {
const ScanTable& scan_table_f32() {
  static const ScanTable t = make_scan_table<false>();
  return t;
}
}  // namespace ssm
