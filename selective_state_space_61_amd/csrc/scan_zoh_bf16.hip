// scan_zoh_bf16.hip -- scan kernels with the exact zero-order-hold input term, bf16 x / delta / B / C / z / y.
#include <hip/hip_runtime.h>
#define SSM_SCAN_TABLE_DEFINE
#include "scan_table.hpp"

namespace ssm {
const ScanTable& scan_table_zoh_bf16() {
  static const ScanTable t = make_table<true, true>();
  return t;
}
}  // namespace ssm
