// scan_rows_table.hpp -- lookup of the state-row scan kernels (scan_rows.hip builds the table).
#pragma once

#include "scan_fwd.hpp"

namespace ssm {

constexpr int kRowsWaves = 16;        // waves per workgroup
constexpr int kRowsMaxScanWaves = 6;  // instantiated: 1 .. 6 scan waves (16 .. 96 channels)

struct RowsVariants {
  void (*k[2])(const ScanArgs);  // [0] 16-step chunks, [1] 32-step chunks (NULL where LDS is short)
};

struct RowsTable {
  RowsVariants v[kRowsMaxScanWaves + 1];  // index = scan waves per workgroup
};

const RowsTable& rows_table(bool bf16);

}  // namespace ssm
