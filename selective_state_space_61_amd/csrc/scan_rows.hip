// scan_rows.hip -- instantiations of the state-row scan (scan_rows.hpp): dstate 16, Delta B input
// term, whole sequences; S scan waves (16 S channels) per workgroup, 16- or 32-step chunks.
#include <hip/hip_runtime.h>

#include "scan_rows.hpp"
#include "scan_rows_table.hpp"

namespace ssm {

namespace {
template <bool BF16, int S>
RowsVariants rows_variants() {
  RowsVariants v{};
  v.k[0] = scan_rows_kernel<BF16, S, 16>;
  if constexpr (rows_lds_bytes(S, 32) <= kLdsBudget) v.k[1] = scan_rows_kernel<BF16, S, 32>;
  return v;
}

template <bool BF16>
RowsTable make_rows_table() {
  RowsTable t{};
  t.v[1] = rows_variants<BF16, 1>();
  t.v[2] = rows_variants<BF16, 2>();
  t.v[3] = rows_variants<BF16, 3>();
  t.v[4] = rows_variants<BF16, 4>();
  t.v[5] = rows_variants<BF16, 5>();
  t.v[6] = rows_variants<BF16, 6>();
  return t;
}
}  // namespace

const RowsTable& rows_table(bool bf16) {
  static const RowsTable tb = make_rows_table<true>();
  static const RowsTable tf = make_rows_table<false>();
  return bf16 ? tb : tf;
}

}  // namespace ssm
