// scan_table.hpp -- the instantiated scan kernels, keyed by (dstate, chains per lane).  Each dtype's
// table is built in a translation unit of its own (scan_f32.hip, scan_bf16.hip) so that they
// compile in parallel; ssm_api.hip only looks kernels up.
#pragma once

#include <map>
#include <utility>

#include "scan_fwd.hpp"

namespace ssm {

using ScanKernel = void (*)(const ScanArgs);

// kernels of one (dstate, chains per lane): [0] chunks of 16 steps, [1] of 32 (NULL where the
// 32-step LDS tiles do not fit)
struct ScanVariants {
  ScanKernel full[2];
  ScanKernel agg[2];
};

using ScanTable = std::map<std::pair<int, int>, ScanVariants>;

const ScanTable& scan_table_f32();
const ScanTable& scan_table_bf16();

#ifdef SSM_SCAN_TABLE_DEFINE
template <bool BF16, int N, int NPL>
void register_scan(ScanTable& m) {
  constexpr int G = N / NPL;
  ScanVariants v{};
  v.full[0] = scan_chunk_kernel<BF16, N, NPL, MODE_FULL, 16>;
  v.agg[0] = scan_chunk_kernel<BF16, N, NPL, MODE_AGG, 16>;
  if constexpr (scan_lds_bytes(G, true, 32) <= kLdsBudget) v.full[1] = scan_chunk_kernel<BF16, N, NPL, MODE_FULL, 32>;
  if constexpr (scan_lds_bytes(G, false, 32) <= kLdsBudget) v.agg[1] = scan_chunk_kernel<BF16, N, NPL, MODE_AGG, 32>;
  m[{N, NPL}] = v;
}

// at most 8 scan waves per workgroup (next to the IO waves, within 1024 threads)
template <bool BF16>
ScanTable make_scan_table() {
  ScanTable m;
  register_scan<BF16, 1, 1>(m);
  register_scan<BF16, 2, 1>(m);
  register_scan<BF16, 2, 2>(m);
  register_scan<BF16, 4, 1>(m);
  register_scan<BF16, 4, 2>(m);
  register_scan<BF16, 4, 4>(m);
  register_scan<BF16, 8, 1>(m);
  register_scan<BF16, 8, 2>(m);
  register_scan<BF16, 8, 4>(m);
  register_scan<BF16, 8, 8>(m);
  register_scan<BF16, 16, 2>(m);
  register_scan<BF16, 16, 4>(m);
  register_scan<BF16, 16, 8>(m);
  register_scan<BF16, 16, 16>(m);
  register_scan<BF16, 32, 4>(m);
  register_scan<BF16, 32, 8>(m);
  register_scan<BF16, 32, 16>(m);
  register_scan<BF16, 64, 8>(m);
  register_scan<BF16, 64, 16>(m);
  return m;
}
#endif

}  // namespace ssm
