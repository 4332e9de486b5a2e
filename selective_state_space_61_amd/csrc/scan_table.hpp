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
// exact zero-order-hold variants: 16-step chunks only (full[1] and agg[1] are NULL)
const ScanTable& scan_table_zoh_f32();
const ScanTable& scan_table_zoh_bf16();

#ifdef SSM_SCAN_TABLE_DEFINE
template <bool BF16, int N, int NPL>
void register_scan(ScanTable& m) {
  constexpr int G = N / NPL;
  ScanVariants v{};
  v.full[0] = scan_chunk_kernel<BF16, N, NPL, MODE_FULL, 16>;
  v.agg[0] = scan_chunk_kernel<BF16, N, NPL, MODE_AGG, 16>;
  // 32-step tiles for at most 4 scan waves (8 would fill all 160 KB of LDS)
  if constexpr (G <= 4 && scan_lds_bytes(G, true, 32) <= kLdsBudget)
    v.full[1] = scan_chunk_kernel<BF16, N, NPL, MODE_FULL, 32>;
  if constexpr (G <= 4 && scan_lds_bytes(G, false, 32) <= kLdsBudget)
    v.agg[1] = scan_chunk_kernel<BF16, N, NPL, MODE_AGG, 32>;
  m[{N, NPL}] = v;
}

template <bool BF16, int N, int NPL>
void register_scan_zoh(ScanTable& m) {
  ScanVariants v{};
  v.full[0] = scan_chunk_kernel<BF16, N, NPL, MODE_FULL, 16, true>;
  v.agg[0] = scan_chunk_kernel<BF16, N, NPL, MODE_AGG, 16, true>;
  m[{N, NPL}] = v;
}

// the same (N, chains per lane) pairs as make_scan_table
template <bool BF16, bool ZOH>
ScanTable make_table() {
  ScanTable m;
  auto reg = [&](auto NN, auto PP) {
    constexpr int n = decltype(NN)::value, npl = decltype(PP)::value;
    if constexpr (ZOH) register_scan_zoh<BF16, n, npl>(m);
    else register_scan<BF16, n, npl>(m);
  };
  using std::integral_constant;
#define SSM_REG(n, c) reg(integral_constant<int, n>{}, integral_constant<int, c>{})
  SSM_REG(1, 1); SSM_REG(2, 1); SSM_REG(2, 2); SSM_REG(4, 1); SSM_REG(4, 2); SSM_REG(4, 4);
  SSM_REG(8, 1); SSM_REG(8, 2); SSM_REG(8, 4); SSM_REG(8, 8); SSM_REG(16, 2); SSM_REG(16, 4);
  SSM_REG(16, 8); SSM_REG(16, 16); SSM_REG(32, 4); SSM_REG(32, 8); SSM_REG(32, 16); SSM_REG(64, 8);
  SSM_REG(64, 16);
#undef SSM_REG
  return m;
}

// at most 8 scan waves per workgroup (next to the IO waves, within 1024 threads)
template <bool BF16>
ScanTable make_scan_table() {
  return make_table<BF16, false>();
}
#endif

}  // namespace ssm
