// ssd_bf16.hip -- the Mamba-2 SSD chunk kernels, one per (dstate, waves per workgroup).
#include <hip/hip_runtime.h>

#include "ssd_fwd.hpp"

namespace ssm {

// Instantiated pairs: 4 waves for every dstate, 2 waves up to dstate 128 and 1 wave up to 64
// (the per-thread staging registers grow as dstate / waves).  The precomputed C B^T tiles are laid
// out for 4 waves, so that mode exists for 4 waves only.
SsdKernel ssd_kernel(int64_t dstate, int waves, int mode) {
#define SSD_CASE(NN, W)                                                                            \
  if (dstate == NN && waves == W) {                                                                \
    if (mode == kSsdStateOnly) return ssd_chunk_kernel<NN, W, kSsdStateOnly>;                      \
    if (mode == kSsdOutputs) return ssd_chunk_kernel<NN, W, kSsdOutputs>;                          \
    if constexpr (W == 4)                                                                          \
      if (mode == kSsdOutputsGram) return ssd_chunk_kernel<NN, 4, kSsdOutputsGram>;                \
    return nullptr;                                                                                \
  }
  SSD_CASE(32, 4) SSD_CASE(64, 4) SSD_CASE(128, 4) SSD_CASE(256, 4)
  SSD_CASE(32, 2) SSD_CASE(64, 2) SSD_CASE(128, 2)
  SSD_CASE(32, 1) SSD_CASE(64, 1)
#undef SSD_CASE
  return nullptr;
}

SsdKernel ssd_gram_kernel_for(int64_t dstate) {
  switch (dstate) {
    case 32: return ssd_gram_kernel<32>;
    case 64: return ssd_gram_kernel<64>;
    case 128: return ssd_gram_kernel<128>;
    case 256: return ssd_gram_kernel<256>;
    default: return nullptr;
  }
}

SsdUpdateKernel ssd_update_kernel(int64_t dstate) {
  switch (dstate) {
    case 32: return ssd_state_update_kernel<32>;
    case 64: return ssd_state_update_kernel<64>;
    case 128: return ssd_state_update_kernel<128>;
    case 256: return ssd_state_update_kernel<256>;
    default: return nullptr;
  }
}

}  // namespace ssm
