// bf16 instances of the matrix-core forward kernel (P kept as bf16 hi + lo).
#include "fa_mfma.h"

namespace fa {
hipError_t launch_mfma_bf16(const Problem& p, hipStream_t stream) {
  return mfma::launch<__bf16, true>(p, stream);
}
#ifdef FA_TILE_SWEEP
hipError_t launch_mfma_shape_bf16(const Problem& p, int waves, int occupancy, int key_groups, int block_n,
                                  hipStream_t stream) {
  return mfma::launch_shape<__bf16, true>(p, waves, occupancy, key_groups, block_n, stream);
}
#endif
}  // namespace fa
