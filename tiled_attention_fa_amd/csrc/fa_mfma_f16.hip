// fp16 instances of the matrix-core forward kernel (P rounded to fp16 once).
#include "fa_mfma.h"

namespace fa {
hipError_t launch_mfma_f16(const Problem& p, hipStream_t stream) {
  return mfma::launch<_Float16, false>(p, stream);
}
#ifdef FA_TILE_SWEEP
hipError_t launch_mfma_shape_f16(const Problem& p, int waves, int occupancy, int key_groups, int block_n,
                                  hipStream_t stream) {
  return mfma::launch_shape<_Float16, false>(p, waves, occupancy, key_groups, block_n, stream);
}
#endif
}  // namespace fa
