// Matrix-core partition kernel, q.K and V depth 64 (heads of 64 dimensions): the same
// per-tile scheme as depth 128 with 8-chunk rows, bf16 K staged through LDS like V
// (FA4Config: any qk_depth / ov_depth pair the tiles divide).
#include "partition_mfma.h"

namespace da {

hipError_t launch_partition_mfma_d64(const PartArgs& a, int page_mode, int HG, int KS, hipStream_t s) {
  if (a.Dk == 64 && !a.k_rope) return mfma::launch_shape<mfma::Shape64>(a, page_mode, HG, KS, s);
  return hipErrorInvalidValue;
}

}  // namespace da
