// Matrix-core partition kernel, q.K depth 192 (128 nope + 64 rotary columns) with V depth
// 128: the nope width equals the V width (FA4Config, rope_depth). The rotary columns sit
// in the K rows, or apart in a bf16 tensor of their own (FA4Config, rope_dtype).
#include "partition_mfma.h"

namespace da {

hipError_t launch_partition_mfma_d192(const PartArgs& a, int page_mode, int HG, int KS, hipStream_t s) {
  if (a.Dk == 192) return mfma::launch_shape<mfma::Shape192>(a, page_mode, HG, KS, s);
  if (a.Dk == 128 && a.k_rope) return mfma::launch_shape<mfma::Shape192R>(a, page_mode, HG, KS, s);
  return hipErrorInvalidValue;
}

}  // namespace da
