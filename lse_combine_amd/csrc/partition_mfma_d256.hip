// Matrix-core partition kernel, q.K depth 256 (192 nope + 64 rotary columns) with V depth
// 256: V is wider than the nope part (FA4Config, rope_depth: the rotary width is the q.K
// depth minus the nope depth, not minus the V depth). The rotary columns sit in the K
// rows, or apart in a bf16 tensor of their own (FA4Config, rope_dtype).
#include "partition_mfma.h"

namespace da {

hipError_t launch_partition_mfma_d256(const PartArgs& a, int page_mode, int HG, int KS, hipStream_t s) {
  if (a.Dk == 256) return mfma::launch_shape<mfma::Shape256>(a, page_mode, HG, KS, s);
  if (a.Dk == 192 && a.k_rope) return mfma::launch_shape<mfma::Shape256R>(a, page_mode, HG, KS, s);
  return hipErrorInvalidValue;
}

}  // namespace da
