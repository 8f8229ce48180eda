// Matrix-core partition kernel, depth 128/128 (q.K and V), bf16 or fp8 caches, and the
// dispatch over the depth shapes of the same kernel (the wider shapes live in their own
// translation units so that they compile in parallel).
#include "partition_mfma.h"

namespace da {

hipError_t launch_partition_mfma(const PartArgs& a, int page_mode, int HG, int KS, hipStream_t s) {
  if (a.Dqk == 128 && a.Dv == 128 && a.Dk == 128) return mfma::launch_shape<mfma::Shape128>(a, page_mode, HG, KS, s);
  if (a.Dqk == 64 && a.Dv == 64) return launch_partition_mfma_d64(a, page_mode, HG, KS, s);
  if (a.Dqk == 192 && a.Dv == 128) return launch_partition_mfma_d192(a, page_mode, HG, KS, s);
  if (a.Dqk == 256 && a.Dv == 256) return launch_partition_mfma_d256(a, page_mode, HG, KS, s);
  return hipErrorInvalidValue;
}

}  // namespace da
