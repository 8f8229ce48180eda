// Split-K pass 1 for the latent-shared layout (one kv head, K rows of 576 = 512 + 64
// rotary columns, V = the first 512 columns of K). Not built yet: the launcher reports
// hipErrorNotSupported and the host API refuses the shape before launching.
#include "da_device.h"

namespace da {

hipError_t launch_partition_latent(const PartArgs&, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace da
