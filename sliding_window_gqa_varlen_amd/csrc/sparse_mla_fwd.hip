#include "device_common.h"
#include "launch.h"

namespace swa {
hipError_t sparse_mla_fwd_launch(const SparseMlaParams&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace swa
