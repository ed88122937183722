// fd_partial_mfma.hip -- split-partial kernel with the q-group x K^T product
// on the matrix cores.  Not built yet: every shape goes to the VALU kernel.
#include "fd_device.h"

namespace fd {

bool mfma_supports(const PartialParams &) { return false; }

hipError_t launch_partial_mfma(const PartialParams &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace fd
