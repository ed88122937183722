// fd_partial_mfma_f8bf16.hip -- the MFMA split-partial kernels for one instantiation type.
#include "fd_partial_mfma.h"

namespace fd {

hipError_t launch_partial_mfma_f8bf16(const PartialParams &p, hipStream_t stream) { return by_dim<kF8 + BF16>(p, stream); }

}  // namespace fd
