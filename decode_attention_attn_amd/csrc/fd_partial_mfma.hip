// fd_partial_mfma.hip -- which MFMA split-partial instantiations exist and
// the dispatch to the per-type translation units (fd_partial_mfma_<type>.hip).
#include "fd_device.h"

namespace fd {

constexpr int kBlkTokens = 16;   // tokens per MFMA block (a block must sit in one page)

bool mfma_supports(const PartialParams &p) {
    if (p.dtype != F16 && p.dtype != BF16 && p.dtype != FP8) return false;
    if (p.d != 64 && p.d != 128) return false;
    if (p.page_size && p.page_size % kBlkTokens) return false;   // a 16-token block must sit in one page
    // unified-max weights reach e^64; fp16 operands would overflow past 65504
    if (p.q_dtype == F16 && p.unified) return false;
    return true;
}

hipError_t launch_partial_mfma(const PartialParams &p, hipStream_t stream) {
    if (p.dtype == FP8) return p.q_dtype == F16 ? launch_partial_mfma_f8f16(p, stream) : launch_partial_mfma_f8bf16(p, stream);
    return p.dtype == F16 ? launch_partial_mfma_f16(p, stream) : launch_partial_mfma_bf16(p, stream);
}

}  // namespace fd
