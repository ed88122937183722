// fd_noalloc.hip -- fd_decode_attn_paged_noalloc: the paged entry point for
// callers that cannot allocate (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  Its split partials live in a
// file-scope device array instead of a caller-provided workspace; everything
// else is fd_decode_attn_paged.
#include <mutex>

#include "fd_decode_attn.h"
#include "fd_internal.h"

#define FD_API extern "C" __attribute__((visibility("default")))

namespace {

// One copy per GPU the library runs on, held until the process ends.  In host
// code `scratch` names a host-side stand-in; the device address comes from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[FD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_init_mutex;
void *g_scratch_ptr[kMaxDevices];   // written once per device under the mutex

// Device address of this device's scratch array, or nullptr if it cannot be
// had.  The first call on a device (with that device current) looks it up.
void *device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_init_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

FD_API fd_status fd_decode_attn_paged_noalloc(const fd_decode_desc *desc, const void *q, const void *k_cache,
                                              const void *v_cache, int32_t num_pages, int32_t page_size,
                                              const int32_t *block_table, int32_t max_blocks_per_seq,
                                              const int32_t *seq_lens, void *out, float *lse, uint8_t *flags,
                                              int32_t *fallback_count, void *stream) {
    const size_t need = fd_workspace_bytes(desc);
    if (need == 0) {
        // an invalid descriptor: let the paged entry point name the error
        return fd_decode_attn_paged(desc, q, k_cache, v_cache, num_pages, page_size, block_table,
                                    max_blocks_per_seq, seq_lens, nullptr, 0, out, lse, flags, fallback_count,
                                    stream);
    }
    if (need > (size_t)FD_NOALLOC_SCRATCH_BYTES) return FD_ERR_WORKSPACE_TOO_SMALL;
    void *ws = device_scratch();
    if (!ws) return FD_ERR_HIP;
    return fd_decode_attn_paged(desc, q, k_cache, v_cache, num_pages, page_size, block_table, max_blocks_per_seq,
                                seq_lens, ws, (size_t)FD_NOALLOC_SCRATCH_BYTES, out, lse, flags, fallback_count,
                                stream);
}
