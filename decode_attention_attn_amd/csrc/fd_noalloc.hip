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

// The array starts with the single-launch merge's counters, which must be
// zero before the first such call; a fill kernel (not a memset node, which a
// captured graph may not replay faithfully) clears them once per device.
__global__ void clear_counters(int32_t *c, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) c[i] = 0;
}

// Device address of this device's scratch array, or nullptr if it cannot be
// had.  The first call on a device (with that device current) looks it up
// and enqueues the clearing of the counters on `stream`, ahead of the call's
// own kernels.
void *device_scratch(hipStream_t stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_init_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        const int n = (int)(FD_TICKET_BYTES / sizeof(int32_t));
        hipLaunchKernelGGL(clear_counters, dim3(64), dim3(256), 0, stream, static_cast<int32_t *>(ptr), n);
        if (hipGetLastError() != hipSuccess) return nullptr;
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
    void *ws = device_scratch(static_cast<hipStream_t>(stream));
    if (!ws) return FD_ERR_HIP;
    return fd_decode_attn_paged(desc, q, k_cache, v_cache, num_pages, page_size, block_table, max_blocks_per_seq,
                                seq_lens, ws, (size_t)FD_NOALLOC_SCRATCH_BYTES, out, lse, flags, fallback_count,
                                stream);
}
