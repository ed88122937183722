// fd_merge.h -- the single-launch merge: the last workgroup of a (request,
// KV head) to finish merges that head's partials into out and lse.
//
// The merge is the Flash-Decoding combine (page "Flash-Decoding: ...",
// "The Rescaling and Online Softmax Reduction Algorithm": m = max_j m_j,
// w_j = l_j exp(m_j - m), out = sum_j w_j O_j / sum_j w_j, lse = m + ln l),
// done inside the partial kernel instead of a second launch: every workgroup
// writes its partial, then takes a ticket from a per-(request, KV head)
// counter, and the one that takes the last ticket reads all partials of that
// head back and merges them in a fixed order (FlashDecoding++ page,
// "Asynchronized Softmax with Unified Max Value", its design choices: a
// reduction across workers after the partial results are written, by atomics
// rather than a relaunch).
//
// Coherence across the GPU's XCDs: each XCD has its own L2, so the partials
// are written with device-scope stores (write-through to the device's
// coherence point) and read back with device-scope loads; a workgroup waits
// for its own stores to complete before it takes its ticket.  The last
// workgroup resets the counter to zero, so a completed call leaves every
// counter as the next call needs it.
#pragma once

#include "fd_device.h"

namespace fd {

constexpr int kBufDeviceScope = 16;   // buffer cache policy: device scope (sc1)

__device__ __forceinline__ void store_dev(float *ptr, float v) {
    __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A partial's element: device-scope store for the single-launch merge, a
// plain store for a later combine launch.
template <bool DEV>
__device__ __forceinline__ void store_partial(float *ptr, float v) {
    if constexpr (DEV)
        store_dev(ptr, v);
    else
        *ptr = v;
}

// Request b's partials as buffer resources (wave-uniform bases); the host
// makes sure one request's partials span less than 4 GiB.
struct ReqPartials {
    __amdgpu_buffer_rsrc_t o, m, l;
    size_t row0;     // first query row of the request
};

__device__ __forceinline__ char *uniform_base(const void *ptr) {
    const uint64_t a = reinterpret_cast<uint64_t>(ptr);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return reinterpret_cast<char *>(((uint64_t)hi << 32) | lo);
}

template <int D>
__device__ __forceinline__ ReqPartials req_partials(const PartialParams &p, int b) {
    constexpr int32_t kWord3 = 0x00020000;   // raw buffer: 32-bit data format, no swizzle, no stride
    ReqPartials r;
    r.row0 = (size_t)b * p.q_len * p.Hq;
    const uint32_t slots = (uint32_t)(p.q_len * p.Hq) * (uint32_t)p.max_splits;
    const size_t s0 = r.row0 * p.max_splits;
    r.o = __builtin_amdgcn_make_buffer_rsrc(uniform_base(p.part_o + s0 * D), 0,
                                            __builtin_amdgcn_readfirstlane(slots * D * 4), kWord3);
    r.m = __builtin_amdgcn_make_buffer_rsrc(uniform_base(p.part_m + s0), 0,
                                            __builtin_amdgcn_readfirstlane(slots * 4), kWord3);
    r.l = __builtin_amdgcn_make_buffer_rsrc(uniform_base(p.part_l + s0), 0,
                                            __builtin_amdgcn_readfirstlane(slots * 4), kWord3);
    return r;
}

__device__ __forceinline__ float load_dev(const __amdgpu_buffer_rsrc_t &r, uint32_t byte_off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, kBufDeviceScope));
}

__device__ __forceinline__ float4 load_dev4(const __amdgpu_buffer_rsrc_t &r, uint32_t byte_off) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kBufDeviceScope);
    return make_float4(__int_as_float(v.x), __int_as_float(v.y), __int_as_float(v.z), __int_as_float(v.w));
}

// After this workgroup's last partial store: wait until its stores have
// completed (device scope), take a ticket of the (request, KV head) counter,
// and return true in the workgroup that takes ticket n - 1 (n workgroups of
// that head take part).  That workgroup also resets the counter.  Every
// thread of the workgroup must call this; the result is uniform.
__device__ __forceinline__ bool arrive_last(int32_t *ticket, int n, int *lds_ticket) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) *lds_ticket = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const bool last = *lds_ticket == n - 1;
    if (last && threadIdx.x == 0) __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return last;
}

// LDS the merge needs, in floats (none: the merge runs in registers and lane
// shuffles; kept as a named size for the kernels' LDS unions).
__host__ __device__ constexpr int merge_lds_floats(int rows_x_parts, int rows, int threads) {
    (void)rows_x_parts;
    (void)rows;
    (void)threads;
    return 4;
}

// Merge n partials (slots 0 .. n-1) of each query row of KV head kvh of
// request b into out and lse.  All THREADS threads of the workgroup call it.
//
// Thread layout: output quad q (row rho = q / (D/4), dims 4 dq .. 4 dq + 3)
// is shared by P adjacent lanes (P a power of two, as many as the
// workgroup's threads allow), lane ph of them taking partials j = ph, ph + P,
// ...  Each lane requests the O quads, m and l of its partials at once (one
// memory round trip for CH of them), keeps a running max-rescaled state
// (M, L, acc) over them in partial order, and the P lanes of a quad merge
// their states by a lane butterfly, each step the same max-rescale rule; the
// fixed order makes the result bitwise repeatable.
template <int D, int THREADS>
__device__ void merge_rows(const PartialParams &p, int b, int kvh, int n, float *lds) {
    (void)lds;
    constexpr int DQ = D / 4;
    constexpr int CH = 16;                    // partials per lane whose loads are in flight together
    const int R = p.R;
    const int tid = threadIdx.x;
    const ReqPartials rp = req_partials<D>(p, b);
    const uint32_t Sm = (uint32_t)p.max_splits;
    const int quads = R * DQ;
    int P = 1;                                // lanes per quad: a power of two, at most 64
    while (P < 64 && 2 * P * quads <= THREADS) P *= 2;
    const int ph = tid & (P - 1);

    for (int q = tid / P; q < quads; q += THREADS / P) {
        const int rho = q / DQ, dq = q - rho * DQ;
        const uint32_t row_slot0 = (uint32_t)(query_row(p, b, kvh, rho) - rp.row0) * Sm;   // slot of partial 0
        float M = -INFINITY, L = 0.f;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j0 = ph; j0 < n; j0 += P * CH) {
            float4 o[CH];
            float mv[CH], lv[CH];
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int j = j0 + P * c;
                const uint32_t sl = row_slot0 + (uint32_t)j;
                const bool ok = j < n;
                o[c] = ok ? load_dev4(rp.o, (sl * D + 4 * dq) * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
                mv[c] = ok ? load_dev(rp.m, sl * 4) : -INFINITY;
                lv[c] = ok ? load_dev(rp.l, sl * 4) : 0.f;
            }
            float mx = M;
#pragma unroll
            for (int c = 0; c < CH; ++c)
                if (lv[c] > 0.f) mx = fmaxf(mx, mv[c]);
            // M, mx are natural-log units (partial m values): exp(M - mx) = exp2((M - mx) log2 e)
            const float fr = M == -INFINITY ? 0.f : exp2_fast((M - mx) * kLog2e);
            L *= fr;
            acc.x *= fr;
            acc.y *= fr;
            acc.z *= fr;
            acc.w *= fr;
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                if (lv[c] > 0.f) {      // an empty partial's O row is never used
                    const float w = lv[c] * exp2_fast((mv[c] - mx) * kLog2e);
                    L += w;
                    acc.x = fmaf(w, o[c].x, acc.x);
                    acc.y = fmaf(w, o[c].y, acc.y);
                    acc.z = fmaf(w, o[c].z, acc.z);
                    acc.w = fmaf(w, o[c].w, acc.w);
                }
            }
            M = mx;
        }
        // the P lanes of the quad: butterfly merge
        for (int off = 1; off < P; off <<= 1) {
            const float M2 = __shfl_xor(M, off), L2 = __shfl_xor(L, off);
            const float4 a2 = make_float4(__shfl_xor(acc.x, off), __shfl_xor(acc.y, off), __shfl_xor(acc.z, off),
                                          __shfl_xor(acc.w, off));
            const float Mx = fmaxf(M, M2);
            const float f1 = M == -INFINITY ? 0.f : exp2_fast((M - Mx) * kLog2e);
            const float f2 = M2 == -INFINITY ? 0.f : exp2_fast((M2 - Mx) * kLog2e);
            L = L * f1 + L2 * f2;
            acc.x = acc.x * f1 + a2.x * f2;
            acc.y = acc.y * f1 + a2.y * f2;
            acc.z = acc.z * f1 + a2.z * f2;
            acc.w = acc.w * f1 + a2.w * f2;
            M = Mx;
        }
        if (ph == 0) {
            const float inv = L > 0.f ? 1.f / L : 0.f;
            const size_t o0 = query_row(p, b, kvh, rho) * D + 4 * dq;
            store_out(p.out, o0 + 0, acc.x * inv, p.out_dtype);
            store_out(p.out, o0 + 1, acc.y * inv, p.out_dtype);
            store_out(p.out, o0 + 2, acc.z * inv, p.out_dtype);
            store_out(p.out, o0 + 3, acc.w * inv, p.out_dtype);
            if (dq == 0 && p.lse) p.lse[query_row(p, b, kvh, rho)] = L > 0.f ? M + logf(L) : -INFINITY;
        }
    }
}

// A request with no tokens: out 0 and lse -inf for the KV head's query rows.
template <int D>
__device__ void write_empty_rows(const PartialParams &p, int b, int kvh, int nthreads) {
    for (int idx = threadIdx.x; idx < p.R * D; idx += nthreads)
        store_out(p.out, query_row(p, b, kvh, idx / D) * D + idx % D, 0.f, p.out_dtype);
    if ((int)threadIdx.x < p.R && p.lse) p.lse[query_row(p, b, kvh, threadIdx.x)] = -INFINITY;
}

}  // namespace fd
