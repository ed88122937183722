// fd_combine.hip -- exact log-sum-exp merge of the split partials.
//
// One workgroup per (request, query head).  With m = max_s m_s over splits
// that hold tokens, w_s = l_s exp(m_s - m), l = sum_s w_s:
//   out = sum_s w_s O_s / l,   lse = m + ln l
// (page "Flash-Decoding: Mathematical Foundations, Split-KV Parallelism, ...",
// section "The Rescaling and Online Softmax Reduction Algorithm", with O_s
// stored already normalised).  A split with l_s = 0 holds no tokens and is
// skipped, so its O row is never read (handbook page "FlashAttention and
// inference kernels", exercise 2).  The weights go to LDS once; each thread
// then owns four output dimensions of one split group and the groups are
// summed in a fixed order, so the result is bitwise repeatable.
#include "fd_device.h"

namespace fd {
namespace {

constexpr int kThreads = 256;

__device__ float block_max(float v, float *red) {
    v = group_max<64>(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) v = fmaxf(v, red[w]);
    __syncthreads();
    return v;
}

__device__ float block_sum(float v, float *red) {
    v = group_sum<64>(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) v += red[w];
    __syncthreads();
    return v;
}

template <int D>
__global__ void __launch_bounds__(kThreads) combine_kernel(const CombineParams p) {
    extern __shared__ float sw[];          // [max_splits] split weights
    constexpr int DQ = D / 4;              // threads per split row (float4 each)
    constexpr int SG = kThreads / DQ;      // split rows in flight
    __shared__ float4 part[SG][DQ];
    __shared__ float red[kThreads / 64];

    const int h = blockIdx.x, b = blockIdx.y;
    int S = p.max_splits;
    if (p.seq_lens) {
        const int len = request_len(p.seq_lens, b, p.max_splits * p.split, p.max_splits * p.split);
        S = (len + p.split - 1) / p.split;
    }
    const size_t row = (size_t)b * p.Hq + h;
    const size_t base = row * p.max_splits;
    const float *pm = p.part_m + base, *pl = p.part_l + base;

    float mx = -INFINITY;
    for (int s = threadIdx.x; s < S; s += kThreads)
        if (pl[s] > 0.f) mx = fmaxf(mx, pm[s]);
    mx = block_max(mx, red);

    float lsum = 0.f;
    for (int s = threadIdx.x; s < S; s += kThreads) {
        const float l = pl[s];
        const float w = l > 0.f ? l * exp2_fast((pm[s] - mx) * kLog2e) : 0.f;
        sw[s] = w;
        lsum += w;
    }
    lsum = block_sum(lsum, red);           // its barrier also publishes sw

    const int dq = threadIdx.x % DQ, sg = threadIdx.x / DQ;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    const float *po = p.part_o + base * D + dq * 4;
    for (int s = sg; s < S; s += SG) {
        const float w = sw[s];
        if (w > 0.f) {
            const float4 o = *reinterpret_cast<const float4 *>(po + (size_t)s * D);
            a.x = fmaf(w, o.x, a.x);
            a.y = fmaf(w, o.y, a.y);
            a.z = fmaf(w, o.z, a.z);
            a.w = fmaf(w, o.w, a.w);
        }
    }
    part[sg][dq] = a;
    __syncthreads();
    if (sg == 0) {
#pragma unroll
        for (int j = 1; j < SG; ++j) {
            const float4 o = part[j][dq];
            a.x += o.x;
            a.y += o.y;
            a.z += o.z;
            a.w += o.w;
        }
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        const size_t o0 = row * D + dq * 4;
        store_out(p.out, o0 + 0, a.x * inv, p.out_dtype);
        store_out(p.out, o0 + 1, a.y * inv, p.out_dtype);
        store_out(p.out, o0 + 2, a.z * inv, p.out_dtype);
        store_out(p.out, o0 + 3, a.w * inv, p.out_dtype);
    }
    if (threadIdx.x == 0 && p.lse) p.lse[row] = lsum > 0.f ? mx + logf(lsum) : -INFINITY;
}

}  // namespace

hipError_t launch_combine(const CombineParams &p, hipStream_t stream) {
    dim3 grid(p.Hq, p.B);
    const size_t smem = (size_t)p.max_splits * sizeof(float);
    if (p.d == 64)
        hipLaunchKernelGGL((combine_kernel<64>), grid, dim3(kThreads), smem, stream, p);
    else
        hipLaunchKernelGGL((combine_kernel<128>), grid, dim3(kThreads), smem, stream, p);
    return hipGetLastError();
}

}  // namespace fd
