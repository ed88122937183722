// fd_combine.hip -- exact log-sum-exp merge of the split partials.
//
// One workgroup per (request, query head).  With m = max_s m_s over splits
// that hold tokens, w_s = l_s exp(m_s - m), l = sum_s w_s:
//   out = sum_s w_s O_s / l,   lse = m + ln l
// (page "Flash-Decoding: Mathematical Foundations, Split-KV Parallelism, ...",
// section "The Rescaling and Online Softmax Reduction Algorithm", with O_s
// stored already normalised).  A split with l_s = 0 holds no tokens and is
// skipped: its O row (never written) gets weight 0 and is never used
// (handbook page "FlashAttention and inference kernels", exercise 2).  Each
// thread owns four output dimensions of one split group; the O loads of up
// to 16 of its splits are issued before the weights are computed so that one
// memory round trip covers them; the weights go to LDS once and the groups
// are summed in a fixed order, so the result is bitwise repeatable.
#include "fd_device.h"

namespace fd {
namespace {

template <int NW>
__device__ float block_max(float v, float *red) {
    v = group_max<64>(v);
    if constexpr (NW == 1) return v;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) v = fmaxf(v, red[w]);
    __syncthreads();
    return v;
}

// (a one-wave block still needs the barrier: it publishes the LDS weights)
template <int NW>
__device__ float block_sum(float v, float *red) {
    v = group_sum<64>(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += red[w];
    __syncthreads();
    return v;
}

// One workgroup of THREADS threads merges DS of the D output dimensions of
// one (request, query head); gridDim.z = D / DS slices.  SPEC: no load waits
// for the request length; O, m and l of all max_splits splits are requested
// at once (rows past the request's last split are masked afterwards, never
// used), so one memory round trip covers the inputs.  Without SPEC the O rows
// are requested once the length is known, only for the request's splits: one
// more round trip, but no reads of rows a short request in a ragged batch
// does not have.
template <int D, int DS, int THREADS, bool SPEC>
__global__ void __launch_bounds__(THREADS) combine_kernel(const CombineParams p) {
    extern __shared__ float sml[];         // [2][max_splits]: m, then l and finally the weights
    constexpr int DQ = DS / 4;             // threads per split row (float4 each)
    constexpr int SG = THREADS / DQ;       // split rows covered by one pass of the block
    constexpr int JC = 16;                 // split rows per thread whose loads are in flight together
    constexpr int NW = THREADS / 64;
    __shared__ float4 part[SG][DQ];
    __shared__ float red[NW];

    const int h = blockIdx.x, b = blockIdx.y, slice = blockIdx.z;
    const int Smax = p.max_splits;
    const size_t row = (size_t)b * p.Hq + h;
    const size_t base = row * Smax;
    const float *pm = p.part_m + base, *pl = p.part_l + base;
    const int dq = threadIdx.x % DQ, sg = threadIdx.x / DQ;
    const int dim0 = slice * DS + dq * 4;
    const float *po = p.part_o + base * D + dim0;
    float *smm = sml, *sww = sml + Smax;

    int S = Smax;
    if (p.seq_lens) {
        const int len = request_len(p.seq_lens, b, Smax * p.split, Smax * p.split);
        S = (len + p.split - 1) / p.split;
    }
    const int Sload = SPEC ? Smax : S;
    float4 o[JC];
#pragma unroll
    for (int j = 0; j < JC; ++j) {
        const int s = sg + SG * j;
        o[j] = s < Sload ? *reinterpret_cast<const float4 *>(po + (size_t)s * D) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int s = threadIdx.x; s < Smax; s += THREADS) {
        smm[s] = pm[s];
        sww[s] = pl[s];
    }

    float mx = -INFINITY;
    for (int s = threadIdx.x; s < S; s += THREADS)
        if (sww[s] > 0.f) mx = fmaxf(mx, smm[s]);
    mx = block_max<NW>(mx, red);

    float lsum = 0.f;
    for (int s = threadIdx.x; s < Smax; s += THREADS) {
        const float l = sww[s];
        const float w = (s < S && l > 0.f) ? l * exp2_fast((smm[s] - mx) * kLog2e) : 0.f;
        sww[s] = w;
        lsum += w;
    }
    lsum = block_sum<NW>(lsum, red);       // its barrier also publishes the weights

    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < S; s0 += SG * JC) {
        if (s0 > 0) {
#pragma unroll
            for (int j = 0; j < JC; ++j) {
                const int s = s0 + sg + SG * j;
                o[j] = s < S ? *reinterpret_cast<const float4 *>(po + (size_t)s * D)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
#pragma unroll
        for (int j = 0; j < JC; ++j) {
            const int s = s0 + sg + SG * j;
            const float w = s < S ? sww[s] : 0.f;
            if (w > 0.f) {       // a split without tokens has an unwritten O row
                a.x = fmaf(w, o[j].x, a.x);
                a.y = fmaf(w, o[j].y, a.y);
                a.z = fmaf(w, o[j].z, a.z);
                a.w = fmaf(w, o[j].w, a.w);
            }
        }
    }
    if constexpr (SG > 1) {
        part[sg][dq] = a;
        __syncthreads();
    }
    if (sg == 0) {
#pragma unroll
        for (int j = 1; j < SG; ++j) {
            const float4 q = part[j][dq];
            a.x += q.x;
            a.y += q.y;
            a.z += q.z;
            a.w += q.w;
        }
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        const size_t o0 = row * D + dim0;
        store_out(p.out, o0 + 0, a.x * inv, p.out_dtype);
        store_out(p.out, o0 + 1, a.y * inv, p.out_dtype);
        store_out(p.out, o0 + 2, a.z * inv, p.out_dtype);
        store_out(p.out, o0 + 3, a.w * inv, p.out_dtype);
    }
    if (threadIdx.x == 0 && slice == 0 && p.lse) p.lse[row] = lsum > 0.f ? mx + logf(lsum) : -INFINITY;
}

// Speculative O loads for a single request or when every request has the
// full length; a batch with lengths reads only the rows it has.  Measured on
// MI355X: B=64 ragged paged batch (lengths U[1024, 16384], 64 splits at most,
// 38.5 on average) 492.6 -> 486.6 us per call; B=4 equal lengths unchanged.
template <int D, int DS, int THREADS>
hipError_t launch_shaped(const CombineParams &p, hipStream_t stream) {
    dim3 grid(p.Hq, p.B, D / DS);
    const size_t smem = 2 * (size_t)p.max_splits * sizeof(float);
    if (p.B == 1 || !p.seq_lens)
        hipLaunchKernelGGL((combine_kernel<D, DS, THREADS, true>), grid, dim3(THREADS), smem, stream, p);
    else
        hipLaunchKernelGGL((combine_kernel<D, DS, THREADS, false>), grid, dim3(THREADS), smem, stream, p);
    return hipGetLastError();
}

// (launch_shaped: one workgroup of 256 threads covers all D dimensions of a
// (request, query head); 32 to 128 dimensions per workgroup with 64 to 256
// threads measured alike.)

// One workgroup of 256 threads per (request, query row); output quad dq (dims
// 4 dq .. 4 dq + 3) is shared by P adjacent lanes, lane ph taking splits ph,
// ph + P, ...  Each lane requests the O quads, m and l of up to 16 of its
// splits at once (one memory round trip: the 32k GQA shape's 128 splits are
// 16 per lane), keeps a running max-rescaled state over them in split order,
// and the P lanes of a quad merge by a lane butterfly.  No LDS, no barrier;
// fixed order, so bitwise repeatable.
template <int D>
__global__ void __launch_bounds__(256) combine_lanes_kernel(const CombineParams p) {
    constexpr int THREADS = 256, DQ = D / 4, P = THREADS / DQ, CH = 16;
    const int tid = threadIdx.x, dq = tid / P, ph = tid % P;
    const int b = blockIdx.y;
    const size_t row = (size_t)b * p.Hq + blockIdx.x;
    const int Smax = p.max_splits;
    int S = Smax;
    if (p.seq_lens) {
        const int len = request_len(p.seq_lens, b, Smax * p.split, Smax * p.split);
        S = (len + p.split - 1) / p.split;
    }
    const float *po = p.part_o + row * Smax * D + 4 * dq;
    const float *pm = p.part_m + row * Smax, *pl = p.part_l + row * Smax;
    float M = -INFINITY, L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = ph; j0 < S; j0 += P * CH) {
        float4 o[CH];
        float mv[CH], lv[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int j = j0 + P * c;
            const bool ok = j < S;
            o[c] = ok ? *reinterpret_cast<const float4 *>(po + (size_t)j * D) : make_float4(0.f, 0.f, 0.f, 0.f);
            mv[c] = ok ? pm[j] : -INFINITY;
            lv[c] = ok ? pl[j] : 0.f;
        }
        float mx = M;
#pragma unroll
        for (int c = 0; c < CH; ++c)
            if (lv[c] > 0.f) mx = fmaxf(mx, mv[c]);
        const float fr = M == -INFINITY ? 0.f : exp2_fast((M - mx) * kLog2e);
        L *= fr;
        acc.x *= fr;
        acc.y *= fr;
        acc.z *= fr;
        acc.w *= fr;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (lv[c] > 0.f) {      // a split without tokens has an unwritten O row
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
#pragma unroll
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
        const size_t o0 = row * D + 4 * dq;
        store_out(p.out, o0 + 0, acc.x * inv, p.out_dtype);
        store_out(p.out, o0 + 1, acc.y * inv, p.out_dtype);
        store_out(p.out, o0 + 2, acc.z * inv, p.out_dtype);
        store_out(p.out, o0 + 3, acc.w * inv, p.out_dtype);
        if (dq == 0 && p.lse) p.lse[row] = L > 0.f ? M + logf(L) : -INFINITY;
    }
}

// Which combine: the lane kernel issues every load of a row at once but each
// lane also reads the m and l of its own splits, which costs more than it
// saves once the splits are many.  Measured on MI355X, three runs each
// (bench.py, step time with the lane kernel against the LDS one): 4 splits
// (tiny MHA) 9.0 against 9.5-9.95 us; 16 (Llama-2-shaped MHA) 17.65-17.72
// against 18.40-18.58; 128 (32k GQA) 29.7-29.95 against 29.0-29.5; 128 with
// 256 rows (B=4, N=128k) alike.
inline bool use_lane_combine(const CombineParams &p) { return p.max_splits <= 32; }

}  // namespace

hipError_t launch_combine(const CombineParams &p, hipStream_t stream) {
    if (use_lane_combine(p)) {
        dim3 grid(p.Hq, p.B);
        if (p.d == 64)
            hipLaunchKernelGGL((combine_lanes_kernel<64>), grid, dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((combine_lanes_kernel<128>), grid, dim3(256), 0, stream, p);
        return hipGetLastError();
    }
    return p.d == 64 ? launch_shaped<64, 64, 256>(p, stream) : launch_shaped<128, 128, 256>(p, stream);
}

}  // namespace fd
