// fd_partial_valu.hip -- split-partial kernel on the vector ALUs, every dtype.
//
// One workgroup (4 waves) per (request b, KV head, split s) covers the whole
// GQA group of that KV head, so each K/V row is read from HBM once for all of
// the group's query heads (handbook page "FlashAttention and inference
// kernels", exercise 3 and the list of improvements after the paged kernel).
//
// Data layout in registers: a cache row (one token of one KV head, d
// elements) is read as 16-byte pieces by LPR = d / E consecutive lanes (E
// elements per 16 bytes), so one wave instruction reads RPW = 64 / LPR whole
// rows.  The dot product of a row with each query head is a per-lane partial
// sum followed by a butterfly over the LPR lanes (DPP).  Each lane group of
// LPR lanes keeps its own online-softmax state (m, l, O) over the rows it
// reads; the states are merged at the end of the split, first across the lane
// groups of a wave and then across the four waves through LDS, by the same
// max-rescale rule the combine kernel uses.
//
// Softmax inside a split:
//   SYNC -- the FlashAttention recurrence with a running maximum, applied once
//     per R rows (page "FlashAttention and inference kernels", section
//     "FlashAttention: tiling plus online softmax").
//   UNIFIED -- p = exp(s - phi) with the fixed constant phi and plain sums, no
//     maximum at all (page "FlashDecoding++: Faster Large Language Model
//     Inference on GPUs", "Asynchronized Softmax with Unified Max Value",
//     Eq. 3 and Eq. 4).  Every valid score is checked against [lo, hi]; if any
//     query head of the group saw a score outside it, the workgroup rescans
//     the split with SYNC and replaces the partials of exactly the flagged
//     heads ("The Overflow Fallback: Recomputation").
#include "fd_device.h"
#include "fd_merge.h"

namespace fd {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int DT, int D, int GMAX>
struct Cfg {
    static constexpr int E = Storage<DT>::E;
    static constexpr int LPR = D / E;                // lanes per cache row
    static constexpr int RPW = 64 / LPR;             // rows per wave instruction
    static constexpr int R = GMAX >= 8 ? 2 : 4;      // rows per lane per step
    static constexpr int TOK_STEP = kWaves * RPW * R;
    static constexpr int BYTES = Storage<DT>::bytes;
};

template <int DT, int D, int GMAX>
struct State {
    static constexpr int E = Cfg<DT, D, GMAX>::E;
    float m[GMAX], l[GMAX], acc[GMAX][E];
    bool bad[GMAX];
    __device__ void init(float m0) {
#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
            m[g] = m0;
            l[g] = 0.f;
            bad[g] = false;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
        }
    }
};

// Element offset of (token t, dim 0) of KV head kvh of request b; ok is
// cleared when a paged entry points outside the pool.
template <bool PAGED, int D>
__device__ __forceinline__ size_t row_offset(const PartialParams &p, int b, int kvh, int t, bool &ok) {
    size_t row;
    if constexpr (PAGED) {
        const int phys = p.block_table[(size_t)b * p.max_blocks + t / p.page_size];
        ok = ok && phys >= 0 && phys < p.num_pages;
        row = ((size_t)(ok ? phys : 0) * p.page_size + t % p.page_size) * p.Hkv + kvh;
    } else {
        row = ((size_t)b * p.kv_capacity + t) * p.Hkv + kvh;
    }
    return row * D;
}

// lim[g]: query row g sees tokens < lim[g] of the split (causal rows);
// sc: the score scale in log2 units (times the KV head's K scale for 8-bit caches)
template <int DT, int D, int GMAX, bool PAGED, bool UNIFIED>
__device__ void scan_split(const PartialParams &p, int b, int kvh, int t0, int t1, float sc, const int (&lim)[GMAX],
                           const float (&qv)[GMAX][Cfg<DT, D, GMAX>::E], State<DT, D, GMAX> &st) {
    using C = Cfg<DT, D, GMAX>;
    constexpr int E = C::E, LPR = C::LPR, RPW = C::RPW, R = C::R;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rg = lane / LPR, c = lane % LPR;
    const char *kb = static_cast<const char *>(p.k);
    const char *vb = static_cast<const char *>(p.v);

    for (int tb = t0; tb < t1; tb += C::TOK_STEP) {
        uint4 kr[R], vr[R];
        bool ok[R];
        int tok[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int t = tb + (wave * R + r) * RPW + rg;
            tok[r] = t;
            ok[r] = t < t1;
            const size_t off = (row_offset<PAGED, D>(p, b, kvh, ok[r] ? t : t0, ok[r]) + (size_t)c * E) * C::BYTES;
            kr[r] = ok[r] ? load_piece<DT>(kb + off) : make_uint4(0, 0, 0, 0);
            vr[r] = ok[r] ? load_piece<DT>(vb + off) : make_uint4(0, 0, 0, 0);
        }
        float s[R][GMAX];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float kf[E];
            unpack<DT>(kr[r], kf);
#pragma unroll
            for (int g = 0; g < GMAX; ++g) {
                float dot = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) dot = fmaf(qv[g][e], kf[e], dot);
                dot = group_sum<LPR>(dot);
                s[r][g] = (ok[r] && tok[r] < lim[g]) ? dot * sc : -INFINITY;
            }
        }
        float vf[R][E];
#pragma unroll
        for (int r = 0; r < R; ++r) unpack<DT>(vr[r], vf[r]);
#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
            float mref;
            if constexpr (UNIFIED) {
#pragma unroll
                for (int r = 0; r < R; ++r)
                    st.bad[g] = st.bad[g] || (s[r][g] != -INFINITY && (s[r][g] < p.lo2 || s[r][g] > p.hi2));
                mref = p.phi2;
            } else {
                float mt = s[0][g];
#pragma unroll
                for (int r = 1; r < R; ++r) mt = fmaxf(mt, s[r][g]);
                const float mn = fmaxf(st.m[g], mt);
                const float corr = rescale(st.m[g], mn);
                st.l[g] *= corr;
#pragma unroll
                for (int e = 0; e < E; ++e) st.acc[g][e] *= corr;
                st.m[g] = mn;
                mref = mn;
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float pr = mref == -INFINITY ? 0.f : exp2_fast(s[r][g] - mref);
                st.l[g] += pr;
#pragma unroll
                for (int e = 0; e < E; ++e) st.acc[g][e] = fmaf(pr, vf[r][e], st.acc[g][e]);
            }
        }
    }
}

// Merge the lane groups of each wave: butterfly over lanes with equal chunk.
template <int DT, int D, int GMAX>
__device__ void merge_wave(State<DT, D, GMAX> &st) {
    using C = Cfg<DT, D, GMAX>;
#pragma unroll
    for (int off = C::LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
            const float mp = __shfl_xor(st.m[g], off);
            const float lp = __shfl_xor(st.l[g], off);
            const float mn = fmaxf(st.m[g], mp);
            const float a = rescale(st.m[g], mn), bb = rescale(mp, mn);
            st.l[g] = st.l[g] * a + lp * bb;
#pragma unroll
            for (int e = 0; e < C::E; ++e) {
                const float ap = __shfl_xor(st.acc[g][e], off);
                st.acc[g][e] = st.acc[g][e] * a + ap * bb;
            }
            st.m[g] = mn;
        }
    }
}

template <int D, int GMAX>
struct Smem {
    float m[kWaves][GMAX];
    float l[kWaves][GMAX];
    float acc[kWaves][GMAX][D];
    uint32_t bad[kWaves];
};

// Wave states -> LDS -> the split's partial for the heads in `write_mask`
// (device-scope stores for the single-launch merge).
template <int DT, int D, int GMAX, bool FUSED>
__device__ void finish_split(const PartialParams &p, State<DT, D, GMAX> &st, Smem<D, GMAX> &sm, int b, int kvh,
                             int s, uint32_t write_mask, float vmul) {
    using C = Cfg<DT, D, GMAX>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    merge_wave(st);
    if (lane < C::LPR) {
#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
#pragma unroll
            for (int e = 0; e < C::E; ++e) sm.acc[wave][g][lane * C::E + e] = st.acc[g][e];
            if (lane == 0) {
                sm.m[wave][g] = st.m[g];
                sm.l[wave][g] = st.l[g];
            }
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < p.R * D; idx += kThreads) {
        const int g = idx / D, dim = idx % D;
        if (!((write_mask >> g) & 1u)) continue;
        float mm = sm.m[0][g];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) mm = fmaxf(mm, sm.m[w][g]);
        float L = 0.f, A = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = rescale(sm.m[w][g], mm);
            L += sm.l[w][g] * f;
            A += sm.acc[w][g][dim] * f;
        }
        float o = L > 0.f ? A / L : 0.f;
        if constexpr (DT == FP8) o *= vmul;
        const float m_nat = (L > 0.f && mm != -INFINITY) ? mm * kLn2 : -INFINITY;
        if (!FUSED && p.direct) {   // the row's only split: its partial is the result
            const size_t row = query_row(p, b, kvh, g);
            store_out(p.out, row * D + dim, o, p.out_dtype);
            if (dim == 0 && p.lse) p.lse[row] = L > 0.f ? m_nat + logf(L) : -INFINITY;
            continue;
        }
        const size_t slot = row_slot(p, b, kvh, g, s);
        store_partial<FUSED>(&p.part_o[slot * D + dim], o);
        if (dim == 0) {
            store_partial<FUSED>(&p.part_m[slot], m_nat);
            store_partial<FUSED>(&p.part_l[slot], L);
        }
    }
}

template <int D, int GMAX>
union VSmem {
    Smem<D, GMAX> st;
    float merge[merge_lds_floats(kFusedMaxRowParts, kMaxGroup, kThreads)];   // the single-launch merge
};

// FUSED: the single-launch merge (one split per workgroup; the last workgroup
// of a (request, KV head) merges its splits into out and lse, fd_merge.h).
template <int DT, int D, int GMAX, bool PAGED, bool FUSED>
__global__ void __launch_bounds__(kThreads) partial_valu_kernel(const PartialParams pk) {
    using C = Cfg<DT, D, GMAX>;
    constexpr int E = C::E;
    __shared__ VSmem<D, GMAX> vsm;
    __shared__ int ticket;
    Smem<D, GMAX> &sm = vsm.st;

    int b;
    const PartialParams p = tile_params(pk, b);
    const int kvh = blockIdx.y;
    const int s = split_index(blockIdx.x, blockIdx.z, kvh, p.Hkv, p.max_splits);
    const int G = p.R;                               // query rows of this workgroup
    const int len = request_len(p.seq_lens, b, p.kv_capacity, p.max_splits * p.split);
    const int tl = tile_len(p, len);                 // tokens the tile's rows see
    const int t0 = s * p.split;
    const int t1 = min(t0 + p.split, tl);

    if (t0 >= t1) {   // empty split: nothing to read
        if (threadIdx.x < G && !p.recompute_rows) {
            const size_t slot = row_slot(p, b, kvh, threadIdx.x, s);
            if (!p.direct) {   // the single launch's merge reads only splits with tokens
                p.part_m[slot] = -INFINITY;
                p.part_l[slot] = 0.f;
            }
            if (p.flags) p.flags[slot] = 0;
        }
        if ((FUSED || p.direct) && !p.recompute_rows && tl <= 0 && s == 0) write_empty_rows<D>(p, b, kvh, kThreads);
        return;
    }
    // whole-row fallback, second pass: only rows flagged in some split of the request
    uint32_t rows_to_write = G >= 32 ? 0xffffffffu : ((1u << G) - 1u);
    if (p.recompute_rows) {
        rows_to_write = rows_flagged_in_request(p, b, kvh, (len + p.split - 1) / p.split);
        if (!rows_to_write) return;
    }
    float sc = p.scale_log2, vmul = p.v_mult;
    if constexpr (DT == FP8) {
        if (p.k_scales) sc *= p.k_scales[kvh];
        if (p.v_scales) vmul = p.v_scales[kvh];
    }

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane % C::LPR;
    float qv[GMAX][E];
    int lim[GMAX];
    const char *qb = static_cast<const char *>(p.q);
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
        lim[g] = row_limit(p, len, t1, g);
        if (g < G) {
            const size_t qrow = query_row(p, b, kvh, g);
            if constexpr (DT == FP8) {   // q is f16 or bf16
                const uint4 raw = load16(qb + (qrow * D + (size_t)c * E) * 2);
                if (p.q_dtype == BF16)
                    unpack<BF16>(raw, qv[g]);
                else
                    unpack<F16>(raw, qv[g]);
            } else {
                const size_t off = (qrow * D + (size_t)c * E) * C::BYTES;
                unpack<DT>(load16(qb + off), qv[g]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) qv[g][e] = 0.f;
        }
    }

    const uint32_t all = G >= 32 ? 0xffffffffu : ((1u << G) - 1u);
    State<DT, D, GMAX> st;
    uint32_t badmask = 0;
    if (p.unified && !p.recompute_rows) {
        st.init(p.phi2);
        scan_split<DT, D, GMAX, PAGED, true>(p, b, kvh, t0, t1, sc, lim, qv, st);
        uint32_t mine = 0;
#pragma unroll
        for (int g = 0; g < GMAX; ++g)
            if (__any(st.bad[g])) mine |= 1u << g;
        if (lane == 0) sm.bad[wave] = mine;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kWaves; ++w) badmask |= sm.bad[w];
        badmask &= all;
        // whole-row fallback: every row's unified partial now, the flagged rows'
        // splits all rewritten by a second pass
        finish_split<DT, D, GMAX, FUSED>(p, st, sm, b, kvh, s, p.row_fallback ? all : all & ~badmask, vmul);
        if (badmask && !p.row_fallback) {   // synchronized recompute of the flagged heads
            __syncthreads();
            st.init(-INFINITY);
            scan_split<DT, D, GMAX, PAGED, false>(p, b, kvh, t0, t1, sc, lim, qv, st);
            finish_split<DT, D, GMAX, FUSED>(p, st, sm, b, kvh, s, badmask, vmul);
        }
        if (threadIdx.x == 0 && badmask && p.fallback_count)
            atomicAdd(p.fallback_count, __builtin_popcount(badmask));
    } else {
        st.init(-INFINITY);
        scan_split<DT, D, GMAX, PAGED, false>(p, b, kvh, t0, t1, sc, lim, qv, st);
        finish_split<DT, D, GMAX, FUSED>(p, st, sm, b, kvh, s, rows_to_write, vmul);
    }
    if (p.flags && threadIdx.x < G && !p.recompute_rows)
        p.flags[row_slot(p, b, kvh, threadIdx.x, s)] = (badmask >> threadIdx.x) & 1u;
    if constexpr (FUSED) {
        const int nb = (tl + p.split - 1) / p.split;        // splits holding tokens
        __syncthreads();                                     // the merge area overlays the epilogue's
        if (arrive_last(&p.tickets[(size_t)blockIdx.z * p.Hkv + kvh], nb, &ticket))
            merge_rows<D, kThreads>(p, b, kvh, nb, vsm.merge);
    }
}

template <int DT, int D, int GMAX, bool PAGED>
hipError_t launch(const PartialParams &p, hipStream_t stream) {
    dim3 grid(p.max_splits, p.Hkv, p.B * p.q_tiles);
    if (p.tickets)
        hipLaunchKernelGGL((partial_valu_kernel<DT, D, GMAX, PAGED, true>), grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((partial_valu_kernel<DT, D, GMAX, PAGED, false>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int DT, int D, int GMAX>
hipError_t by_paged(const PartialParams &p, hipStream_t s) {
    return p.page_size ? launch<DT, D, GMAX, true>(p, s) : launch<DT, D, GMAX, false>(p, s);
}

template <int DT, int D>
hipError_t by_group(const PartialParams &p, hipStream_t s) {
    if (p.R <= 1) return by_paged<DT, D, 1>(p, s);
    if (p.R <= 2) return by_paged<DT, D, 2>(p, s);
    if (p.R <= 4) return by_paged<DT, D, 4>(p, s);
    if (p.R <= 8) return by_paged<DT, D, 8>(p, s);
    return by_paged<DT, D, 16>(p, s);
}

template <int DT>
hipError_t by_dim(const PartialParams &p, hipStream_t s) {
    return p.d == 64 ? by_group<DT, 64>(p, s) : by_group<DT, 128>(p, s);
}

}  // namespace

hipError_t launch_partial_valu(const PartialParams &p, hipStream_t stream) {
    switch (p.dtype) {
    case F32: return by_dim<F32>(p, stream);
    case F16: return by_dim<F16>(p, stream);
    case FP8: return by_dim<FP8>(p, stream);
    default: return by_dim<BF16>(p, stream);
    }
}

}  // namespace fd
