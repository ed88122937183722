// fd_partial_mfma.h -- split-partial kernel on the gfx950 matrix cores
// (f16 / bf16 / E4M3 caches).  Included by one translation unit per
// instantiation type (fd_partial_mfma_<type>.hip), which keeps each unit's
// compile short; fd_partial_mfma.hip holds the dispatch.
//
// Work decomposition (as in the VALU kernel): one workgroup per (request b,
// KV head, split s) covering all query rows of that KV head -- its G query
// heads times the request's q_len query tokens, up to 32 rows; more rows go
// in query tiles, each its own slice of the grid -- so K and V are read from
// HBM once per group (handbook page "FlashAttention and inference kernels",
// exercise 3).  Each wave walks 16-token blocks of the split.  Four or more
// query tiles per KV head run in workgroups of four tiles that share each
// K/V block (shared_kv_mfma_kernel below).
// 8-bit (E4M3) caches are widened exactly to the 16-bit operand type in
// registers before the LDS tiles; everything after the tiles is shared.
//
// Per block:
//   loads: K and V rows with 16-byte non-temporal loads, 16 lanes per 256-byte
//      row (coalesced), written to wave-private LDS tiles.  The K tile's
//      16-byte chunks are XOR-swizzled by (row & 15), the V tile's by
//      2 * (row & 7), so the two operand reads below are bank-conflict-free.
//   S^T[token][head] = K q^T: D / 32 v_mfma_f32_16x16x32; A = the K tile
//      (lane l: token l % 16, dims 8 * (l / 16) .. + 8 of each 32-dim step),
//      B = q of the group's query rows (rows >= R zero).  Result lane l: row l % 16,
//      tokens 4 * (l / 16) .. + 3 of the block.
//   softmax in that layout: SYNC keeps a running per-head maximum across the
//      wave's blocks (page "FlashAttention and inference kernels", section
//      "FlashAttention: tiling plus online softmax"); UNIFIED uses the fixed
//      constant phi and checks every score against [lo, hi] (page
//      "FlashDecoding++: Faster Large Language Model Inference on GPUs",
//      Eq. 3 / Eq. 4 and "The Overflow Fallback: Recomputation").
//   O[head][dim] += P V: D / 16 slices of v_mfma_f32_16x16x16.  The result
//      layout of S^T is the A-operand layout of P (head l % 16, tokens
//      4 * (l / 16) + e), so the probabilities stay in registers; they enter
//      for bf16 caches (and under unified max) as a 16-bit high part plus the
//      16-bit rounding of the fp32 residual (two MFMAs), which keeps the
//      weights to about 14 bits or better; with f16 and 8-bit caches under the
//      synchronized softmax, as one f16 operand rounded to nearest against
//      f16 V tiles.
//      B (lane j of lane group q: V[token 4q + k][dim j] of the slice) comes
//      from the V tile with ds_read_b64_tr_b16, whose result is lane j,
//      element k = element j % 4 of the 8-byte row addressed by lane 4k + j / 4
//      of the group.  O lands with heads on rows: 4 registers per slice,
//      independent of G, and no cross-lane reduction at the end.
// The wave states are merged across waves by the max-rescale rule and
// written as one split partial.
#pragma once

#include <type_traits>

#include "fd_device.h"
#include "fd_merge.h"

namespace fd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(const uint4 &a, const uint4 &b, f32x4 c) {
    if constexpr (DT == BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                      c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                     0, 0, 0);
}

// O += P V for one 16-dim slice: A = 4 probabilities, B = 4 values (16-bit each)
template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x16(const s16x4 &a, const s16x4 &b, f32x4 c) {
    if constexpr (DT == BF16)
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c,
                                                    0, 0, 0);
}

// Four fp32 probabilities -> 16-bit high parts and 16-bit parts of the exact
// fp32 residuals, packed as MFMA operands.  bf16: the high part is the top
// 16 bits (truncation); f16: round toward zero.  Either way hi + lo carries
// the weight to a relative error below 2^-14.
template <int DT>
__device__ __forceinline__ void split_probs(const float (&pr)[4], s16x4 &hi, s16x4 &lo) {
    uint32_t h[2], l[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float a = pr[2 * i], b = pr[2 * i + 1];
        if constexpr (DT == BF16) {
            const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
            const float ra = a - __uint_as_float(ua & 0xffff0000u);
            const float rb = b - __uint_as_float(ub & 0xffff0000u);
            h[i] = __builtin_amdgcn_perm(ub, ua, 0x07060302u);      // [ua.hi16 | ub.hi16 << 16]
            l[i] = __builtin_amdgcn_perm(__float_as_uint(rb), __float_as_uint(ra), 0x07060302u);
        } else {
            const auto hh = __builtin_amdgcn_cvt_pkrtz(a, b);
            const float ra = a - (float)hh[0], rb = b - (float)hh[1];
            const auto ll = __builtin_amdgcn_cvt_pkrtz(ra, rb);
            h[i] = __builtin_bit_cast(uint32_t, hh);
            l[i] = __builtin_bit_cast(uint32_t, ll);
        }
    }
    hi = __builtin_bit_cast(s16x4, make_uint2(h[0], h[1]));
    lo = __builtin_bit_cast(s16x4, make_uint2(l[0], l[1]));
}

constexpr int kBlk = 16;   // tokens per MFMA block

// The wave of this thread among the WAVES waves that share one split (a
// kernel whose waves each scan a split of their own passes WAVES = 1).
template <int WAVES>
__device__ __forceinline__ int head_wave() {
    return WAVES == 1 ? 0 : (int)(threadIdx.x >> 6) % WAVES;
}

// Register budget and the order of the P x V operand reads, by query rows
// per KV head (measured on MI355X, each A/B in one session).  Up to four
// rows: at least 4 waves per SIMD (128 registers), each V slice read just
// before its MFMAs (32k GQA: 23.4 us against 23.7 with the alternative).
// More rows: at least 2 waves per SIMD, which leaves the compiler room to
// read all V slices before the first MFMA (B=4, N=128k, 8 rows: 344.5 us
// against 351.5; B=64 paged: 491.8 against 498.7; 4 query tokens of the 32k
// GQA shape, 16 rows: 24.4 against 25.3).
__host__ __device__ constexpr int min_waves_per_eu(int GMAX) { return GMAX > 4 ? 2 : 4; }

// 16-row tiles of query rows per KV head: the MFMA B operand holds 16 rows,
// so up to 32 rows take two tiles that share each block's K and V tiles.
__host__ __device__ constexpr int row_tiles(int GMAX) { return (GMAX + 15) / 16; }
__host__ __device__ constexpr bool batch_v_reads(int GMAX) { return GMAX > 4; }

// Instantiation type T: the 16-bit operand type of the matrix instructions
// (F16 or BF16, also the type of q), plus 16 when the cache holds 8-bit E4M3
// values that are widened to it in registers (exactly: an E4M3 value has four
// significant bits and its exponent range fits both 16-bit types).
constexpr int kF8 = 16;
__host__ __device__ constexpr int op_of(int T) { return T & 15; }
__host__ __device__ constexpr bool f8_of(int T) { return T >= kF8; }

// P x V operand type.  f16 caches, and 8-bit caches (whose widened V values
// are exact in f16), take f16 for both operands under the synchronized
// softmax: every probability lies in [0, 1], so one MFMA on P rounded to
// nearest f16 (relative error <= 2^-11, absolute <= 2^-25 below the normal
// range) replaces the high/residual pair (Llama-2-shaped MHA, f16: partial
// 13.40-13.44 against 13.57-13.63 us).  bf16 caches keep the pair, bf16's
// 8-bit significand being too coarse for P alone, and so does the
// unified-max softmax, since e^{s - phi} may exceed f16's range.
__host__ __device__ constexpr bool pv_single(int T, bool UNIFIED) {
    return (f8_of(T) || op_of(T) == F16) && !UNIFIED;
}
__host__ __device__ constexpr int pv_type(int T, bool UNIFIED) { return pv_single(T, UNIFIED) ? F16 : op_of(T); }

// How a block's cache rows are loaded: 16 bytes per lane, LPR lanes per row.
template <int T, int D>
struct KLoad {
    static constexpr int EB = f8_of(T) ? 1 : 2;     // bytes per cache element
    static constexpr int LPR = D * EB / 16;         // lanes per row
    static constexpr int RPI = 64 / LPR;            // rows per load instruction
    static constexpr int LI = kBlk / RPI;           // load instructions per block (K, and again V)
};

template <int D, int GMAX, int WAVES>
struct MCfg {
    static constexpr int KS = D / 32;                 // MFMA k-steps over the head dimension (QK)
    static constexpr int SL = D / 16;                 // 16-dim output slices (PV)
    static constexpr int LPR = D / 8;                 // 16-byte chunks per 16-bit tile row
    static constexpr int ROWB = D * 2;                // bytes per tile row
    static constexpr int THREADS = 64 * WAVES;
};

template <int D, int GMAX, int WAVES>
struct MSmem {
    using C = MCfg<D, GMAX, WAVES>;
    static constexpr int GQ = (GMAX + 3) / 4;      // head quads
    struct Handover {                             // wave 1's state, lane for lane, for wave 0
        float4 o[D / 16][64];
        float l[16], m[16];
    };
    union {
        uint4 k[WAVES][kBlk * C::ROWB / 16];      // wave-private K tiles ...
        // ... reused by the epilogue once both waves of a head are done (one wave: no hand-over)
        typename std::conditional<(WAVES > 1), Handover, char>::type ho;
    };
    uint4 v[WAVES][kBlk * C::ROWB / 16];          // wave-private V tiles
    float corr[WAVES][16];                        // running-max rescale factors per head row
    uint32_t bad[WAVES];
};

template <int D, int GMAX>
struct MState {
    float m, l;             // head l % 16 (S^T layout)
    bool bad;
    f32x4 o[D / 16];        // O[head 4 * (l / 16) + r][16 * slice + l % 16]
    __device__ void init(float m0) {
        m = m0;
        l = 0.f;
        bad = false;
#pragma unroll
        for (int i = 0; i < D / 16; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
};

// Rows of one 16-token block: where they live and whether their page exists.
struct BlockRows {
    int tb;          // first token of the block
    size_t row0;     // element offset of (token tb, kvh, dim 0); rows step by Hkv * d
    bool page_ok;
};

// The split's block-table entries, one per lane (pages t0 / page .. + 63),
// read once per workgroup; blocks beyond them read the table directly.
struct PageCache {
    int base;        // first page index held
    int entry;       // this lane's entry: page base + lane
};

template <bool PAGED>
__device__ __forceinline__ PageCache load_pages(const PartialParams &p, int b, int t0, int t1) {
    PageCache pc{0, -1};
    if constexpr (PAGED) {
        const int lane = threadIdx.x & 63;
        pc.base = t0 / p.page_size;
        const int last = (t1 - 1) / p.page_size;          // t1 > t0 here
        if (pc.base + lane <= last) pc.entry = p.block_table[(size_t)b * p.max_blocks + pc.base + lane];
    }
    return pc;
}

template <int D, bool PAGED>
__device__ __forceinline__ BlockRows block_rows(const PartialParams &p, const PageCache &pc, int b, int kvh, int tb,
                                                int t1) {
    BlockRows r;
    r.tb = tb;
    r.page_ok = true;
    const size_t head_off = (size_t)kvh * D;
    if (tb >= t1) {                                       // past the split: every row reads the safe row
        r.page_ok = false;
        r.row0 = head_off;
        return r;
    }
    if constexpr (PAGED) {
        const int pg = tb / p.page_size;                  // wave-uniform
        const int phys = pg - pc.base < 64 ? __builtin_amdgcn_readlane(pc.entry, pg - pc.base)
                                           : p.block_table[(size_t)b * p.max_blocks + pg];
        r.page_ok = phys >= 0 && phys < p.num_pages;
        r.row0 = (((size_t)(r.page_ok ? phys : 0) * p.page_size + tb % p.page_size) * p.Hkv) * D + head_off;
    } else {
        r.row0 = (((size_t)b * p.kv_capacity + tb) * p.Hkv) * D + head_off;
    }
    return r;
}

// Block loads go through buffer resources: the wave-uniform base is the
// block's first row, each lane's byte offset within a block is the same for
// every block (computed once), and rows past the block's valid range lie
// beyond num_records, so the hardware returns zeros for them without a memory
// access.  Word 3 of a raw buffer resource on this GPU family: 32-bit data
// format, no swizzle, no stride.
constexpr int32_t kBufferWord3 = 0x00020000;
constexpr int kLoadNT = 2;                            // cache policy: non-temporal (streamed once)

template <int LI>
struct LaneOffsets {
    uint32_t k[LI], v[LI];
};

template <int T, int D>
__device__ __forceinline__ LaneOffsets<KLoad<T, D>::LI> lane_offsets(const PartialParams &p) {
    using L = KLoad<T, D>;
    const int lane = threadIdx.x & 63;
    const int rg = lane / L::LPR, ch = lane % L::LPR;
    const uint32_t rbytes = (uint32_t)p.Hkv * D * L::EB;   // bytes between consecutive tokens of a head
    LaneOffsets<L::LI> o;
#pragma unroll
    for (int i = 0; i < L::LI; ++i) {
        const int r = i * L::RPI + rg;
        // 16-bit K chunks arrive XOR-swizzled by row; 8-bit rows are swizzled
        // when widened into the tile
        o.k[i] = r * rbytes + 16 * (f8_of(T) ? ch : (ch ^ (r & (L::LPR - 1))));
        o.v[i] = r * rbytes + 16 * ch;
    }
    return o;
}

__device__ __forceinline__ const char *uniform_ptr(const char *ptr) {
    const uint64_t a = reinterpret_cast<uint64_t>(ptr);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return reinterpret_cast<const char *>(((uint64_t)hi << 32) | lo);
}

// K and V of a block, 16 bytes per lane each.
template <int T, int D>
__device__ __forceinline__ void load_block(const PartialParams &p, const BlockRows &br, int t1,
                                           const LaneOffsets<KLoad<T, D>::LI> &off,
                                           uint4 (&kr)[KLoad<T, D>::LI], uint4 (&vr)[KLoad<T, D>::LI]) {
    using C = KLoad<T, D>;
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    const int valid = br.page_ok ? max(0, min(kBlk, t1 - br.tb)) : 0;   // wave-uniform
    // the resources are the same for every lane; say so, or the compiler wraps
    // each load in a loop over distinct resource values
    const int32_t bytes = __builtin_amdgcn_readfirstlane(valid * p.Hkv * D * C::EB);
    const char *kb = uniform_ptr(static_cast<const char *>(p.k) + br.row0 * C::EB);
    const char *vb = uniform_ptr(static_cast<const char *>(p.v) + br.row0 * C::EB);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(kb), 0, bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(vb), 0, bytes, kBufferWord3);
#pragma unroll
    for (int i = 0; i < C::LI; ++i) {
        const i32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rk, off.k[i], 0, kLoadNT);
        const i32x4 c = __builtin_amdgcn_raw_buffer_load_b128(rv, off.v[i], 0, kLoadNT);
        kr[i] = make_uint4(a.x, a.y, a.z, a.w);
        vr[i] = make_uint4(c.x, c.y, c.z, c.w);
    }
}

// 16 E4M3 values -> 16 values of the operand type, as two 16-byte chunks.
// gfx950's v_cvt_scalef32_pk_{bf16,f16}_fp8 with scale 1 converts two values
// per instruction, exactly for all 256 codes (checked on the hardware): an
// E4M3 value has four significant bits and its exponents fit both types.
template <int OP>
__device__ __forceinline__ void widen_f8(const uint4 &raw, uint4 &lo, uint4 &hi) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (OP == BF16) {
            o[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false));
            o[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true));
        } else {
            o[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, false));
            o[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, true));
        }
    }
    lo = make_uint4(o[0], o[1], o[2], o[3]);
    hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// Tile slot of 16-byte chunk c before the row swizzle.  8-bit caches widen
// 16 values per lane into chunks 2 ch and 2 ch + 1 of a row, so each of the
// two stores covers every other chunk of the row; with 256-byte rows (d =
// 128) chunks c and c + 8 share banks, and flipping bit 0 of the upper half
// spreads a store's eight lanes over all of them.  The tiles of 16-bit caches
// are written row-contiguous and need no flip.
template <int T>
__device__ __forceinline__ int chunk_slot(int c) {
    return f8_of(T) ? c ^ ((c >> 3) & 1) : c;
}

// The lanes of one wave exchange data through its private LDS tiles (and the
// rescale factors): a wavefront-scope fence plus a wave barrier keep every
// lane's LDS writes ordered before other lanes' reads, and those reads before
// the next writes.  Both are compiler-only; no s_barrier is emitted.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A block's K and V registers -> LDS tiles (the registers are free again
// afterwards).
template <int T, int D, bool UNIFIED>
__device__ __forceinline__ void write_tiles_at(const uint4 (&kr)[KLoad<T, D>::LI],
                                               const uint4 (&vr)[KLoad<T, D>::LI], char *ktile, char *vtile) {
    using C = MCfg<D, 1, 1>;
    using L = KLoad<T, D>;
    constexpr int DT = op_of(T);
    const int lane = threadIdx.x & 63;
    const int rg = lane / L::LPR, ch = lane % L::LPR;
    // tiles: 16-byte chunk c of row r lives at slot chunk_slot(c) ^ (r & (LPR-1))
    // (K) and chunk_slot(c) ^ (2 * (r & (LPR/2 - 1))) (V), LPR = D / 8 chunks per row
#pragma unroll
    for (int i = 0; i < L::LI; ++i) {
        const int r = i * L::RPI + rg;
        if constexpr (f8_of(T)) {   // this lane's 16 values are chunks 2 ch and 2 ch + 1
            uint4 k0, k1, v0, v1;
            widen_f8<DT>(kr[i], k0, k1);
            widen_f8<pv_type(T, UNIFIED)>(vr[i], v0, v1);
            const int c0 = chunk_slot<T>(2 * ch), c1 = chunk_slot<T>(2 * ch + 1);
            const int ks = r & (C::LPR - 1), vs = 2 * (r & (C::LPR / 2 - 1));
            *reinterpret_cast<uint4 *>(ktile + r * C::ROWB + 16 * (c0 ^ ks)) = k0;
            *reinterpret_cast<uint4 *>(ktile + r * C::ROWB + 16 * (c1 ^ ks)) = k1;
            *reinterpret_cast<uint4 *>(vtile + r * C::ROWB + 16 * (c0 ^ vs)) = v0;
            *reinterpret_cast<uint4 *>(vtile + r * C::ROWB + 16 * (c1 ^ vs)) = v1;
        } else {                    // K chunks arrive pre-swizzled
            *reinterpret_cast<uint4 *>(ktile + i * L::RPI * C::ROWB + lane * 16) = kr[i];
            *reinterpret_cast<uint4 *>(vtile + r * C::ROWB + 16 * (ch ^ (2 * (r & (C::LPR / 2 - 1))))) = vr[i];
        }
    }
}

// ... into the wave's private tiles.
template <int T, int D, int GMAX, int WAVES, bool UNIFIED>
__device__ __forceinline__ void write_tiles(const uint4 (&kr)[KLoad<T, D>::LI], const uint4 (&vr)[KLoad<T, D>::LI],
                                            MSmem<D, GMAX, WAVES> &sm) {
    const int wave = head_wave<WAVES>();
    write_tiles_at<T, D, UNIFIED>(kr, vr, reinterpret_cast<char *>(sm.k[wave]), reinterpret_cast<char *>(sm.v[wave]));
}

// One block from the wave's tiles into the running state.
// lim: this lane's query row (lane % 16) sees tokens < lim of the split;
// sc: the score scale in log2 units (scale * log2(e), times the KV head's K
// scale for 8-bit caches)
// ktile, vtile: the block's LDS tiles; corr: the wave's 16 rescale slots.
template <int T, int D, int GMAX, bool UNIFIED>
__device__ __forceinline__ void compute_tiles_at(const PartialParams &p, const BlockRows &br, int lim, float sc,
                                                 const uint4 (&qop)[D / 32], MState<D, GMAX> &st,
                                                 const char *ktile, const char *vtile, float *corr_lds) {
    using C = MCfg<D, GMAX, 1>;
    constexpr int DT = op_of(T);
    const int lane = threadIdx.x & 63;
    const int mrow = lane & 15, mq = lane >> 4;                 // MFMA coordinates

    // ---- S^T = K q^T on the matrix cores
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
        const int slot = chunk_slot<T>(4 * ks + mq) ^ (mrow & (C::LPR - 1));
        const uint4 a = *reinterpret_cast<const uint4 *>(ktile + mrow * C::ROWB + slot * 16);
        acc = mfma16x16x32<DT>(a, qop[ks], acc);
    }
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const bool ok = br.page_ok && br.tb + 4 * mq + r < lim;
        s[r] = ok ? acc[r] * sc : -INFINITY;
    }

    // ---- softmax for head mrow over these 16 tokens
    float pr[4];
    if constexpr (UNIFIED) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            st.bad = st.bad || (s[r] != -INFINITY && (s[r] < p.lo2 || s[r] > p.hi2));
            pr[r] = exp2_fast(s[r] - p.phi2);
            st.l += pr[r];
        }
    } else {
        float mt = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(st.m, mt);
        const float corr = rescale(st.m, mn);
        const bool moved = mn != st.m;
        st.m = mn;
        st.l *= corr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pr[r] = mn == -INFINITY ? 0.f : exp2_fast(s[r] - mn);
            st.l += pr[r];
        }
        // rescale the P x V accumulators (heads on rows 4 * (l / 16) + r)
        if (__any(moved)) {
            if (lane < 16) corr_lds[lane] = corr;
            wave_lds_sync();
            const float4 cf = *reinterpret_cast<const float4 *>(&corr_lds[4 * mq]);
#pragma unroll
            for (int i = 0; i < C::SL; ++i) {
                st.o[i][0] *= cf.x;
                st.o[i][1] *= cf.y;
                st.o[i][2] *= cf.z;
                st.o[i][3] *= cf.w;
            }
        }
    }

    // ---- O += P V on the matrix cores
    constexpr int PT = pv_type(T, UNIFIED);
    // this lane's 8-byte row of the transposing read: token 4 * mq + mrow / 4,
    // dims 16 * slice + 4 * (mrow % 4) .. + 3
    const int vrow = 4 * mq + (mrow >> 2);
    const char *vrow_base = vtile + vrow * C::ROWB;
    const int vsw = 2 * (vrow & (C::LPR / 2 - 1));
    auto read_v = [&](int i) {
        const int dim = 16 * i + 4 * (mrow & 3);
        const int slot = chunk_slot<T>(dim >> 3) ^ vsw;
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(vrow_base + slot * 16 + (dim & 7) * 2));
    };
    // with batch_v_reads every slice is read before the first MFMA, so that
    // the LDS latencies overlap; otherwise each just before its MFMAs
    s16x4 bv[C::SL];
    if constexpr (batch_v_reads(GMAX)) {
#pragma unroll
        for (int i = 0; i < C::SL; ++i) bv[i] = read_v(i);
    }
    s16x4 phi, plo;
    if constexpr (pv_single(T, UNIFIED)) {
        const f16x4 ph = {(_Float16)pr[0], (_Float16)pr[1], (_Float16)pr[2], (_Float16)pr[3]};
        phi = __builtin_bit_cast(s16x4, ph);
    } else {
        split_probs<DT>(pr, phi, plo);
    }
#pragma unroll
    for (int i = 0; i < C::SL; ++i) {
        const s16x4 b = batch_v_reads(GMAX) ? bv[i] : read_v(i);
        st.o[i] = mfma16x16x16<PT>(phi, b, st.o[i]);
        if constexpr (!pv_single(T, UNIFIED)) st.o[i] = mfma16x16x16<PT>(plo, b, st.o[i]);
    }
}

constexpr float kLazyRescale = 8.f;   // direct output: weights below 2^8, sums of up to 2^16 tokens in fp32

// Two consecutive blocks (32 tokens) from their LDS tiles into the running
// states of all of the wave's 16-row tiles, synchronized softmax: the scores
// of both blocks, one running-max update for the 32, and O += P V on
// 16x16x32 instructions, whose 32-long k dimension takes this lane's four
// tokens of the first block (k = 8 (lane / 16) + 0..3) and its four of the
// second (+ 4..7) in P and in V alike.  Half the P x V instructions of two
// single-block steps, each doing twice the work; every K and V operand is
// read from LDS once for all row tiles.  The rescale factors reach the
// accumulator lanes by lane shuffles (no LDS).  LAZY (a row's result written
// directly, no partial): the reference maximum moves only when a score
// exceeds it by more than kLazyRescale (log2 units), so weights stay below
// 2^kLazyRescale and the rescale of the accumulators is rare; out = O / l and
// lse = m + ln l do not depend on which reference m is used.
template <int T, int D, int GMAX, bool LAZY = false>
__device__ __forceinline__ void compute_pair_at(const PartialParams &p, const BlockRows &ba, const BlockRows &bb,
                                                const int (&lim)[row_tiles(GMAX)], float sc,
                                                const uint4 (&qop)[row_tiles(GMAX)][D / 32],
                                                MState<D, GMAX> (&st)[row_tiles(GMAX)], const char *ka,
                                                const char *va, const char *kb, const char *vb) {
    using C = MCfg<D, GMAX, 1>;
    constexpr int DT = op_of(T), NT = row_tiles(GMAX);
    const int lane = threadIdx.x & 63;
    const int mrow = lane & 15, mq = lane >> 4;
    f32x4 acc[NT][2];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) acc[rt][0] = acc[rt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
        const int slot = chunk_slot<T>(4 * ks + mq) ^ (mrow & (C::LPR - 1));
        const uint4 a0 = *reinterpret_cast<const uint4 *>(ka + mrow * C::ROWB + slot * 16);
        const uint4 a1 = *reinterpret_cast<const uint4 *>(kb + mrow * C::ROWB + slot * 16);
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
            acc[rt][0] = mfma16x16x32<DT>(a0, qop[rt][ks], acc[rt][0]);
            acc[rt][1] = mfma16x16x32<DT>(a1, qop[rt][ks], acc[rt][1]);
        }
    }
    auto pack8 = [](const s16x4 &x, const s16x4 &y) {
        const uint2 u = __builtin_bit_cast(uint2, x), w = __builtin_bit_cast(uint2, y);
        return make_uint4(u.x, u.y, w.x, w.y);
    };
    uint4 phi[NT], plo[NT];
    const bool pages_ok = ba.page_ok && bb.page_ok;
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
        // Row 16 rt (lane 0) has the tile's smallest causal limit: when both
        // blocks end below it every score of the pair is visible and no mask
        // is applied (all but the blocks on the causal diagonal).
        float s[2][4];
        if (pages_ok && bb.tb + kBlk <= __builtin_amdgcn_readfirstlane(lim[rt])) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s[0][r] = acc[rt][0][r] * sc;
                s[1][r] = acc[rt][1][r] * sc;
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s[0][r] = ba.page_ok && ba.tb + 4 * mq + r < lim[rt] ? acc[rt][0][r] * sc : -INFINITY;
                s[1][r] = bb.page_ok && bb.tb + 4 * mq + r < lim[rt] ? acc[rt][1][r] * sc : -INFINITY;
            }
        }
        float mt = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) mt = fmaxf(mt, fmaxf(s[0][r], s[1][r]));
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        MState<D, GMAX> &t = st[rt];
        const float mn = (!LAZY || t.m == -INFINITY || mt > t.m + kLazyRescale) ? fmaxf(t.m, mt) : t.m;
        const float corr = rescale(t.m, mn);
        const bool moved = mn != t.m;
        t.m = mn;
        t.l *= corr;
        // a row with no visible score yet (mn = -inf) has only -inf scores,
        // whose weights exp2(-inf - 0) = 0 need a finite reference
        const float mref = mn == -INFINITY ? 0.f : mn;
        float pr[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pr[h][r] = exp2_fast(s[h][r] - mref);
                t.l += pr[h][r];
            }
        }
        if (__any(moved)) {
            // rows 4 mq + 0..3 of this lane's accumulators; lane r (< 16) holds row r's factor
            const float4 cf = make_float4(__shfl(corr, 4 * mq), __shfl(corr, 4 * mq + 1), __shfl(corr, 4 * mq + 2),
                                          __shfl(corr, 4 * mq + 3));
#pragma unroll
            for (int i = 0; i < C::SL; ++i) {
                t.o[i][0] *= cf.x;
                t.o[i][1] *= cf.y;
                t.o[i][2] *= cf.z;
                t.o[i][3] *= cf.w;
            }
        }
        if constexpr (pv_single(T, false)) {
            const f16x4 h0 = {(_Float16)pr[0][0], (_Float16)pr[0][1], (_Float16)pr[0][2], (_Float16)pr[0][3]};
            const f16x4 h1 = {(_Float16)pr[1][0], (_Float16)pr[1][1], (_Float16)pr[1][2], (_Float16)pr[1][3]};
            phi[rt] = pack8(__builtin_bit_cast(s16x4, h0), __builtin_bit_cast(s16x4, h1));
        } else {
            s16x4 h0, l0, h1, l1;
            split_probs<DT>(pr[0], h0, l0);
            split_probs<DT>(pr[1], h1, l1);
            phi[rt] = pack8(h0, h1);
            plo[rt] = pack8(l0, l1);
        }
    }
    constexpr int PT = pv_type(T, false);
    const int vrow = 4 * mq + (mrow >> 2);
    const int vsw = 2 * (vrow & (C::LPR / 2 - 1));
    auto read_v = [&](const char *vtile, int i) {
        const int dim = 16 * i + 4 * (mrow & 3);
        const int slot = chunk_slot<T>(dim >> 3) ^ vsw;
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(vtile + vrow * C::ROWB + slot * 16 + (dim & 7) * 2));
    };
#pragma unroll
    for (int i = 0; i < C::SL; ++i) {
        const uint4 b = pack8(read_v(va, i), read_v(vb, i));
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
            st[rt].o[i] = mfma16x16x32<PT>(phi[rt], b, st[rt].o[i]);
            if constexpr (!pv_single(T, false)) st[rt].o[i] = mfma16x16x32<PT>(plo[rt], b, st[rt].o[i]);
        }
    }
}

// ... from the wave's private tiles.
template <int T, int D, int GMAX, int WAVES, bool UNIFIED>
__device__ __forceinline__ void compute_tiles(const PartialParams &p, const BlockRows &br, int lim, float sc,
                                              const uint4 (&qop)[D / 32], MState<D, GMAX> &st,
                                              MSmem<D, GMAX, WAVES> &sm) {
    const int wave = head_wave<WAVES>();
    compute_tiles_at<T, D, GMAX, UNIFIED>(p, br, lim, sc, qop, st, reinterpret_cast<const char *>(sm.k[wave]),
                                          reinterpret_cast<const char *>(sm.v[wave]), sm.corr[wave]);
}

// One wave's share of the split: blocks wave, wave + WAVES, ...  Paged caches
// read the split's block-table entries once (one per lane) and pick each
// block's page from them with a lane read.  Each block runs through the
// matrix work once per 16-row tile of query rows.
template <int T, int D, int GMAX, int WAVES, bool PAGED, bool UNIFIED>
__device__ void scan_split(const PartialParams &p, int b, int kvh, int t0, int t1, float sc,
                           const int (&lim)[row_tiles(GMAX)], const uint4 (&qop)[row_tiles(GMAX)][D / 32],
                           MState<D, GMAX> (&st)[row_tiles(GMAX)], MSmem<D, GMAX, WAVES> &sm) {
    using L = KLoad<T, D>;
    const int wave = __builtin_amdgcn_readfirstlane(head_wave<WAVES>());
    const auto off = lane_offsets<T, D>(p);
    const int nblk = (t1 - t0 + kBlk - 1) / kBlk;
    const PageCache pc = load_pages<PAGED>(p, b, t0, t1);
    // one register set: once a block sits in the LDS tiles its registers
    // take the next block's loads, which are then in flight during the
    // block's matrix work.  The load after the last block is of an empty
    // block (no rows in range), which reads no memory.
    const int n = wave < nblk ? (nblk - wave + WAVES - 1) / WAVES : 0;   // this wave's blocks
    if (n == 0) return;
    const int tw = t0 + wave * kBlk, tstep = WAVES * kBlk;
    BlockRows br = block_rows<D, PAGED>(p, pc, b, kvh, tw, t1);
    uint4 kr[L::LI], vr[L::LI];
    load_block<T, D>(p, br, t1, off, kr, vr);
    for (int j = 0; j < n; ++j) {
        write_tiles<T, D, GMAX, WAVES, UNIFIED>(kr, vr, sm);
        wave_lds_sync();
        const BlockRows bn = block_rows<D, PAGED>(p, pc, b, kvh, tw + (j + 1) * tstep, t1);
        load_block<T, D>(p, bn, t1, off, kr, vr);
#pragma unroll
        for (int rt = 0; rt < row_tiles(GMAX); ++rt)
            compute_tiles<T, D, GMAX, WAVES, UNIFIED>(p, br, lim[rt], sc, qop[rt], st[rt], sm);
        wave_lds_sync();   // this block's tile reads before the next block's writes
        br = bn;
    }
}

// Wave states of row tile rt (query rows 16 rt ..) -> the split's partial
// for the rows in write_mask (DIRECT: a row's only split, written as the
// result to out and lse).
template <int T, int D, int GMAX, int WAVES, bool DIRECT>
__device__ void finish_split(const PartialParams &p, MState<D, GMAX> &st, MSmem<D, GMAX, WAVES> &sm, int b, int kvh,
                             int s, uint32_t write_mask, int rt, float vmul) {
    using C = MCfg<D, GMAX, WAVES>;
    constexpr int GQ = MSmem<D, GMAX, WAVES>::GQ < 4 ? MSmem<D, GMAX, WAVES>::GQ : 4;   // head quads per tile
    const int lane = threadIdx.x & 63, wave = head_wave<WAVES>();
    const int mrow = lane & 15, mq = lane >> 4;
    // wave 0 writes the partial straight from its registers: lane
    // (mrow, mq) holds dim 16 * slice + mrow of rows 4 * mq + r, and reads
    // l and m of those rows from the lanes that hold them.  A second wave
    // first hands its state over through LDS, lane for lane, and is merged
    // in by the max-rescale rule.
    float lsum = st.l + __shfl_xor(st.l, 16);
    lsum += __shfl_xor(lsum, 32);
    if constexpr (WAVES == 2) {
        __syncthreads();   // the hand-over area overlays the K tiles of both waves
        if (wave == 1) {
            if (mq < GQ) {
#pragma unroll
                for (int i = 0; i < C::SL; ++i)
                    sm.ho.o[i][lane] = make_float4(st.o[i][0], st.o[i][1], st.o[i][2], st.o[i][3]);
            }
            if (mq == 0) {
                sm.ho.l[mrow] = lsum;
                sm.ho.m[mrow] = st.m;
            }
        }
        __syncthreads();
        if (wave == 1) return;
    }
    if (mq >= GQ) return;
    float4 x[C::SL];
    if constexpr (WAVES == 2) {
#pragma unroll
        for (int i = 0; i < C::SL; ++i) x[i] = sm.ho.o[i][lane];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int gl = 4 * mq + r, g = 16 * rt + gl;     // row within the tile, query row
        float L = __shfl(lsum, gl, 16), M = __shfl(st.m, gl, 16);
        float f0 = 1.f, f1 = 0.f;
        if constexpr (WAVES == 2) {
            const float L1 = sm.ho.l[gl], M1 = sm.ho.m[gl];
            const float Mx = fmaxf(M, M1);
            f0 = rescale(M, Mx);
            f1 = rescale(M1, Mx);
            L = fmaf(L1, f1, L * f0);
            M = Mx;
        }
        if (g >= p.R || !((write_mask >> g) & 1u)) continue;
        float inv = L > 0.f ? 1.f / L : 0.f;
        if constexpr (f8_of(T)) inv *= vmul;   // a stored V unit stands for the head's V scale
        float a[C::SL];
#pragma unroll
        for (int i = 0; i < C::SL; ++i) {
            a[i] = st.o[i][r];
            if constexpr (WAVES == 2) {
                const float xr = r == 0 ? x[i].x : r == 1 ? x[i].y : r == 2 ? x[i].z : x[i].w;
                a[i] = fmaf(xr, f1, a[i] * f0);
            }
        }
        const float m_nat = (L > 0.f && M != -INFINITY) ? M * kLn2 : -INFINITY;
        if constexpr (DIRECT) {   // the row's only split: its partial is the result
            const size_t row = query_row(p, b, kvh, g);
#pragma unroll
            for (int i = 0; i < C::SL; ++i) store_out(p.out, row * D + 16 * i + mrow, a[i] * inv, p.out_dtype);
            if (mrow == 0 && p.lse) p.lse[row] = L > 0.f ? m_nat + logf(L) : -INFINITY;
        } else {
            // device-scope stores, written through the XCD's L2: a step (partials
            // and their merge) measured ~1% faster than with plain stores, whose
            // dirty lines the L2 writes back when the kernel ends
            const size_t slot = row_slot(p, b, kvh, g, s);
#pragma unroll
            for (int i = 0; i < C::SL; ++i) store_dev(&p.part_o[slot * D + 16 * i + mrow], a[i] * inv);
            if (mrow == 0) {
                store_dev(&p.part_m[slot], m_nat);
                store_dev(&p.part_l[slot], L);
            }
        }
    }
}

// KV head of grid row y.  Consecutive workgroups go to the eight XCDs in
// turn, and an XCD hands its share to its CUs round by round, so in grid order
// a grid that is resident at once with two workgroups per CU (32 KV heads, 16
// splits: 512 workgroups) gives each CU the workgroups of heads h and
// h + Hkv / 2, of equal parity; the odd heads, whose rows start at an odd
// multiple of 256 bytes of each token row, ran ~10% slower in traces.  Such
// grids take the odd heads first, which pairs one odd and one even head on
// each CU.  Measured on MI355X at the Llama-2 shape: 13.7-14.1 -> 13.2-13.6
// us on two devices, within 1% on a third (as were resident GQA grids of 256
// and 512 workgroups there); grids with four workgroups per CU are unchanged
// (32k GQA, 1024 workgroups) and a grid several waves deep is slower (B=4,
// N=128k: 351 against 358 us), so those keep grid order.
__device__ __forceinline__ int kv_head_of(const PartialParams &p, int y) {
    const int64_t wgs = (int64_t)gridDim.x * gridDim.y * gridDim.z;
    if ((p.Hkv & 1) || wgs >= 4 * p.num_cus) return y;
    const int half = p.Hkv >> 1;
    return y < half ? 2 * y + 1 : 2 * (y - half);
}

// The B operand of each 16-row tile (q of query row 16 rt + lane % 16, dims
// 8 * (lane / 16) of each 32-dim step; rows >= R zero) and each lane's causal
// limit within the split ending at t1.
template <int D, int GMAX>
__device__ __forceinline__ void load_q_operand(const PartialParams &p, int b, int kvh, int len, int t1,
                                               uint4 (&qop)[row_tiles(GMAX)][D / 32], int (&lim)[row_tiles(GMAX)]) {
    const int lane = threadIdx.x & 63, R = p.R;
#pragma unroll
    for (int rt = 0; rt < row_tiles(GMAX); ++rt) {
        const int rho = 16 * rt + (lane & 15);
        lim[rt] = row_limit(p, len, t1, rho);
        const char *qb = static_cast<const char *>(p.q);
        const size_t qrow = rho < R ? query_row(p, b, kvh, rho) : 0;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            qop[rt][ks] = make_uint4(0, 0, 0, 0);
            if (rho < R) qop[rt][ks] = load16(qb + (qrow * D + 32 * ks + 8 * (lane >> 4)) * 2);
        }
    }
}

// Query rows of the wave whose scores left [lo, hi] (bit 16 rt + row).
template <int GMAX, int D>
__device__ __forceinline__ uint32_t flagged_rows(const MState<D, GMAX> (&st)[row_tiles(GMAX)]) {
    uint32_t mine = 0;
#pragma unroll
    for (int rt = 0; rt < row_tiles(GMAX); ++rt) {
        const uint64_t bal = __ballot(st[rt].bad);
        mine |= (uint32_t)((bal | (bal >> 16) | (bal >> 32) | (bal >> 48)) & 0xffffu) << (16 * rt);
    }
    return mine;
}

// Score scale (log2 units) and V multiplier of KV head kvh: 8-bit caches fold
// the head's K scale into the score scale and apply its V scale to O.
template <int T>
__device__ __forceinline__ void head_scales(const PartialParams &p, int kvh, float &sc, float &vmul) {
    sc = p.scale_log2;
    vmul = p.v_mult;
    if constexpr (f8_of(T)) {
        if (p.k_scales) sc *= p.k_scales[kvh];
        if (p.v_scales) vmul = p.v_scales[kvh];
    }
}

template <int T, int D, int GMAX, int WAVES, bool PAGED, bool UNI, bool DIRECT>
__global__ void __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(min_waves_per_eu(GMAX))))
partial_mfma_kernel(const PartialParams pk) {
    using C = MCfg<D, GMAX, WAVES>;
    static_assert(WAVES == 1 || WAVES == 2, "the epilogue merges at most two waves");
    static_assert(sizeof(MSmem<D, GMAX, WAVES>) <= 65536, "LDS budget of one workgroup");
    __shared__ MSmem<D, GMAX, WAVES> sm;
    int b;
    const PartialParams p = tile_params(pk, b);
    const int kvh = kv_head_of(p, blockIdx.y);
    const int s = split_index(blockIdx.x, blockIdx.z, kvh, p.Hkv, p.max_splits);
    const int R = p.R;                               // query rows of this workgroup
    const int len = request_len(p.seq_lens, b, p.kv_capacity, p.max_splits * p.split);
    const int t0 = s * p.split;
    const int t1 = min(t0 + p.split, tile_len(p, len));

    if (t0 >= t1) {
        if (threadIdx.x < R && !p.recompute_rows) {
            const size_t slot = row_slot(p, b, kvh, threadIdx.x, s);
            if (!DIRECT) {
                p.part_m[slot] = -INFINITY;
                p.part_l[slot] = 0.f;
            }
            if (p.flags) p.flags[slot] = 0;
        }
        if (DIRECT && !p.recompute_rows) write_empty_rows<D>(p, b, kvh, 64 * WAVES);   // rows that see nothing
        return;
    }
    // whole-row fallback, second pass: only rows flagged in some split of the request
    uint32_t rows_to_write = R >= 32 ? 0xffffffffu : (1u << R) - 1u;
    if (!UNI && p.recompute_rows) {
        rows_to_write = rows_flagged_in_request(p, b, kvh, (len + p.split - 1) / p.split);
        if (!rows_to_write) return;
    }

    constexpr int NT = row_tiles(GMAX);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float sc, vmul;
    head_scales<T>(p, kvh, sc, vmul);
    // B operand of tile rt: q of query row 16 rt + lane % 16, dims 8 * (lane / 16)
    // of each step; lim[rt]: that row's causal limit
    uint4 qop[NT][C::KS];
    int lim[NT];
    load_q_operand<D, GMAX>(p, b, kvh, len, t1, qop, lim);

    const uint32_t all = R >= 32 ? 0xffffffffu : (1u << R) - 1u;
    MState<D, GMAX> st[NT];
    uint32_t badmask = 0;
    if constexpr (UNI) {
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) st[rt].init(p.phi2);
        scan_split<T, D, GMAX, WAVES, PAGED, true>(p, b, kvh, t0, t1, sc, lim, qop, st, sm);
        const uint32_t mine = flagged_rows<GMAX>(st);
        if constexpr (WAVES == 1) {
            badmask = mine;                          // wave-uniform: the one wave
        } else {
            if (lane == 0) sm.bad[wave] = mine;
            __syncthreads();
#pragma unroll
            for (int w = 0; w < WAVES; ++w) badmask |= sm.bad[w];
        }
        badmask &= all;
        // whole-row fallback: every row's unified partial now, the flagged rows'
        // splits all rewritten by a second pass
        const uint32_t keep = p.row_fallback ? all : all & ~badmask;
#pragma unroll
        for (int rt = 0; rt < NT; ++rt)
            finish_split<T, D, GMAX, WAVES, DIRECT>(p, st[rt], sm, b, kvh, s, keep, rt, vmul);
        if (badmask && !p.row_fallback) {   // synchronized recompute of the flagged heads
            if constexpr (WAVES > 1) __syncthreads();   // the hand-over area overlays the K tiles
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) st[rt].init(-INFINITY);
            scan_split<T, D, GMAX, WAVES, PAGED, false>(p, b, kvh, t0, t1, sc, lim, qop, st, sm);
#pragma unroll
            for (int rt = 0; rt < NT; ++rt)
                finish_split<T, D, GMAX, WAVES, DIRECT>(p, st[rt], sm, b, kvh, s, badmask, rt, vmul);
        }
        if (threadIdx.x == 0 && badmask && p.fallback_count)
            atomicAdd(p.fallback_count, __builtin_popcount(badmask));
    } else {
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) st[rt].init(-INFINITY);
        scan_split<T, D, GMAX, WAVES, PAGED, false>(p, b, kvh, t0, t1, sc, lim, qop, st, sm);
#pragma unroll
        for (int rt = 0; rt < NT; ++rt)
            finish_split<T, D, GMAX, WAVES, DIRECT>(p, st[rt], sm, b, kvh, s, rows_to_write, rt, vmul);
    }
    if (p.flags && threadIdx.x < R && !p.recompute_rows)
        p.flags[row_slot(p, b, kvh, threadIdx.x, s)] = (badmask >> threadIdx.x) & 1u;
}

// ---------------------------------------------------------------------------
// query tiles sharing K and V (a prompt's worth of query rows per KV head)
// ---------------------------------------------------------------------------
// Four waves, one query tile each (up to 32 rows, two 16-row matrix tiles),
// scan the same tokens of a split: of every 64 tokens each wave loads one
// 16-token block, the four blocks pass through LDS once, and every wave runs
// its rows against all four.  Per query row, K and V come through the cache
// hierarchy a quarter as often as with one workgroup per tile (the handbook
// page's forward kernel likewise stages K and V tiles in shared memory for a
// block of query rows, section "A working FlashAttention forward kernel").
// Synchronized softmax; each wave writes its rows' partials (or, DIRECT, the
// result) like a one-wave workgroup.
constexpr int kShareWaves = 4;

template <int D>
struct PSmem {
    // two buffers of 64 tokens: the waves compute on one while the next is
    // written to the other, one barrier per 64 tokens; block j of a buffer is
    // loaded by wave j
    uint4 k[2][kShareWaves][kBlk * D * 2 / 16];
    uint4 v[2][kShareWaves][kBlk * D * 2 / 16];
};

// Register budget: two waves per SIMD (two workgroups per CU).
template <int T, int D, bool PAGED, bool DIRECT>
__global__ void __launch_bounds__(64 * kShareWaves) __attribute__((amdgpu_waves_per_eu(2)))
shared_kv_mfma_kernel(const PartialParams pk) {
    constexpr int GMAX = 32, NT = row_tiles(GMAX), W = kShareWaves;
    using C = MCfg<D, GMAX, 1>;
    using L = KLoad<T, D>;
    static_assert(sizeof(PSmem<D>) <= 65536, "LDS budget of one workgroup");
    __shared__ PSmem<D> sm;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    // grid z = b * groups + j: request b, tile group groups - 1 - j (the
    // groups of later query tokens see more of the cache and start first)
    const int groups = (pk.q_tiles + W - 1) / W;
    const int b = (int)blockIdx.z / groups;
    const int grp = groups - 1 - ((int)blockIdx.z - b * groups);
    const int kvh = blockIdx.y;
    const int s = split_index(blockIdx.x, blockIdx.z, kvh, pk.Hkv, pk.max_splits);
    const int tile = grp * W + w, last = min(grp * W + W - 1, pk.q_tiles - 1);
    PartialParams p = pk;                        // this wave's tile
    p.i0 = tile * pk.tile_tokens;
    p.R = tile < pk.q_tiles ? min(pk.tile_tokens, pk.q_len - p.i0) * pk.G : 0;
    PartialParams pl = pk;                       // the group's last tile: its tokens bound the scan
    pl.i0 = last * pk.tile_tokens;
    pl.R = min(pk.tile_tokens, pk.q_len - pl.i0) * pk.G;
    const int R = p.R;
    const int len = request_len(pk.seq_lens, b, pk.kv_capacity, pk.max_splits * pk.split);
    const int t0 = s * pk.split;
    const int t1 = min(t0 + pk.split, tile_len(pl, len));

    if (t0 >= t1) {   // no row of the group sees a token of this split
        if (DIRECT) {
            for (int idx = lane; idx < R * D; idx += 64)
                store_out(p.out, query_row(p, b, kvh, idx / D) * D + idx % D, 0.f, p.out_dtype);
            if (lane < R && p.lse) p.lse[query_row(p, b, kvh, lane)] = -INFINITY;
        } else if (lane < R) {
            const size_t slot = row_slot(p, b, kvh, lane, s);
            p.part_m[slot] = -INFINITY;
            p.part_l[slot] = 0.f;
        }
        if (p.flags && lane < R) p.flags[row_slot(p, b, kvh, lane, s)] = 0;
        return;
    }

    float sc, vmul;
    head_scales<T>(p, kvh, sc, vmul);
    uint4 qop[NT][C::KS];
    int lim[NT];
    load_q_operand<D, GMAX>(p, b, kvh, len, t1, qop, lim);
    MState<D, GMAX> st[NT];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) st[rt].init(-INFINITY);
    const int wlen = R > 0 ? min(tile_len(p, len), t1) : t0;   // this wave's rows see tokens < wlen

    const auto off = lane_offsets<T, D>(p);
    const PageCache pc = load_pages<PAGED>(p, b, t0, t1);
    const int nsup = (t1 - t0 + W * kBlk - 1) / (W * kBlk);
    // one register set, as in the one-wave kernel: the next 64 tokens' loads
    // are in flight during the matrix work on these
    const int tstep = W * kBlk;
    uint4 kr[L::LI], vr[L::LI];
    load_block<T, D>(p, block_rows<D, PAGED>(p, pc, b, kvh, t0 + w * kBlk, t1), t1, off, kr, vr);
    write_tiles_at<T, D, false>(kr, vr, reinterpret_cast<char *>(sm.k[0][w]), reinterpret_cast<char *>(sm.v[0][w]));
    __syncthreads();
    load_block<T, D>(p, block_rows<D, PAGED>(p, pc, b, kvh, t0 + tstep + w * kBlk, t1), t1, off, kr, vr);
    for (int k = 0; k < nsup; ++k) {
        const int tsup = t0 + k * tstep, cur = k & 1;
#pragma unroll
        for (int j = 0; j < W; j += 2) {          // blocks in pairs: 32 tokens per matrix step
            const int tb = tsup + j * kBlk;
            if (tb >= wlen) continue;             // past this wave's rows
            const BlockRows ba = block_rows<D, PAGED>(p, pc, b, kvh, tb, t1);
            const BlockRows bb = block_rows<D, PAGED>(p, pc, b, kvh, tb + kBlk, t1);
            compute_pair_at<T, D, GMAX, DIRECT>(p, ba, bb, lim, sc, qop, st, reinterpret_cast<const char *>(sm.k[cur][j]),
                                        reinterpret_cast<const char *>(sm.v[cur][j]),
                                        reinterpret_cast<const char *>(sm.k[cur][j + 1]),
                                        reinterpret_cast<const char *>(sm.v[cur][j + 1]));
        }
        // the next 64 tokens into the other buffer, whose last readers passed
        // the previous barrier; then one barrier for both orders
        write_tiles_at<T, D, false>(kr, vr, reinterpret_cast<char *>(sm.k[cur ^ 1][w]),
                                    reinterpret_cast<char *>(sm.v[cur ^ 1][w]));
        __syncthreads();
        load_block<T, D>(p, block_rows<D, PAGED>(p, pc, b, kvh, tsup + 2 * tstep + w * kBlk, t1), t1, off, kr, vr);
    }
    if (R > 0) {
        const uint32_t all = R >= 32 ? 0xffffffffu : (1u << R) - 1u;
        auto &one = *reinterpret_cast<MSmem<D, GMAX, 1> *>(&sm);   // unused by a one-wave epilogue
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) finish_split<T, D, GMAX, 1, DIRECT>(p, st[rt], one, b, kvh, s, all, rt, vmul);
        if (p.flags && lane < R) p.flags[row_slot(p, b, kvh, lane, s)] = 0;
    }
}

template <int T, int D, bool PAGED>
hipError_t launch_shared_kv(const PartialParams &p, hipStream_t stream) {
    const int groups = (p.q_tiles + kShareWaves - 1) / kShareWaves;
    dim3 grid(p.max_splits, p.Hkv, p.B * groups);
    if (p.direct)
        hipLaunchKernelGGL((shared_kv_mfma_kernel<T, D, PAGED, true>), grid, dim3(64 * kShareWaves), 0, stream, p);
    else
        hipLaunchKernelGGL((shared_kv_mfma_kernel<T, D, PAGED, false>), grid, dim3(64 * kShareWaves), 0, stream, p);
    return hipGetLastError();
}

// Whether a launch takes the shared-K/V kernel: four or more query tiles per
// KV head (a prompt's worth of rows; fewer leave waves idle), synchronized
// softmax, partials or the direct result (the single-launch merge and the
// unified-max passes keep one tile per workgroup).
inline bool use_shared_kv(const PartialParams &p) {
    return p.q_tiles >= kShareWaves && !p.unified && !p.tickets && !p.recompute_rows && !p.row_fallback;
}

// ---------------------------------------------------------------------------
// single launch: partials and their merge in one kernel
// ---------------------------------------------------------------------------
// A workgroup covers SW consecutive splits of one (request, KV head), one
// wave per split, each wave scanning its split exactly as above.  The waves'
// split states are merged in the workgroup (max-rescale, in split order) into
// one partial of the SW splits, written with device-scope stores to slot x of
// the head's partial rows; the last workgroup of the head to finish merges
// the head's workgroup partials into out and lse (fd_merge.h).  The merge is
// the same log-sum-exp merge as the separate combine, taken as a two-level
// tree (splits within a workgroup, then workgroups), which the merge's
// associativity makes exact (Flash-Decoding page, "The Rescaling and Online
// Softmax Reduction Algorithm").  Under unified max a wave whose split holds
// an out-of-range score rescans the split with the synchronized softmax and
// carries that state for every row of the split.
template <int D, int GMAX, int SW>
struct FSmem {
    static constexpr int NT = row_tiles(GMAX);
    struct Hand {                                       // one wave's state, lane for lane
        float4 o[D / 16][64];
        float l[16], m[16];
    };
    union {
        MSmem<D, GMAX, 1> tiles[SW];                    // each wave's K / V tiles
        Hand ho[SW > 1 ? SW - 1 : 1][NT];               // waves 1 .. SW-1 hand over to wave 0
        float merge[merge_lds_floats(kFusedMaxRowParts, kMaxRows, 64 * SW)];   // the last workgroup's merge
    };
    int ticket;
};

// Wave 0: merge the handed-over states of waves 1 .. SW-1 into its own (row
// tile rt) and write the workgroup's partial to slot x, device scope.
template <int T, int D, int GMAX, int SW>
__device__ void store_group_partial(const PartialParams &p, const MState<D, GMAX> &st, float lsum,
                                    const FSmem<D, GMAX, SW> &sm, int rt, int b, int kvh, int x, float vmul) {
    constexpr int SL = D / 16;
    const int lane = threadIdx.x & 63, mrow = lane & 15, mq = lane >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int gl = 4 * mq + r, g = 16 * rt + gl;    // row within the tile, query row
        float L = __shfl(lsum, gl, 16), M = __shfl(st.m, gl, 16);
        float a[SL];
#pragma unroll
        for (int i = 0; i < SL; ++i) a[i] = st.o[i][r];
#pragma unroll
        for (int v = 0; v < SW - 1; ++v) {
            const float L1 = sm.ho[v][rt].l[gl], M1 = sm.ho[v][rt].m[gl];
            const float Mx = fmaxf(M, M1);
            const float f0 = rescale(M, Mx), f1 = rescale(M1, Mx);
            L = fmaf(L1, f1, L * f0);
#pragma unroll
            for (int i = 0; i < SL; ++i) {
                const float4 o1 = sm.ho[v][rt].o[i][lane];
                const float xr = r == 0 ? o1.x : r == 1 ? o1.y : r == 2 ? o1.z : o1.w;
                a[i] = fmaf(xr, f1, a[i] * f0);
            }
            M = Mx;
        }
        if (g >= p.R) continue;
        const size_t slot = row_slot(p, b, kvh, g, x);
        float inv = L > 0.f ? 1.f / L : 0.f;
        if constexpr (f8_of(T)) inv *= vmul;
#pragma unroll
        for (int i = 0; i < SL; ++i) store_dev(&p.part_o[slot * D + 16 * i + mrow], a[i] * inv);
        if (mrow == 0) {
            store_dev(&p.part_m[slot], (L > 0.f && M != -INFINITY) ? M * kLn2 : -INFINITY);
            store_dev(&p.part_l[slot], L);
        }
    }
}

// Register budget: two waves per SIMD (the merge's loads in flight next to
// the scan state need more than 128 registers; a grid of one workgroup of
// four waves per CU, the 32k GQA shape's, holds only one wave per SIMD).
template <int T, int D, int GMAX, int SW, bool PAGED, bool UNI>
__global__ void __launch_bounds__(64 * SW) __attribute__((amdgpu_waves_per_eu(2)))
fused_mfma_kernel(const PartialParams pk) {
    using C = MCfg<D, GMAX, 1>;
    constexpr int NT = row_tiles(GMAX);
    static_assert(sizeof(FSmem<D, GMAX, SW>) <= 65536, "LDS budget of one workgroup");
    __shared__ FSmem<D, GMAX, SW> sm;
    int b;
    const PartialParams p = tile_params(pk, b);
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // this wave's split in the group
    const int kvh = blockIdx.y;
    const int x = split_index(blockIdx.x, blockIdx.z, kvh, p.Hkv, gridDim.x);   // the group's index in the head
    const int s = x * SW + w;                                                // this wave's split
    const int R = p.R, lane = threadIdx.x & 63;
    const int len = request_len(p.seq_lens, b, p.kv_capacity, p.max_splits * p.split);
    const int tl = tile_len(p, len);                                         // tokens the tile's rows see
    const int nb = (tl + SW * p.split - 1) / (SW * p.split);                // groups holding tokens

    if (x >= nb) {   // none of the group's splits holds a token
        if (p.flags && lane < R && s < p.max_splits) p.flags[row_slot(p, b, kvh, lane, s)] = 0;
        if (nb == 0 && x == 0) write_empty_rows<D>(p, b, kvh, 64 * SW);
        return;
    }

    const int t0 = s * p.split, t1 = min(t0 + p.split, tl);   // t0 >= t1: a split past the tile's tokens
    float sc, vmul;
    head_scales<T>(p, kvh, sc, vmul);
    uint4 qop[NT][C::KS];
    int lim[NT];
    load_q_operand<D, GMAX>(p, b, kvh, len, t1, qop, lim);
    const uint32_t all = R >= 32 ? 0xffffffffu : (1u << R) - 1u;
    MState<D, GMAX> st[NT];
    uint32_t badmask = 0;
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) st[rt].init(-INFINITY);
    if (t0 < t1) {
        if constexpr (UNI) {
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) st[rt].init(p.phi2);
            scan_split<T, D, GMAX, 1, PAGED, true>(p, b, kvh, t0, t1, sc, lim, qop, st, sm.tiles[w]);
            badmask = flagged_rows<GMAX>(st) & all;
            if (badmask) {   // synchronized recompute of the split
#pragma unroll
                for (int rt = 0; rt < NT; ++rt) st[rt].init(-INFINITY);
                scan_split<T, D, GMAX, 1, PAGED, false>(p, b, kvh, t0, t1, sc, lim, qop, st, sm.tiles[w]);
                if (lane == 0 && p.fallback_count) atomicAdd(p.fallback_count, __builtin_popcount(badmask));
            }
        } else {
            scan_split<T, D, GMAX, 1, PAGED, false>(p, b, kvh, t0, t1, sc, lim, qop, st, sm.tiles[w]);
        }
    }
    if (p.flags && lane < R && s < p.max_splits) p.flags[row_slot(p, b, kvh, lane, s)] = (badmask >> lane) & 1u;

    float lsum[NT];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
        lsum[rt] = st[rt].l + __shfl_xor(st[rt].l, 16);
        lsum[rt] += __shfl_xor(lsum[rt], 32);
    }
    if constexpr (SW > 1) {
        __syncthreads();                                  // the hand-over area overlays the tiles
        if (w > 0) {
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) {
#pragma unroll
                for (int i = 0; i < D / 16; ++i)
                    sm.ho[w - 1][rt].o[i][lane] = make_float4(st[rt].o[i][0], st[rt].o[i][1], st[rt].o[i][2],
                                                              st[rt].o[i][3]);
                if (lane < 16) {
                    sm.ho[w - 1][rt].l[lane] = lsum[rt];
                    sm.ho[w - 1][rt].m[lane] = st[rt].m;
                }
            }
        }
        __syncthreads();
    }
    if (w == 0) {
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) store_group_partial<T, D, GMAX, SW>(p, st[rt], lsum[rt], sm, rt, b, kvh, x, vmul);
    }
    if (arrive_last(&p.tickets[(size_t)blockIdx.z * p.Hkv + kvh], nb, &sm.ticket))
        merge_rows<D, 64 * SW>(p, b, kvh, nb, sm.merge);
}

template <int T, int D, int GMAX, int SW, bool PAGED>
hipError_t launch_fused_shaped(const PartialParams &p, hipStream_t stream) {
    dim3 grid((p.max_splits + SW - 1) / SW, p.Hkv, p.B * p.q_tiles);
    if (p.unified)
        hipLaunchKernelGGL((fused_mfma_kernel<T, D, GMAX, SW, PAGED, true>), grid, dim3(64 * SW), 0, stream, p);
    else
        hipLaunchKernelGGL((fused_mfma_kernel<T, D, GMAX, SW, PAGED, false>), grid, dim3(64 * SW), 0, stream, p);
    return hipGetLastError();
}

// Splits per workgroup of the single-launch kernel (the host picks 2 or 4).
template <int T, int D, int GMAX, bool PAGED>
hipError_t launch_fused(const PartialParams &p, hipStream_t stream) {
    return p.splits_per_wg == 2 ? launch_fused_shaped<T, D, GMAX, 2, PAGED>(p, stream)
                                : launch_fused_shaped<T, D, GMAX, 4, PAGED>(p, stream);
}

// Waves per workgroup, chosen from measurements on MI355X.  A grid of fewer
// than four workgroups per CU takes two, whose loads it needs in flight
// (Llama-2 shape, 512 workgroups: 14.6 us against 17.6 with one).  From four
// per CU a 16-bit cache takes one, which saves the hand-over between waves
// (32k GQA, 1024 workgroups: 23.3 us against 25.2; verifying 4 tokens, 16
// rows: 25.4-25.7 against 26.3; B=64 paged: 499 against 503; B=4, N=128k:
// 352 against 349, the one shape measured the other way, by 1%).  An 8-bit
// cache keeps two waves for up to four query rows, where the second wave
// covers the widening (32k GQA E4M3: 14.7 us against 19.0 with one), and
// takes one with more rows.
template <int T>
inline int launch_waves(const PartialParams &p) {
    const int64_t wgs = (int64_t)p.max_splits * p.Hkv * p.B * p.q_tiles;
    if (wgs < 4 * (int64_t)p.num_cus) return 2;
    return (!f8_of(T) || p.R > 4) ? 1 : 2;
}

template <int T, int D, int GMAX, int WAVES, bool PAGED, bool DIRECT = false>
hipError_t launch_shaped(const PartialParams &p, hipStream_t stream) {
    dim3 grid(p.max_splits, p.Hkv, p.B * p.q_tiles);
    if constexpr (DIRECT) {   // the synchronized softmax only (the host sends unified max to the merge path)
        if (p.unified) return hipErrorInvalidValue;
        hipLaunchKernelGGL((partial_mfma_kernel<T, D, GMAX, WAVES, PAGED, false, true>), grid, dim3(64 * WAVES), 0,
                           stream, p);
    } else if (p.unified) {
        hipLaunchKernelGGL((partial_mfma_kernel<T, D, GMAX, WAVES, PAGED, true, false>), grid, dim3(64 * WAVES), 0,
                           stream, p);
    } else {
        hipLaunchKernelGGL((partial_mfma_kernel<T, D, GMAX, WAVES, PAGED, false, false>), grid, dim3(64 * WAVES), 0,
                           stream, p);
    }
    return hipGetLastError();
}

template <int T, int D, int GMAX, bool PAGED>
hipError_t launch(const PartialParams &p, hipStream_t stream) {
    if (p.tickets) return launch_fused<T, D, GMAX, PAGED>(p, stream);
    // one split per row, written as the result: one-wave workgroups (a
    // separate instantiation keeps the other kernels free of its epilogue)
    if (p.direct) return launch_shaped<T, D, GMAX, 1, PAGED, true>(p, stream);
    if constexpr (GMAX > 4 || !f8_of(T)) {
        if (launch_waves<T>(p) == 1) return launch_shaped<T, D, GMAX, 1, PAGED>(p, stream);
    }
    return launch_shaped<T, D, GMAX, 2, PAGED>(p, stream);
}

template <int T, int D, int GMAX>
hipError_t by_paged(const PartialParams &p, hipStream_t s) {
    return p.page_size ? launch<T, D, GMAX, true>(p, s) : launch<T, D, GMAX, false>(p, s);
}

template <int T, int D>
hipError_t by_group(const PartialParams &p, hipStream_t s) {
    if (use_shared_kv(p))   // tiles of more than 16 rows (the host balances them): GMAX 32
        return p.page_size ? launch_shared_kv<T, D, true>(p, s) : launch_shared_kv<T, D, false>(p, s);
    if (p.R <= 1) return by_paged<T, D, 1>(p, s);
    if (p.R <= 2) return by_paged<T, D, 2>(p, s);
    if (p.R <= 4) return by_paged<T, D, 4>(p, s);
    if (p.R <= 8) return by_paged<T, D, 8>(p, s);
    if (p.R <= 16) return by_paged<T, D, 16>(p, s);
    return by_paged<T, D, 32>(p, s);
}

template <int T>
hipError_t by_dim(const PartialParams &p, hipStream_t s) {
    return p.d == 64 ? by_group<T, 64>(p, s) : by_group<T, 128>(p, s);
}

}  // namespace
}  // namespace fd
