// fd_device.h -- gfx950 device helpers: 16-byte KV loads, storage-type
// unpacking, wave64 cross-lane reductions, output rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_internal.h"

namespace fd {

// ---------------------------------------------------------------------------
// storage types: a 16-byte load holds E elements
// ---------------------------------------------------------------------------
template <int DT> struct Storage;
template <> struct Storage<F32> { static constexpr int E = 4; static constexpr int bytes = 4; };
template <> struct Storage<F16> { static constexpr int E = 8; static constexpr int bytes = 2; };
template <> struct Storage<BF16> { static constexpr int E = 8; static constexpr int bytes = 2; };
// 8-bit caches are read 8 bytes per lane so that a lane holds as many elements
// as with a 16-bit cache
template <> struct Storage<FP8> { static constexpr int E = 8; static constexpr int bytes = 1; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16_bits_to_float(uint32_t h16) {
    _Float16 h;
    uint16_t bits = (uint16_t)h16;
    __builtin_memcpy(&h, &bits, 2);
    return (float)h;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Widen the E elements in `raw` (16 bytes; 8 for FP8) to fp32.  The E4M3
// conversion of gfx950 (v_cvt_pk_f32_fp8) is exact for all 256 codes,
// NaN included.
template <int DT>
__device__ __forceinline__ void unpack(const uint4 &raw, float *out) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    if constexpr (DT == FP8) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
            const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
            out[4 * i] = a.x;
            out[4 * i + 1] = a.y;
            out[4 * i + 2] = b.x;
            out[4 * i + 3] = b.y;
        }
    } else if constexpr (DT == F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(w[i]);
    } else if constexpr (DT == BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = bf16_lo(w[i]);
            out[2 * i + 1] = bf16_hi(w[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = f16_bits_to_float(w[i] & 0xffffu);
            out[2 * i + 1] = f16_bits_to_float(w[i] >> 16);
        }
    }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte global load of streamed (read-once) data, with the non-temporal hint.
__device__ __forceinline__ uint4 load16_stream(const void *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 load16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// One lane's piece of a cache row: E elements (16 bytes; 8 for FP8), streamed.
template <int DT>
__device__ __forceinline__ uint4 load_piece(const void *p) {
    if constexpr (Storage<DT>::E * Storage<DT>::bytes == 16) {
        return load16_stream(p);
    } else {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
        return make_uint4(v.x, v.y, 0u, 0u);
    }
}

// ---------------------------------------------------------------------------
// cross-lane reductions inside aligned lane groups of W (W | 64)
// ---------------------------------------------------------------------------
// DPP row-local permutations (16-lane rows): quad_perm xor1 / xor2,
// row_half_mirror (i <-> 7 - i), row_mirror (i <-> 15 - i).  After xor1 and
// xor2 every lane of a quad holds the quad's value, so the mirrors complete an
// 8- and a 16-lane butterfly.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

template <int W>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "W");
    if constexpr (W >= 2) v += dpp<kDppXor1>(v);
    if constexpr (W >= 4) v += dpp<kDppXor2>(v);
    if constexpr (W >= 8) v += dpp<kDppHalfMirror>(v);
    if constexpr (W >= 16) v += dpp<kDppMirror>(v);
    if constexpr (W >= 32) v += __shfl_xor(v, 16);
    if constexpr (W >= 64) v += __shfl_xor(v, 32);
    return v;
}

template <int W>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (W >= 2) v = fmaxf(v, dpp<kDppXor1>(v));
    if constexpr (W >= 4) v = fmaxf(v, dpp<kDppXor2>(v));
    if constexpr (W >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
    if constexpr (W >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
    if constexpr (W >= 32) v = fmaxf(v, __shfl_xor(v, 16));
    if constexpr (W >= 64) v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2(a - b) with the convention that an absent state (a = -inf) weighs 0,
// also when b is -inf.
__device__ __forceinline__ float rescale(float a, float b) {
    return a == -INFINITY ? 0.0f : exp2_fast(a - b);
}

// ---------------------------------------------------------------------------
// output rounding (round to nearest even)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;   // NaN stays a quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t float_to_f16_bits(float f) {
    _Float16 h = (_Float16)f;
    uint16_t bits;
    __builtin_memcpy(&bits, &h, 2);
    return bits;
}

__device__ __forceinline__ void store_out(void *out, size_t idx, float val, int dt) {
    if (dt == F32)
        reinterpret_cast<float *>(out)[idx] = val;
    else if (dt == BF16)
        reinterpret_cast<uint16_t *>(out)[idx] = float_to_bf16_bits(val);
    else
        reinterpret_cast<uint16_t *>(out)[idx] = float_to_f16_bits(val);
}

// Split handled by the workgroup at grid column x of (request b, KV head kvh).
// Consecutive workgroups are dealt to the eight XCDs in turn, so with the split
// index fastest in the grid, XCD i would get splits i, i + 8, ... of every
// (request, KV head).  Requests shorter than the longest leave their high
// splits empty, and the leftover splits beyond a multiple of eight would then
// always land on the low XCDs (about 20% more work on XCD 0 than on XCD 7 for
// lengths spread over 1k..16k).  Rotating the split index by the (request, KV
// head) number deals those leftovers to the XCDs in turn.
__device__ __forceinline__ int split_index(int x, int b, int kvh, int Hkv, int S) {
    return (int)(((unsigned)x + (unsigned)(b * Hkv + kvh)) % (unsigned)S);
}

// The workgroup's view of the launch parameters: grid z = b * q_tiles + j
// picks its request b and its query tile, tokens i0 .. i0 + tile_tokens - 1
// (fewer in the last tile), whose rows become rows 0 .. R - 1.  The tiles go
// in reverse (j = 0 is the last tile): later query tokens see more of the
// cache, so the longest workgroups start first and the short ones fill the
// tail.
// Branch-free, so that the compiler issues every parameter load at once (a
// branch on q_tiles delayed the other loads behind it by a load round trip).
__device__ __forceinline__ PartialParams tile_params(const PartialParams &pk, int &b) {
    PartialParams p = pk;
    const unsigned z = blockIdx.z, nt = (unsigned)pk.q_tiles;
    b = (int)(z / nt);
    const int tile = (int)(nt - 1u - (z - (unsigned)b * nt));
    p.i0 = tile * pk.tile_tokens;
    p.R = min(pk.tile_tokens, pk.q_len - p.i0) * pk.G;
    return p;
}

// Query row rho < R of KV head kvh in request b: query token i = i0 + rho / G
// of head kvh * G + rho % G.  Its global row (b * q_len + i) * Hq + head
// indexes q, out and lse; its split slot indexes the partials and flags.
__device__ __forceinline__ size_t query_row(const PartialParams &p, int b, int kvh, int rho) {
    const int t = rho / p.G, g = rho - t * p.G;
    return ((size_t)b * p.q_len + p.i0 + t) * p.Hq + (size_t)kvh * p.G + g;
}

__device__ __forceinline__ size_t row_slot(const PartialParams &p, int b, int kvh, int rho, int s) {
    return query_row(p, b, kvh, rho) * p.max_splits + s;
}

// Causal limit of query row rho inside the split ending at t1: query token i
// sits at position len - q_len + i and sees the tokens up to it.
__device__ __forceinline__ int row_limit(const PartialParams &p, int len, int t1, int rho) {
    const int lim = len - p.q_len + p.i0 + rho / p.G + 1;
    return lim < t1 ? lim : t1;
}

// Tokens of a request of len tokens that some row of the workgroup's tile
// sees: those before its last query token's causal limit.  The splits past
// it are empty for the tile (all len of them when rows are not tiled).
__device__ __forceinline__ int tile_len(const PartialParams &p, int len) {
    const int lim = len - p.q_len + p.i0 + p.R / p.G;
    return lim < 0 ? 0 : lim;
}

// Whole-row fallback, second pass: the query rows (bit rho) of KV head kvh
// of request b with a flagged split among the request's first nsplit splits.
// Every lane of the wave reads a share of the flags; the result is
// wave-uniform.
__device__ __forceinline__ uint32_t rows_flagged_in_request(const PartialParams &p, int b, int kvh, int nsplit) {
    const int lane = threadIdx.x & 63;
    uint32_t m = 0;
    for (int idx = lane; idx < p.R * nsplit; idx += 64) {
        const int rho = idx / nsplit, s = idx - rho * nsplit;
        if (p.flags[row_slot(p, b, kvh, rho, s)]) m |= 1u << rho;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) m |= (uint32_t)__shfl_xor((int)m, off);
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)m);   // uniform: a scalar register
}

// Number of tokens of request b that the kernels read.
__device__ __forceinline__ int request_len(const int32_t *seq_lens, int b, int cap, int limit) {
    int n = seq_lens ? seq_lens[b] : cap;
    n = n < 0 ? 0 : n;
    n = n > cap ? cap : n;
    return n > limit ? limit : n;
}

}  // namespace fd
