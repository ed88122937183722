// fd_internal.h -- launch parameters shared by the host entry points and the
// gfx950 kernels of the split-KV decode-attention library.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fd {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxGroup = 16;       // query heads per KV head
constexpr int kMaxRows = 32;        // query rows per workgroup (MFMA kernel; VALU: kMaxGroup)
constexpr int kMaxQueryTokens = 65536;
constexpr int kMaxGridZ = 65535;    // requests x row tiles
constexpr int kMaxSplits = 4096;    // the combine stages m and l of every split in LDS
constexpr int kMaxSplitSize = 1 << 20;
// single-launch merge: query rows x partials that one workgroup merges
constexpr int kFusedMaxRowParts = 2048;
// single-launch merge: (request, KV head) counters at the start of the workspace
constexpr int kMaxTickets = 65536;
constexpr size_t kTicketBytes = kMaxTickets * sizeof(int32_t);
// unified max: |lo - phi|, |hi - phi| bound, so exp(s - phi) <= e^64 leaves
// fp32 headroom for sums of up to 2^20 terms times |v|
constexpr float kMaxUnifiedRange = 64.f;

enum DType : int32_t { F32 = 0, F16 = 1, BF16 = 2, FP8 = 3 };   // FP8: OCP E4M3, K and V only

// Everything a split-partial kernel reads.  Scores are handled in log2
// units: s2 = scale * log2(e) * <q, k>, so that exp(s - m) = exp2(s2 - m2).
struct PartialParams {
    const void *q;              // [B, Hq, d]
    const void *k;              // contiguous [B, cap, Hkv, d] or paged [P, page, Hkv, d]
    const void *v;
    const int32_t *seq_lens;    // [B] or nullptr
    const int32_t *block_table; // [B, max_blocks] (paged) or nullptr
    float *part_o;              // [B, Hq, S_max, d]
    float *part_m;              // [B, Hq, S_max]  natural-log units
    float *part_l;              // [B, Hq, S_max]
    uint8_t *flags;             // [B, Hq, S_max] or nullptr
    int32_t *fallback_count;    // [1] or nullptr
    int32_t B, Hq, Hkv, G, d;
    int32_t q_len;              // query tokens per request (causal)
    int32_t R;                  // query rows of a workgroup: host, a full tile's; device, its own tile's
    int32_t kv_capacity;        // contiguous: tokens per request row; paged: max_blocks * page
    int32_t page_size;          // 0 = contiguous
    int32_t max_blocks;
    int32_t num_pages;
    int32_t split, max_splits;
    float scale_log2;           // scale * log2(e)
    float phi2, lo2, hi2;       // unified max, log2 units
    int32_t unified;            // 1 = unified max with fallback
    int32_t dtype;              // DType of k and v (and of q unless FP8)
    int32_t q_dtype;            // DType of q (F16 or BF16 when dtype is FP8)
    float v_mult;               // FP8: value of one stored V unit (v_scale); else 1
    const float *k_scales;      // FP8: per-KV-head K scales [Hkv] or nullptr (then scale_log2 holds k_scale)
    const float *v_scales;      // FP8: per-KV-head V scales [Hkv] or nullptr (then v_mult)
    int32_t num_cus;            // compute units of the device (launch-shape choice only)
    // single-launch merge (tickets != nullptr): one counter per (request, KV
    // head), zero on entry and left zero; the merged result goes to out / lse
    int32_t *tickets;
    void *out;                  // [B, q_len * Hq, d] of out_dtype
    float *lse;                 // [B, q_len * Hq] or nullptr
    int32_t out_dtype;
    int32_t splits_per_wg;      // MFMA kernel: consecutive splits per workgroup (2 or 4)
    // one split per row (max_splits == 1): the partial kernel writes the
    // result itself to out / lse (out_dtype) and no partials
    int32_t direct;
    // whole-row fallback of unified max: the unified pass writes every row's
    // partial and only flags (row_fallback); a second, synchronized pass
    // (recompute_rows) rewrites every split of the rows flagged anywhere
    int32_t row_fallback;
    int32_t recompute_rows;
    // A KV head's q_len * G query rows go in query tiles of tile_tokens whole
    // query tokens (the last tile may be shorter); grid z = b * q_tiles + tile.
    // (Last in the struct: the kernels' first parameter loads keep their shape.)
    int32_t q_tiles;
    int32_t tile_tokens;
    int32_t i0;                 // device: first query token of the workgroup's tile
};

struct CombineParams {
    const float *part_o, *part_m, *part_l;
    const int32_t *seq_lens;
    void *out;                  // [B, Hq, d]
    float *lse;                 // [B, Hq] or nullptr
    int32_t B, Hq, d;           // Hq: query rows per request (q_len * heads)
    int32_t split, max_splits;
    int32_t out_dtype;
};

// Each launcher checks nothing (the entry points validate) and returns the
// launch status.
hipError_t launch_partial_valu(const PartialParams &p, hipStream_t stream);
hipError_t launch_partial_mfma(const PartialParams &p, hipStream_t stream);
// one per instantiation type (operand type, and whether the cache is E4M3)
hipError_t launch_partial_mfma_f16(const PartialParams &p, hipStream_t stream);
hipError_t launch_partial_mfma_bf16(const PartialParams &p, hipStream_t stream);
hipError_t launch_partial_mfma_f8f16(const PartialParams &p, hipStream_t stream);
hipError_t launch_partial_mfma_f8bf16(const PartialParams &p, hipStream_t stream);
bool mfma_supports(const PartialParams &p);
hipError_t launch_combine(const CombineParams &p, hipStream_t stream);

}  // namespace fd
