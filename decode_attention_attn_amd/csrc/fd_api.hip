// fd_api.hip -- host side of the C ABI declared in include/fd_decode_attn.h:
// argument validation, the split heuristic, workspace layout and kernel
// dispatch.  Nothing here allocates, synchronises or touches device memory.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "fd_decode_attn.h"
#include "fd_internal.h"

#define FD_API extern "C" __attribute__((visibility("default")))

static_assert(FD_TICKET_BYTES == fd::kTicketBytes, "the header's ticket area is the library's");

namespace {

using fd::kMaxGroup;
using fd::kMaxRows;
using fd::kMaxSplits;
using fd::kMaxSplitSize;

bool finite(float x) { return isfinite(x) != 0; }

fd_status validate_desc(const fd_decode_desc *d) {
    if (!d) return FD_ERR_INVALID_ARG;
    if (d->B < 0 || d->B > 65535 || d->Hq <= 0 || d->Hkv <= 0 || d->Hkv > 65535) return FD_ERR_INVALID_ARG;
    if (d->Hq % d->Hkv) return FD_ERR_INVALID_ARG;
    if (d->Hq / d->Hkv > kMaxGroup) return FD_ERR_UNSUPPORTED;
    if (d->q_len > fd::kMaxQueryTokens || (int64_t)d->q_len * d->Hq > INT32_MAX) return FD_ERR_UNSUPPORTED;
    {   // requests x query tiles index grid z; bounded for the kernel with the smaller tiles (16 rows)
        const int64_t tok = kMaxGroup / (d->Hq / d->Hkv), q_len = d->q_len > 1 ? d->q_len : 1;
        if ((int64_t)d->B * ((q_len + tok - 1) / tok) > fd::kMaxGridZ) return FD_ERR_UNSUPPORTED;
    }
    if (d->d != 64 && d->d != 128) return FD_ERR_UNSUPPORTED;
    if (d->kv_dtype < FD_F32 || d->kv_dtype > FD_FP8_E4M3) return FD_ERR_INVALID_ARG;
    if (d->kv_dtype == FD_FP8_E4M3) {
        if (d->q_dtype != FD_F16 && d->q_dtype != FD_BF16) return FD_ERR_INVALID_ARG;
        if (!finite(d->k_scale) || !finite(d->v_scale)) return FD_ERR_INVALID_ARG;
    }
    if (d->out_dtype < FD_F32 || d->out_dtype > FD_BF16) return FD_ERR_INVALID_ARG;
    if (d->split_size < 1 || d->split_size > kMaxSplitSize) return FD_ERR_INVALID_ARG;
    if (d->max_splits < 1 || d->max_splits > kMaxSplits) return FD_ERR_INVALID_ARG;
    if ((int64_t)d->max_splits * d->split_size > INT32_MAX) return FD_ERR_INVALID_ARG;
    if (!finite(d->scale)) return FD_ERR_INVALID_ARG;
    if (d->mode != FD_SOFTMAX_SYNC && d->mode != FD_SOFTMAX_UNIFIED_MAX) return FD_ERR_INVALID_ARG;
    if (d->mode == FD_SOFTMAX_UNIFIED_MAX) {
        if (!finite(d->phi) || !finite(d->lo) || !finite(d->hi)) return FD_ERR_INVALID_ARG;
        if (!(d->lo <= d->hi)) return FD_ERR_INVALID_ARG;
        // exp(s - phi) must stay a finite, normal fp32 number for every in-range score
        if (fabsf(d->lo - d->phi) > fd::kMaxUnifiedRange || fabsf(d->hi - d->phi) > fd::kMaxUnifiedRange)
            return FD_ERR_INVALID_ARG;
    }
    if (d->kernel < FD_KERNEL_AUTO || d->kernel > FD_KERNEL_MFMA) return FD_ERR_INVALID_ARG;
    if (d->merge < FD_MERGE_AUTO || d->merge > FD_MERGE_FUSED) return FD_ERR_INVALID_ARG;
    if (d->fallback < FD_FALLBACK_SPLIT || d->fallback > FD_FALLBACK_ROW) return FD_ERR_INVALID_ARG;
    if (d->kv_dtype == FD_FP8_E4M3 &&
        ((reinterpret_cast<uintptr_t>(d->k_scales) & 3) || (reinterpret_cast<uintptr_t>(d->v_scales) & 3)))
        return FD_ERR_INVALID_ARG;
    return FD_OK;
}

// Compute units of the current device, read once per device (host threads
// may race to fill an entry; they store the same value).
int32_t device_cus() {
    static std::atomic<int32_t> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int32_t n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1) v = 256;
        n = v;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

fd::PartialParams base_params(const fd_decode_desc *d) {
    fd::PartialParams p;
    memset(&p, 0, sizeof p);
    p.B = d->B;
    p.Hq = d->Hq;
    p.Hkv = d->Hkv;
    p.G = d->Hq / d->Hkv;
    p.q_len = d->q_len > 1 ? d->q_len : 1;
    p.q_tiles = 1;
    p.tile_tokens = p.q_len;
    p.R = p.q_len * p.G;
    p.d = d->d;
    p.split = d->split_size;
    p.max_splits = d->max_splits;
    double scale = d->scale > 0.f ? (double)d->scale : (double)(1.0f / sqrtf((float)d->d));
    p.q_dtype = d->kv_dtype;
    p.v_mult = 1.f;
    if (d->kv_dtype == FD_FP8_E4M3) {   // stored K / V values stand for stored * scale
        p.q_dtype = d->q_dtype;
        // per-KV-head scales replace the per-tensor ones; the kernels multiply
        // the score scale and V by the head's entry
        p.k_scales = d->k_scales;
        p.v_scales = d->v_scales;
        if (!d->k_scales) scale *= d->k_scale > 0.f ? (double)d->k_scale : 1.0;
        if (!d->v_scales) p.v_mult = d->v_scale > 0.f ? d->v_scale : 1.f;
    }
    const double log2e = 1.4426950408889634;
    p.scale_log2 = (float)(scale * log2e);
    p.unified = d->mode == FD_SOFTMAX_UNIFIED_MAX;
    p.phi2 = (float)((double)d->phi * log2e);
    p.lo2 = (float)((double)d->lo * log2e);
    p.hi2 = (float)((double)d->hi * log2e);
    p.dtype = d->kv_dtype;
    p.num_cus = device_cus();
    return p;
}

// Which partial kernel runs: MFMA or VALU (FD_ERR_UNSUPPORTED if the one asked
// for cannot), and the query tiles of a KV head's q_len * G query rows: as few
// tiles as the kernel's rows per workgroup allow (32 MFMA, 16 VALU), of
// whole query tokens, balanced (40 single-head tokens: two tiles of 20).
fd_status pick_kernel(const fd_decode_desc *d, fd::PartialParams &p, bool &mfma) {
    mfma = false;
    if (d->kernel == FD_KERNEL_MFMA) {
        if (!fd::mfma_supports(p)) return FD_ERR_UNSUPPORTED;
        mfma = true;
    } else if (d->kernel == FD_KERNEL_AUTO) {
        mfma = fd::mfma_supports(p);
    }
    const int cap = (mfma ? kMaxRows : kMaxGroup) / p.G;   // query tokens per workgroup; G <= 16
    p.q_tiles = (p.q_len + cap - 1) / cap;
    p.tile_tokens = (p.q_len + p.q_tiles - 1) / p.q_tiles;
    p.R = p.tile_tokens * p.G;
    return (int64_t)p.B * p.q_tiles <= fd::kMaxGridZ ? FD_OK : FD_ERR_UNSUPPORTED;   // validate_desc ensures it
}

bool whole_row_fallback(const fd_decode_desc *d) {
    return d->mode == FD_SOFTMAX_UNIFIED_MAX && d->fallback == FD_FALLBACK_ROW;
}

// The split partials.  With the whole-row fallback: the unified pass writes
// every row's partials and the flags, then a synchronized pass rewrites all
// splits of every row that has a flagged split (its workgroups read the
// flags and leave at once where no row of theirs is flagged).
fd_status run_partial(const fd_decode_desc *d, fd::PartialParams &p, hipStream_t stream) {
    bool mfma = false;
    const fd_status st = pick_kernel(d, p, mfma);
    if (st != FD_OK) return st;
    const bool rows = whole_row_fallback(d);
    if (rows && !p.flags) return FD_ERR_INVALID_ARG;   // the second pass reads the flags
    p.row_fallback = rows;
    auto launch = [&](const fd::PartialParams &q) {
        return mfma ? fd::launch_partial_mfma(q, stream) : fd::launch_partial_valu(q, stream);
    };
    hipError_t e = launch(p);
    if (e == hipSuccess && rows) {
        fd::PartialParams r = p;
        r.unified = 0;
        r.row_fallback = 0;
        r.recompute_rows = 1;
        r.fallback_count = nullptr;
        e = launch(r);
    }
    return e == hipSuccess ? FD_OK : FD_ERR_HIP;
}

// Splits per workgroup of the single-launch MFMA kernel: four waves' worth
// of splits, so that the merging workgroup has 256 threads and a head's
// workgroup partials stay few (two for short requests).
int fused_splits_per_wg(const fd::PartialParams &p) { return p.max_splits >= 8 ? 4 : 2; }

// Whether the single-launch merge can run this shape: the counters fit the
// workspace's ticket area, one request's partials span less than 4 GiB (the
// merge addresses them with 32-bit offsets), and one workgroup's merge fits
// its LDS.
bool fused_fits(const fd::PartialParams &p, bool mfma) {
    if ((int64_t)p.B * p.q_tiles * p.Hkv > fd::kMaxTickets) return false;   // one counter per (tile, KV head)
    if ((int64_t)p.q_len * p.Hq * p.max_splits * p.d * 4 >= ((int64_t)1 << 32)) return false;
    const int64_t parts = mfma ? (p.max_splits + p.splits_per_wg - 1) / p.splits_per_wg : p.max_splits;
    return (int64_t)p.R * parts <= fd::kFusedMaxRowParts;
}

// The single launch where it is asked for, and under FD_MERGE_AUTO where it
// was measured to win: it saves the second launch and the re-read of the
// partials, which pays when the partials are many, and costs its
// four-wave workgroups and the tail of the last merges otherwise.  Measured
// on MI355X (bench.py --merge fused / separate, two runs each): B=64 ragged
// paged batch at split 256, 128 MiB of partial rows: 458 against 488 us per
// call; B=4, N=128k at split 1024, 16 MiB: 368 against 361 us; 32k GQA,
// 2 MiB: 29.6 against 29.1-29.3 us; Llama-2-shaped MHA, 256 KiB: 20.7
// against 18.3-18.9 us.  The VALU kernel's single launch keeps one split per
// workgroup (no four-wave groups) and wins while the last workgroup merges
// few splits: fp32 8-head MHA, N=512, 4 splits: 8.8-8.9 against 9.6 us;
// Llama-2-shaped MHA on the VALU kernel, 16 splits: 19.5 against 19.8-19.9
// us; 32k GQA on the VALU kernel, 128 splits: 46.6 against 40.8-41.1 us.
bool fused_wanted(const fd_decode_desc *d, const fd::PartialParams &p, bool mfma) {
    if (d->merge != FD_MERGE_AUTO) return d->merge == FD_MERGE_FUSED;
    if (!mfma && p.max_splits <= 16) return true;
    const double partial_bytes = (double)p.B * p.q_len * p.Hq * p.max_splits * p.d * sizeof(float);
    return partial_bytes >= 64.0 * (1 << 20);
}

// The single launch has no room for the whole-row fallback's second pass.
bool fused_possible(const fd_decode_desc *d, const fd::PartialParams &p, bool mfma) {
    return !whole_row_fallback(d) && fused_fits(p, mfma);
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Alignment of a base pointer (NULL passes: optional tensors are checked for
// presence elsewhere).  Tensors read or written 16 bytes at a time (q, K, V,
// part_o, out) need 16 bytes; the others their element size.
bool aligned(const void *ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

bool aligned_partials(const float *part_o, const float *part_m, const float *part_l) {
    return aligned(part_o, 16) && aligned(part_m, 4) && aligned(part_l, 4);
}

bool aligned_io(const void *q, const void *k, const void *v, const void *out, const float *lse,
                const int32_t *seq_lens, const int32_t *fallback_count) {
    return aligned(q, 16) && aligned(k, 16) && aligned(v, 16) && aligned(out, 16) && aligned(lse, 4) &&
           aligned(seq_lens, 4) && aligned(fallback_count, 4);
}

// Workspace: the single-launch merge's counters (fd::kTicketBytes), then
// part_o, part_m and part_l, each on a 256-byte boundary.
struct WorkspaceLayout {
    size_t o_off, m_off, l_off, total;
};

WorkspaceLayout layout(const fd_decode_desc *d) {
    const size_t rows = (size_t)d->B * (d->q_len > 1 ? d->q_len : 1) * d->Hq * d->max_splits;
    WorkspaceLayout w;
    w.o_off = fd::kTicketBytes;
    w.m_off = w.o_off + round256(rows * d->d * sizeof(float));
    w.l_off = w.m_off + round256(rows * sizeof(float));
    w.total = w.l_off + round256(rows * sizeof(float));
    return w;
}

fd_status run_combine(const fd_decode_desc *d, const float *part_o, const float *part_m, const float *part_l,
                      const int32_t *seq_lens, void *out, float *lse, hipStream_t stream) {
    fd::CombineParams c;
    c.part_o = part_o;
    c.part_m = part_m;
    c.part_l = part_l;
    c.seq_lens = seq_lens;
    c.out = out;
    c.lse = lse;
    c.B = d->B;
    c.Hq = (d->q_len > 1 ? d->q_len : 1) * d->Hq;   // query rows per request
    c.d = d->d;
    c.split = d->split_size;
    c.max_splits = d->max_splits;
    c.out_dtype = d->out_dtype;
    return fd::launch_combine(c, stream) == hipSuccess ? FD_OK : FD_ERR_HIP;
}

}  // namespace

FD_API fd_status fd_decode_attn_partial(const fd_decode_desc *desc, const void *q, const void *k, const void *v,
                                        int32_t kv_capacity, const int32_t *seq_lens, float *part_o,
                                        float *part_m, float *part_l, uint8_t *flags, int32_t *fallback_count,
                                        void *stream) {
    fd_status st = validate_desc(desc);
    if (st != FD_OK) return st;
    if (kv_capacity < 0) return FD_ERR_INVALID_ARG;
    if (desc->B == 0) return FD_OK;
    if (!q || !k || !v || !part_o || !part_m || !part_l) return FD_ERR_INVALID_ARG;
    if (!aligned_io(q, k, v, nullptr, nullptr, seq_lens, fallback_count) ||
        !aligned_partials(part_o, part_m, part_l))
        return FD_ERR_INVALID_ARG;
    fd::PartialParams p = base_params(desc);
    p.q = q;
    p.k = k;
    p.v = v;
    p.seq_lens = seq_lens;
    p.kv_capacity = kv_capacity;
    p.part_o = part_o;
    p.part_m = part_m;
    p.part_l = part_l;
    p.flags = flags;
    p.fallback_count = fallback_count;
    return run_partial(desc, p, static_cast<hipStream_t>(stream));
}

FD_API fd_status fd_decode_attn_combine(const fd_decode_desc *desc, const float *part_o, const float *part_m,
                                        const float *part_l, const int32_t *seq_lens, void *out, float *lse,
                                        void *stream) {
    fd_status st = validate_desc(desc);
    if (st != FD_OK) return st;
    if (desc->B == 0) return FD_OK;
    if (!part_o || !part_m || !part_l || !out) return FD_ERR_INVALID_ARG;
    if (!aligned_partials(part_o, part_m, part_l) || !aligned_io(nullptr, nullptr, nullptr, out, lse, seq_lens, nullptr))
        return FD_ERR_INVALID_ARG;
    return run_combine(desc, part_o, part_m, part_l, seq_lens, out, lse, static_cast<hipStream_t>(stream));
}

FD_API size_t fd_workspace_bytes(const fd_decode_desc *desc) {
    if (validate_desc(desc) != FD_OK) return 0;
    return layout(desc).total;
}

// Partial + merge over the caller's workspace, for both cache layouts:
// a separate combine launch, or the single launch with the merge inside.
fd_status run_full(const fd_decode_desc *desc, fd::PartialParams &p, void *workspace, size_t workspace_bytes,
                   const int32_t *seq_lens, void *out, float *lse, hipStream_t s) {
    if (!aligned(workspace, 256)) return FD_ERR_INVALID_ARG;
    const WorkspaceLayout w = layout(desc);
    if (workspace_bytes < w.total) return FD_ERR_WORKSPACE_TOO_SMALL;
    char *ws = static_cast<char *>(workspace);
    p.part_o = reinterpret_cast<float *>(ws + w.o_off);
    p.part_m = reinterpret_cast<float *>(ws + w.m_off);
    p.part_l = reinterpret_cast<float *>(ws + w.l_off);
    bool mfma = false;
    fd_status st = pick_kernel(desc, p, mfma);
    if (st != FD_OK) return st;
    p.out = out;
    p.lse = lse;
    p.out_dtype = desc->out_dtype;
    if (desc->merge == FD_MERGE_AUTO && p.max_splits == 1 && !p.unified) {
        // one split per row: its partial is the result, written by the partial
        // kernel itself (no partials, no merge: the Flash-Decoding page's
        // "Production Implementation Guidelines" need no split once the batch
        // and heads fill the GPU).  Synchronized softmax only: unified max,
        // with its recompute passes, keeps the partials and the merge.
        p.direct = 1;
        return run_partial(desc, p, s);
    }
    p.splits_per_wg = fused_splits_per_wg(p);
    const bool fits = fused_possible(desc, p, mfma);
    if (desc->merge == FD_MERGE_FUSED && !fits) return FD_ERR_UNSUPPORTED;
    if (fits && fused_wanted(desc, p, mfma)) {
        p.tickets = reinterpret_cast<int32_t *>(ws);
        const hipError_t e = mfma ? fd::launch_partial_mfma(p, s) : fd::launch_partial_valu(p, s);
        return e == hipSuccess ? FD_OK : FD_ERR_HIP;
    }
    st = run_partial(desc, p, s);
    if (st != FD_OK) return st;
    return run_combine(desc, p.part_o, p.part_m, p.part_l, seq_lens, out, lse, s);
}

FD_API fd_status fd_decode_attn(const fd_decode_desc *desc, const void *q, const void *k, const void *v,
                                int32_t kv_capacity, const int32_t *seq_lens, void *workspace, size_t workspace_bytes,
                                void *out, float *lse, uint8_t *flags, int32_t *fallback_count, void *stream) {
    fd_status st = validate_desc(desc);
    if (st != FD_OK) return st;
    if (kv_capacity < 0) return FD_ERR_INVALID_ARG;
    if (desc->B == 0) return FD_OK;
    if (!q || !k || !v || !workspace || !out) return FD_ERR_INVALID_ARG;
    if (!aligned_io(q, k, v, out, lse, seq_lens, fallback_count)) return FD_ERR_INVALID_ARG;
    fd::PartialParams p = base_params(desc);
    p.q = q;
    p.k = k;
    p.v = v;
    p.seq_lens = seq_lens;
    p.kv_capacity = kv_capacity;
    p.flags = flags;
    p.fallback_count = fallback_count;
    return run_full(desc, p, workspace, workspace_bytes, seq_lens, out, lse, static_cast<hipStream_t>(stream));
}

FD_API fd_status fd_decode_attn_paged(const fd_decode_desc *desc, const void *q, const void *k_cache,
                                      const void *v_cache, int32_t num_pages, int32_t page_size,
                                      const int32_t *block_table, int32_t max_blocks_per_seq,
                                      const int32_t *seq_lens, void *workspace, size_t workspace_bytes, void *out,
                                      float *lse, uint8_t *flags, int32_t *fallback_count, void *stream) {
    fd_status st = validate_desc(desc);
    if (st != FD_OK) return st;
    if (page_size < 1 || num_pages < 0 || max_blocks_per_seq < 1) return FD_ERR_INVALID_ARG;
    if (desc->split_size % page_size) return FD_ERR_INVALID_ARG;
    if ((int64_t)max_blocks_per_seq * page_size > INT32_MAX) return FD_ERR_INVALID_ARG;
    if (desc->B == 0) return FD_OK;
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !workspace || !out) return FD_ERR_INVALID_ARG;
    if (!aligned(workspace, 256) || !aligned(block_table, 4) ||
        !aligned_io(q, k_cache, v_cache, out, lse, seq_lens, fallback_count))
        return FD_ERR_INVALID_ARG;
    fd::PartialParams p = base_params(desc);
    p.q = q;
    p.k = k_cache;
    p.v = v_cache;
    p.seq_lens = seq_lens;
    p.block_table = block_table;
    p.page_size = page_size;
    p.max_blocks = max_blocks_per_seq;
    p.num_pages = num_pages;
    p.kv_capacity = max_blocks_per_seq * page_size;
    p.flags = flags;
    p.fallback_count = fallback_count;
    return run_full(desc, p, workspace, workspace_bytes, seq_lens, out, lse, static_cast<hipStream_t>(stream));
}

FD_API fd_status fd_split_heuristic(int32_t B, int32_t Hq, int32_t Hkv, int32_t max_seq_len, int32_t page_size,
                                    int32_t num_cus, int32_t *split_size_out, int32_t *num_splits_out) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || max_seq_len < 0 || page_size < 0 || num_cus < 1)
        return FD_ERR_INVALID_ARG;
    if (!split_size_out || !num_splits_out) return FD_ERR_INVALID_ARG;
    const int64_t unit = page_size > 0 ? page_size : 1;
    const int64_t n = max_seq_len > 0 ? max_seq_len : 1;
    const int64_t work = (int64_t)B * Hkv;                 // workgroups per split index
    const int64_t cus = num_cus;
    int64_t split;
    if (work * ((n + 255) / 256) <= 8 * cus) {
        // at split 256 the grid fits on the GPU at once (<= 8 workgroups per
        // CU): the page's granularity, aiming at about 2 workgroups per CU
        const int64_t want = (2 * cus + work - 1) / work;   // splits per (request, KV head)
        split = std::min<int64_t>(256, std::max<int64_t>(128, (n + want - 1) / want));
    } else {
        // several waves of workgroups: every split costs a partial write, so
        // grow the split up to 1024 while the grid keeps ~8 workgroups per CU
        split = std::min<int64_t>(1024, std::max<int64_t>(256, (n * work + 8 * cus - 1) / (8 * cus)));
    }
    split = std::max<int64_t>(split, (n + kMaxSplits - 1) / kMaxSplits);
    split = (split + unit - 1) / unit * unit;             // whole pages
    if (split > kMaxSplitSize) split = (kMaxSplitSize / unit) * unit;
    if (split < 1) return FD_ERR_UNSUPPORTED;
    const int64_t S = (n + split - 1) / split;
    if (S > kMaxSplits) return FD_ERR_UNSUPPORTED;
    *split_size_out = (int32_t)split;
    *num_splits_out = (int32_t)S;
    return FD_OK;
}

FD_API const char *fd_status_string(fd_status status) {
    switch (status) {
    case FD_OK: return "FD_OK";
    case FD_ERR_INVALID_ARG: return "FD_ERR_INVALID_ARG";
    case FD_ERR_UNSUPPORTED: return "FD_ERR_UNSUPPORTED";
    case FD_ERR_WORKSPACE_TOO_SMALL: return "FD_ERR_WORKSPACE_TOO_SMALL";
    case FD_ERR_HIP: return "FD_ERR_HIP";
    }
    return "FD_UNKNOWN_STATUS";
}
