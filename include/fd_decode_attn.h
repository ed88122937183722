/*
 * fd_decode_attn.h -- C ABI of the split-KV decode-attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes exact single-query attention o = softmax(q K^T / sqrt(d)) V
 * over a long KV cache (page "Flash-Decoding: Mathematical Foundations, Split-KV
 * Parallelism, Online Softmax Reduction, and Serving Latency Optimization",
 * section "The Single-Token Generation Bottleneck"), parallelised along the KV
 * sequence: each split of `split_size` tokens yields partials (m, l, O)
 * (same page, "Mathematical Formulation of Split-KV Parallelism") that a second
 * kernel merges exactly by log-sum-exp ("The Rescaling and Online Softmax
 * Reduction Algorithm"; the two launches follow "Hardware Execution Topology
 * and Memory Traffic").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    library never allocates, frees or synchronises; it enqueues kernels on
 *    `stream` (a hipStream_t; NULL = the null stream) and returns a status.
 *    Device faults (for instance from a table entry the caller got wrong) show
 *    up at the caller's next synchronisation, not in the status.
 *  - Tensors are dense and row-major; offsets are computed in 64 bits.  q, K,
 *    V, part_o and out must be 16-byte aligned (they move 16 bytes at a time;
 *    the Flash-Decoding page's "Production Implementation Guidelines" ask for
 *    aligned buffers), every other tensor aligned to its element size;
 *    a misaligned pointer returns FD_ERR_INVALID_ARG.
 *  - q has shape [B, q_len, Hq, d] ([B, Hq, d] for q_len = 1) and the same
 *    element type as the cache, except with an 8-bit cache, where q is f16 or
 *    bf16 (desc->q_dtype).
 *  - Query rows: r = (b * q_len + i) * Hq + h is query token i of request b,
 *    head h.  With q_len > 1 (drafted tokens to verify, or a chunk of new
 *    tokens whose K and V are already in the cache) the q_len tokens are the
 *    last q_len positions of the request and attend causally: token i sees
 *    cache tokens t <= len_b - q_len + i (the causal mask of the handbook's
 *    FlashAttention forward kernel, page "FlashAttention and inference
 *    kernels", section "FlashAttention: tiling plus online softmax").  Every
 *    per-head shape below is per query row: out [B, q_len, Hq, d], lse, m, l
 *    and flags [B, q_len, Hq, ...].  q_len <= FD_MAX_Q_LEN and
 *    q_len * Hq < 2^31.  A workgroup holds up to 32 query rows of one KV
 *    head (MFMA kernel; VALU kernel: 16): a KV head with more rows, e.g. a
 *    prefill chunk, is processed in query tiles of whole query tokens, each
 *    tile its own set of split workgroups that reads only the cache tokens
 *    its rows can see.  The handbook page's forward kernel likewise gives
 *    each block of query rows its own pass over K and V (section "A working
 *    FlashAttention forward kernel"), and the tiled causal algorithm skips
 *    the tiles past the diagonal (section "How FlashAttention evolved").
 *    B * ceil(q_len / floor(16 / (Hq / Hkv))) must stay <= 65535 (the tile
 *    count of the VALU kernel, the larger of the two), else
 *    FD_ERR_UNSUPPORTED.
 *  - 8-bit caches (FD_FP8_E4M3, OCP FP8 E4M3: bias 7, no infinities, largest
 *    finite 448, S.1111.111 = NaN) stand for stored * k_scale and
 *    stored * v_scale, with one scale per tensor or one per KV head
 *    (desc->k_scales, desc->v_scales); the handbook page lists caches
 *    stored in FP8, read in wide loads and converted in registers (section
 *    "A paged decode attention kernel (with GQA)", its list of improvements).
 *  - GQA: query head h reads KV head h / (Hq / Hkv); consecutive query heads
 *    share a KV head (page "FlashAttention and inference kernels", section
 *    "A paged decode attention kernel (with GQA)").  Hq must be a multiple
 *    of Hkv, and Hq / Hkv <= 16.
 *  - d is 64 or 128.
 *  - seq_lens (int32 [B], device) gives each request's number of tokens; NULL
 *    means every request holds `kv_capacity` tokens.  Negative lengths count
 *    as 0; lengths beyond the cache or beyond max_splits * split_size are
 *    clamped to what fits.
 *  - Split s of request b covers tokens [s * split_size, min((s+1) * split_size,
 *    len_b)); the last split holds the remainder.  A split with no tokens
 *    reports m = -inf, l = 0 and leaves its O row unwritten.
 *  - Partials (fp32): part_o [B, q_len, Hq, max_splits, d] holds the split's
 *    output already divided by its l; part_m, part_l [B, q_len, Hq, max_splits]
 *    hold the
 *    split's scaling constant m (natural-log units of scaled scores) and
 *    l = sum_t exp(s_t - m).
 *  - lse (fp32 [B, q_len, Hq]) = ln sum_t exp(s_t) with s_t = scale * <q, k_t>;
 *    -inf for a row that sees no token, whose out row is 0.
 *  - Results are bitwise repeatable run to run (no floating-point atomics).
 *  - Errors are returned, never thrown; on error nothing is enqueued.
 */
#ifndef FD_DECODE_ATTN_H
#define FD_DECODE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fd_status {
    FD_OK = 0,
    FD_ERR_INVALID_ARG = 1,          /* a NULL where a tensor is required, a bad size or range */
    FD_ERR_UNSUPPORTED = 2,          /* a valid request the library has no kernel for */
    FD_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes < fd_workspace_bytes(desc) */
    FD_ERR_HIP = 4                   /* the HIP runtime rejected a launch */
} fd_status;

typedef enum fd_dtype { FD_F32 = 0, FD_F16 = 1, FD_BF16 = 2, FD_FP8_E4M3 = 3 /* K and V only */ } fd_dtype;

/* Softmax scaling inside a split.
 * SYNC: each split tracks its own running maximum (the FlashAttention online
 *   recurrence, page "FlashAttention and inference kernels", section
 *   "FlashAttention: tiling plus online softmax").
 * UNIFIED_MAX: every split scales by the same constant phi and keeps plain
 *   numerator / denominator sums; a split holding a score outside [lo, hi] is
 *   flagged and recomputed with SYNC (page "FlashDecoding++: Faster Large
 *   Language Model Inference on GPUs", section "Asynchronized Softmax with
 *   Unified Max Value", Eq. 3 and 4, "The Overflow Fallback: Recomputation"). */
typedef enum fd_softmax_mode { FD_SOFTMAX_SYNC = 0, FD_SOFTMAX_UNIFIED_MAX = 1 } fd_softmax_mode;

/* What UNIFIED_MAX recomputes with SYNC when a score leaves [lo, hi].
 * SPLIT: the flagged split only, inside the partial kernel (exact, since the
 *   merge of split partials is exact).
 * ROW: every split of a query row that has a flagged split -- the
 *   FlashDecoding++ page's own granularity ("The Overflow Fallback:
 *   Recomputation" recomputes the whole attention row) -- by a second,
 *   synchronized launch over the flagged rows; needs flags (not NULL) and
 *   the separate merge. */
typedef enum fd_fallback { FD_FALLBACK_SPLIT = 0, FD_FALLBACK_ROW = 1 } fd_fallback;

/* Which split-partial kernel runs.  Every choice computes the same result to
 * within floating-point rounding. */
typedef enum fd_kernel {
    FD_KERNEL_AUTO = 0,  /* the fastest kernel for the shape */
    FD_KERNEL_VALU = 1,  /* vector-ALU dot products; every dtype */
    FD_KERNEL_MFMA = 2   /* matrix cores; 16- and 8-bit caches, d in {64, 128}, pages of a
                            multiple of 16 tokens; not with f16 q in UNIFIED_MAX mode */
} fd_kernel;

/* How the split partials are merged by fd_decode_attn and fd_decode_attn_paged.
 * SEPARATE: a second kernel launch merges them (the Flash-Decoding page's
 *   "Hardware Execution Topology and Memory Traffic": partials to global
 *   memory, then a reduction kernel).
 * FUSED: one launch; the last workgroup of each (request, KV head) to finish
 *   merges that head's partials (the FlashDecoding++ page, "Asynchronized
 *   Softmax with Unified Max Value", its design choices: a reduction across
 *   workers by atomics instead of a relaunch).  Needs the workspace's ticket
 *   area to be zero when the call starts (see fd_workspace_bytes); requires
 *   B * (query tiles) * Hkv <= 65536 and reports shapes whose merge does not
 *   fit one workgroup, and FD_FALLBACK_ROW, FD_ERR_UNSUPPORTED.
 * AUTO: whichever the library measured faster for the shape; with
 *   max_splits == 1 in FD_SOFTMAX_SYNC mode neither: each row's one split is
 *   its result, which the partial kernel writes to out and lse itself (the
 *   workspace's partials are then left unwritten), as the Flash-Decoding
 *   page's "Production Implementation Guidelines" drop the split once batch
 *   and heads fill the GPU.
 * Both give the same result to within floating-point rounding (the merge is
 * exact; FUSED takes it as a tree: the splits of a workgroup, then the
 * workgroups).  fd_decode_attn_partial and fd_decode_attn_combine ignore it. */
typedef enum fd_merge { FD_MERGE_AUTO = 0, FD_MERGE_SEPARATE = 1, FD_MERGE_FUSED = 2 } fd_merge;

typedef struct fd_decode_desc {
    int32_t B, Hq, Hkv, d;   /* batch, query heads, KV heads, head dimension */
    int32_t kv_dtype;        /* fd_dtype of K and V (and of q, unless FD_FP8_E4M3) */
    int32_t out_dtype;       /* fd_dtype of out (not FD_FP8_E4M3) */
    int32_t split_size;      /* tokens per split, 1..2^20; a multiple of page_size when paged */
    int32_t max_splits;      /* S_max, the split extent of the partial buffers, 1..4096;
                                max_splits * split_size < 2^31 */
    float scale;             /* score = scale * <q, k>; <= 0 selects 1 / sqrt(d) */
    int32_t mode;            /* fd_softmax_mode */
    float phi, lo, hi;       /* UNIFIED_MAX: p = exp(s - phi); flag when s < lo or s > hi.
                                Requires lo <= hi, all finite, |lo - phi| <= 64 and
                                |hi - phi| <= 64, so that exp(s - phi) of an in-range
                                score and its sums stay finite, normal fp32 numbers. */
    int32_t kernel;          /* fd_kernel */
    int32_t q_dtype;         /* FD_FP8_E4M3 caches: fd_dtype of q, FD_F16 or FD_BF16;
                                ignored otherwise (q has kv_dtype) */
    float k_scale, v_scale;  /* FD_FP8_E4M3 caches: a stored K / V value stands for
                                stored * scale; <= 0 selects 1; ignored otherwise */
    int32_t q_len;           /* query tokens per request, causal; <= 0 selects 1 */
    const float *k_scales;   /* FD_FP8_E4M3 caches: NULL, or a device array [Hkv] of per-KV-head K
                                scales replacing k_scale (values finite and > 0, not checked);
                                4-byte aligned; ignored for other caches */
    const float *v_scales;   /* the same for V, replacing v_scale */
    int32_t merge;           /* fd_merge */
    int32_t fallback;        /* fd_fallback (UNIFIED_MAX only) */
} fd_decode_desc;

/* Split-partial kernel over a contiguous cache.
 *   k, v          : [B, kv_capacity, Hkv, d] of kv_dtype
 *   part_o/m/l    : as in the conventions above (written for every split < max_splits)
 *   flags         : uint8 [B, q_len, Hq, max_splits] or NULL (required by
 *                   FD_FALLBACK_ROW); UNIFIED_MAX writes 1 for a
 *                   (request, query head, split) whose scores left [lo, hi], else 0
 *   fallback_count: int32 [1] or NULL; UNIFIED_MAX adds the number of flagged
 *                   (request, query head, split) triples (set it to 0 first for
 *                   a per-call count)
 * Splits follow the Flash-Decoding page, "Mathematical Formulation of Split-KV
 * Parallelism". */
fd_status fd_decode_attn_partial(const fd_decode_desc *desc, const void *q, const void *k,
                                 const void *v, int32_t kv_capacity, const int32_t *seq_lens,
                                 float *part_o, float *part_m, float *part_l, uint8_t *flags,
                                 int32_t *fallback_count, void *stream);

/* Exact merge of the partials of every (request, query head):
 * m = max_s m_s, w_s = l_s exp(m_s - m) over splits with l_s > 0, l = sum w_s,
 * out = sum_s w_s O_s / l, lse = m + ln l (Flash-Decoding page, "The Rescaling
 * and Online Softmax Reduction Algorithm"; empty splits skipped as in the
 * handbook's split-K merge exercise).  Request b reads splits
 * s < ceil(len_b / split_size) (all max_splits when seq_lens is NULL; then
 * kv_capacity is unused).  out: [B, q_len, Hq, d] of out_dtype; lse: fp32 [B, q_len, Hq] or NULL. */
fd_status fd_decode_attn_combine(const fd_decode_desc *desc, const float *part_o, const float *part_m,
                                 const float *part_l, const int32_t *seq_lens, void *out, float *lse,
                                 void *stream);

/* Partial + merge over a contiguous cache: fd_decode_attn_partial followed by
 * fd_decode_attn_combine, or the single launch (desc->merge), with the
 * partials in the caller's workspace (layout as for fd_decode_attn_paged).
 *   k, v : [B, kv_capacity, Hkv, d] of kv_dtype
 *   out, lse, flags, fallback_count : as for the entry points above.
 * Split partials are the Flash-Decoding page's "Mathematical Formulation of
 * Split-KV Parallelism", their merge its "The Rescaling and Online Softmax
 * Reduction Algorithm". */
fd_status fd_decode_attn(const fd_decode_desc *desc, const void *q, const void *k, const void *v,
                         int32_t kv_capacity, const int32_t *seq_lens, void *workspace, size_t workspace_bytes,
                         void *out, float *lse, uint8_t *flags, int32_t *fallback_count, void *stream);

/* Partial + merge over a paged cache (page "FlashAttention and inference
 * kernels", section "PagedAttention": token t of request b lives at slot
 * t % page_size of physical block block_table[b][t / page_size]).
 *   k_cache, v_cache : [num_pages, page_size, Hkv, d] of kv_dtype
 *   block_table      : int32 [B, max_blocks_per_seq]; entries past a request's
 *                      last page are not read.  An entry outside
 *                      [0, num_pages) is never dereferenced: its tokens count
 *                      as absent.
 *   workspace        : >= fd_workspace_bytes(desc) bytes of device memory, 256-byte
 *                      aligned: FD_TICKET_BYTES of merge counters, then part_o,
 *                      part_m and part_l, each starting on a 256-byte boundary.
 *                      The counters must be zero before the first single-launch
 *                      call on a workspace (allocate it zeroed, or clear the
 *                      first FD_TICKET_BYTES once); every completed call leaves
 *                      them zero.  Calls that overlap on one workspace race.
 *   flags, fallback_count : as for fd_decode_attn_partial.
 * split_size must be a multiple of page_size so that split boundaries fall on
 * page boundaries (Flash-Decoding page, "Production Implementation Guidelines"). */
fd_status fd_decode_attn_paged(const fd_decode_desc *desc, const void *q, const void *k_cache,
                               const void *v_cache, int32_t num_pages, int32_t page_size,
                               const int32_t *block_table, int32_t max_blocks_per_seq,
                               const int32_t *seq_lens, void *workspace, size_t workspace_bytes,
                               void *out, float *lse, uint8_t *flags, int32_t *fallback_count,
                               void *stream);

/* fd_decode_attn_paged for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, whose role a
 * file-scope device array of FD_NOALLOC_SCRATCH_BYTES bytes takes, one per GPU,
 * held until the process ends.  The call itself allocates nothing; its first
 * call on a device looks up that device's copy of the array.
 *   Returns FD_ERR_WORKSPACE_TOO_SMALL when fd_workspace_bytes(desc) exceeds
 *   FD_NOALLOC_SCRATCH_BYTES, FD_ERR_HIP if the array's address cannot be had;
 *   otherwise exactly what fd_decode_attn_paged returns, with the same results.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (on different streams, or from different host threads without
 * ordering) race and give wrong results; calls ordered on one stream are safe.
 * The array keeps the last call's partials; nothing in it is read before this
 * call writes it. */
#define FD_NOALLOC_SCRATCH_BYTES (64u << 20)
fd_status fd_decode_attn_paged_noalloc(const fd_decode_desc *desc, const void *q, const void *k_cache,
                                       const void *v_cache, int32_t num_pages, int32_t page_size,
                                       const int32_t *block_table, int32_t max_blocks_per_seq,
                                       const int32_t *seq_lens, void *out, float *lse, uint8_t *flags,
                                       int32_t *fallback_count, void *stream);

/* Most query tokens per request (desc->q_len). */
#define FD_MAX_Q_LEN 65536

/* Bytes of the merge counters at the start of a workspace. */
#define FD_TICKET_BYTES (65536u * 4u)

/* Bytes of workspace fd_decode_attn and fd_decode_attn_paged need for `desc`
 * (0 for an invalid desc): the counters plus the fp32 partials. */
size_t fd_workspace_bytes(const fd_decode_desc *desc);

/* Host-only split choice, no GPU call.  Work units W = B * Hkv (one workgroup
 * covers a GQA group), S256 = ceil(N / 256).
 *   W * S256 <= 8 * num_cus (the grid fits on the GPU at once): the split
 *     gives about 2 * num_cus workgroups, clamped to 128..256 tokens (the
 *     Flash-Decoding page's granularity, "Production Implementation
 *     Guidelines").
 *   otherwise: split = ceil(N * W / (8 * num_cus)) clamped to 256..1024, so
 *     the grid keeps about 8 workgroups per CU while writing fewer partials.
 *     This departs from the page's "no split once B * H >= 2 * SMs" rule:
 *     on MI355X one workgroup streams a (request, KV head) far slower than
 *     the GPU's share of bandwidth, and partial writes interleaved with
 *     saturated reads are expensive (measured: B=4, N=128k GQA 399 -> 353 us
 *     per step at split 1024; B=64 ragged paged 495 -> 482 us).
 * The split is then raised so that S <= 4096 and rounded up to whole pages;
 * S = ceil(N / split) ("Mathematical Formulation of Split-KV Parallelism").
 * page_size 0 means a contiguous cache. */
fd_status fd_split_heuristic(int32_t B, int32_t Hq, int32_t Hkv, int32_t max_seq_len, int32_t page_size,
                             int32_t num_cus, int32_t *split_size_out, int32_t *num_splits_out);

/* Static, NUL-terminated name of a status. */
const char *fd_status_string(fd_status status);

#ifdef __cplusplus
}
#endif

#endif /* FD_DECODE_ATTN_H */
