/*
 * oracle.c -- plain, slow fp64 CPU reference for single-query decode attention.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the GPU library, and the GPU library never calls it.
 *
 * What it computes (every function below cites the passage it follows):
 *
 *   o = softmax(q K^T / sqrt(d)) V  for one query row
 *     -- "Flash-Decoding: Mathematical Foundations, Split-KV Parallelism, ...",
 *        section "The Single-Token Generation Bottleneck" (definition of o_t).
 *   two passes (max, then exp-sum and weighted V), fp64 throughout
 *     -- "FlashAttention and inference kernels", section "A paged decode
 *        attention kernel (with GQA)", its CPU reference: dot in double, then
 *        times the scale, max, exp, sum, weighted V, divide.
 *   GQA: query head h reads KV head h / (Hq / Hkv)   -- same section.
 *   paged cache: token t lives at slot t % page of physical block
 *     block_table[t / page]   -- same page, section "PagedAttention".
 *   per-split partials m, l, O (O normalised by l)
 *     -- Flash-Decoding page, "Mathematical Formulation of Split-KV Parallelism".
 *   exact merge (max-rescale form and log-sum-exp alpha form)
 *     -- Flash-Decoding page, "The Rescaling and Online Softmax Reduction
 *        Algorithm"; empty splits (l = 0, m = -inf) are skipped as in the
 *        handbook's split-K merge exercise.
 *   FlashAttention tile recurrence (m, l, O rescaled per tile, divide at end)
 *     -- handbook, "FlashAttention: tiling plus online softmax".
 *   unified max value: every split uses the same constant phi, numerator and
 *   denominator sums per split, one final reduction; a split whose scores
 *   leave the safe range is flagged and recomputed with its own max
 *     -- "FlashDecoding++: Faster Large Language Model Inference on GPUs",
 *        "Asynchronized Softmax with Unified Max Value" (Eq. 3, Eq. 4,
 *        "The Overflow Fallback: Recomputation", Figure 6).
 *
 *   8-bit KV cache: the handbook page lists KV caches stored in FP8 and read
 *   in wide loads, converted in registers (section "A paged decode attention
 *   kernel (with GQA)", its list of improvements; section on the KV cache's
 *   size names KV cache quantization).  The format is OCP FP8 E4M3 (OCP 8-bit
 *   Floating Point Specification, "E4M3"); a stored K or V value means
 *   stored * k_scale or stored * v_scale, with one scale per tensor or, when
 *   per-head arrays are given, one per KV head (the scale of KV head kvh
 *   multiplies every element of that head's rows).
 *   several query tokens per request (verification of drafted tokens, or a
 *   chunk of new tokens whose K and V are already in the cache): the causal
 *   mask of the handbook's FlashAttention forward kernel (section
 *   "FlashAttention: tiling plus online softmax", its causal flag: query
 *   row i sees keys j <= i), with the q_len new tokens at the last q_len
 *   positions of the request: query i sees tokens t <= len - q_len + i.
 *
 * Readings taken where the pages leave a step open:
 *   - the last split holds the remainder n - (S-1)*split tokens;
 *   - a split with no tokens is reported as m = -inf, l = 0, O = 0;
 *   - a request of length 0 gives out = 0, lse = -inf;
 *   - safe range given as absolute score bounds [lo, hi]; a score exactly on
 *     a bound is in range (the FlashDecoding++ worked example passes 9-6 = 3
 *     = b); a split is flagged iff some score s < lo or s > hi;
 *   - the fallback recomputes the flagged split only (its merge is exact, so
 *     the result does not depend on this choice); whole_row = 1 takes the
 *     page's own granularity instead: a row with any flagged split has every
 *     one of its splits recomputed with the synchronized softmax.
 *
 * Parity pins for every function live in tests/test_oracle.py.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

/* storage types of q, K and V */
#define ODT_F32 0
#define ODT_F16 1
#define ODT_BF16 2
#define ODT_FP8_E4M3 3   /* K and V only */

typedef struct {
    int32_t B, Hq, Hkv, d;
    int32_t dtype;       /* ODT_* : storage type of k and v                   */
    int32_t N;           /* contiguous: token capacity per request            */
    int32_t page_size;   /* 0 -> contiguous [B][N][Hkv][d]; else paged        */
    int32_t max_blocks;  /* paged: row length of block_table                  */
    double scale;        /* score = scale * <q, k>                            */
    int32_t q_dtype;     /* ODT_F32 / F16 / BF16: storage type of q           */
    double k_scale;      /* a stored K value means stored * k_scale            */
    double v_scale;      /* a stored V value means stored * v_scale            */
    int32_t q_len;       /* query tokens per request (q is [B][q_len][Hq][d]) */
    const double *k_scales;  /* [Hkv] or NULL: per-KV-head K scales, replacing k_scale */
    const double *v_scales;  /* [Hkv] or NULL: per-KV-head V scales, replacing v_scale */
} oracle_problem;

/* the scale a stored K / V value of KV head kvh is multiplied by */
static double k_scale_of(const oracle_problem *p, int kvh) { return p->k_scales ? p->k_scales[kvh] : p->k_scale; }
static double v_scale_of(const oracle_problem *p, int kvh) { return p->v_scales ? p->v_scales[kvh] : p->v_scale; }

/* ---------------------------------------------------------------------- */
/* exact decoding of the storage types                                     */
/* ---------------------------------------------------------------------- */
static double f16_bits_to_double(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25);    /* 1.m * 2^(e-15)       */
    return sign ? -v : v;
}

static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP FP8 E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0
 * is subnormal (m * 2^-9); S.1111.111 is NaN; there are no infinities, the
 * largest finite magnitude is 448. */
static double e4m3_bits_to_double(uint8_t b)
{
    int sign = b >> 7, e = (b >> 3) & 0xf, m = b & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);                  /* subnormal: m/8 * 2^-6 */
    else
        v = ldexp((double)(m | 8), e - 10);        /* 1.m * 2^(e-7)         */
    return sign ? -v : v;
}

static double elem(const void *base, int dtype, size_t i)
{
    switch (dtype) {
    case ODT_F32: return (double)((const float *)base)[i];
    case ODT_F16: return f16_bits_to_double(((const uint16_t *)base)[i]);
    case ODT_FP8_E4M3: return e4m3_bits_to_double(((const uint8_t *)base)[i]);
    default:      return bf16_bits_to_double(((const uint16_t *)base)[i]);
    }
}

void oracle_decode(int dtype, const void *src, size_t n, double *dst)
{
    for (size_t i = 0; i < n; ++i) dst[i] = elem(src, dtype, i);
}

/* ---------------------------------------------------------------------- */
/* addressing                                                              */
/* ---------------------------------------------------------------------- */
/* element index of (token t, dim 0) of KV head kvh for request b */
static size_t kv_row(const oracle_problem *p, const int32_t *block_table, int b, int t, int kvh)
{
    size_t row; /* index of the (token, kv head) row, in units of d elements */
    if (p->page_size == 0) {
        row = ((size_t)b * p->N + t) * p->Hkv + kvh;
    } else {
        int32_t phys = block_table[(size_t)b * p->max_blocks + t / p->page_size];
        int slot = t % p->page_size;
        row = ((size_t)phys * p->page_size + slot) * p->Hkv + kvh;
    }
    return row * (size_t)p->d;
}

static int check_problem(const oracle_problem *p, const int32_t *seq_lens, const int32_t *block_table)
{
    if (!p || p->B < 0 || p->Hq <= 0 || p->Hkv <= 0 || p->d <= 0) return ORACLE_EINVAL;
    if (p->Hq % p->Hkv) return ORACLE_EINVAL;
    if (p->q_len < 1) return ORACLE_EINVAL;
    if (p->dtype < ODT_F32 || p->dtype > ODT_FP8_E4M3) return ORACLE_EINVAL;
    if (p->q_dtype < ODT_F32 || p->q_dtype > ODT_BF16) return ORACLE_EINVAL;
    if (!(p->k_scale > 0.0) || !(p->v_scale > 0.0) || isinf(p->k_scale) || isinf(p->v_scale))
        return ORACLE_EINVAL;
    for (int h = 0; h < p->Hkv; ++h)
        if (!(k_scale_of(p, h) > 0.0) || !(v_scale_of(p, h) > 0.0) || isinf(k_scale_of(p, h)) ||
            isinf(v_scale_of(p, h)))
            return ORACLE_EINVAL;
    if (p->page_size < 0) return ORACLE_EINVAL;
    if (p->page_size > 0 && (!block_table || p->max_blocks <= 0)) return ORACLE_EINVAL;
    for (int b = 0; b < p->B; ++b) {
        int n = seq_lens ? seq_lens[b] : p->N;
        if (n < 0) return ORACLE_EINVAL;
        if (p->page_size == 0 && n > p->N) return ORACLE_EINVAL;
        if (p->page_size > 0 && (n + p->page_size - 1) / p->page_size > p->max_blocks) return ORACLE_EINVAL;
    }
    return ORACLE_OK;
}

/* Row r = (b * q_len + i) * Hq + h is query token i of request b, head h;
 * it reads tokens [0, row_tokens) of the request: the causal limit of query
 * token i, len - q_len + i + 1, clamped to [0, len]. */
static void row_coords(const oracle_problem *p, int r, int *b, int *h)
{
    *b = r / (p->q_len * p->Hq);
    *h = r % p->Hq;
}

static int row_tokens(const oracle_problem *p, const int32_t *seq_lens, int r)
{
    int b = r / (p->q_len * p->Hq), i = (r / p->Hq) % p->q_len;
    int n = seq_lens ? seq_lens[b] : p->N;
    int lim = n - p->q_len + i + 1;
    lim = lim < 0 ? 0 : lim;
    return lim < n ? lim : n;
}

/* scores s_t = scale * <q_r, k_t> for t in [t0, t1), fp64, sequential sums */
static void scores(const oracle_problem *p, const void *q, const void *k, const int32_t *block_table,
                   int r, int b, int h, int t0, int t1, double *s)
{
    int kvh = h / (p->Hq / p->Hkv);
    double ks = k_scale_of(p, kvh);
    size_t qoff = (size_t)r * (size_t)p->d;
    for (int t = t0; t < t1; ++t) {
        size_t koff = kv_row(p, block_table, b, t, kvh);
        double dot = 0.0;
        for (int i = 0; i < p->d; ++i)
            dot += elem(q, p->q_dtype, qoff + i) * (ks * elem(k, p->dtype, koff + i));
        s[t - t0] = dot * p->scale;
    }
}

/* The softmax-weighted V over tokens [t0, t1) given their scores, with the
 * scaling constant c: w_t = exp(s_t - c), den = sum w_t, num = sum w_t v_t
 * (sums in token order).  o = num / den (o = 0 when den = 0).  Returns den.
 * The scores in s are overwritten by the weights w_t. */
static double weighted_v(const oracle_problem *p, const void *v, const int32_t *block_table,
                         int b, int h, int t0, int t1, double *s, double c, double *o)
{
    int kvh = h / (p->Hq / p->Hkv);
    double vs = v_scale_of(p, kvh);
    double den = 0.0;
    for (int t = t0; t < t1; ++t) {
        s[t - t0] = exp(s[t - t0] - c);
        den += s[t - t0];
    }
    for (int i = 0; i < p->d; ++i) o[i] = 0.0;
    for (int t = t0; t < t1; ++t) {
        size_t voff = kv_row(p, block_table, b, t, kvh);
        for (int i = 0; i < p->d; ++i) o[i] += s[t - t0] * (vs * elem(v, p->dtype, voff + i));
    }
    for (int i = 0; i < p->d; ++i) o[i] = den > 0.0 ? o[i] / den : 0.0;
    return den;
}

static int row_of(const int32_t *rows, int n_rows, int i) { return rows ? rows[i] : i; }

static int n_rows_total(const oracle_problem *p, const int32_t *rows, int n_rows)
{
    return rows ? n_rows : p->B * p->q_len * p->Hq;
}

/* ---------------------------------------------------------------------- */
/* exact attention, two passes                                             */
/* ---------------------------------------------------------------------- */
/* out[r*d + i], lse[r] for each selected row r = b*Hq + h (rows == NULL: all). */
int oracle_attention(const oracle_problem *p, const void *q, const void *k, const void *v,
                     const int32_t *seq_lens, const int32_t *block_table,
                     const int32_t *rows, int n_rows, int n_threads, double *out, double *lse)
{
    int rc = check_problem(p, seq_lens, block_table);
    if (rc) return rc;
    int total = n_rows_total(p, rows, n_rows);
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
    for (int i = 0; i < total; ++i) {
        int r = row_of(rows, n_rows, i);
        int b, h;
        row_coords(p, r, &b, &h);
        int n = row_tokens(p, seq_lens, r);
        double *o = out + (size_t)r * p->d;
        if (n == 0) {
            for (int j = 0; j < p->d; ++j) o[j] = 0.0;
            lse[r] = -INFINITY;
            continue;
        }
        double *s = (double *)malloc((size_t)n * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        scores(p, q, k, block_table, r, b, h, 0, n, s);
        double m = s[0];                              /* pass 1: the maximum */
        for (int t = 1; t < n; ++t) m = s[t] > m ? s[t] : m;
        double z = weighted_v(p, v, block_table, b, h, 0, n, s, m, o);   /* pass 2 */
        lse[r] = m + log(z);
        free(s);
    }
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* per-split partials                                                      */
/* ---------------------------------------------------------------------- */
/* part_o [rows][S_max][d], part_m / part_l [rows][S_max], indexed by row r.
 * Split s covers tokens [s*split, min((s+1)*split, n)). */
int oracle_split_partials(const oracle_problem *p, const void *q, const void *k, const void *v,
                          const int32_t *seq_lens, const int32_t *block_table, int split, int S_max,
                          const int32_t *rows, int n_rows, int n_threads,
                          double *part_o, double *part_m, double *part_l)
{
    int rc = check_problem(p, seq_lens, block_table);
    if (rc) return rc;
    if (split <= 0 || S_max <= 0) return ORACLE_EINVAL;
    for (int b = 0; b < p->B; ++b) {
        int n = seq_lens ? seq_lens[b] : p->N;
        if ((n + split - 1) / split > S_max) return ORACLE_EINVAL;
    }
    int total = n_rows_total(p, rows, n_rows);
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
    for (int i = 0; i < total; ++i) {
        int r = row_of(rows, n_rows, i);
        int b, h;
        row_coords(p, r, &b, &h);
        int n = row_tokens(p, seq_lens, r);
        double *s = (double *)malloc((size_t)split * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        for (int sp = 0; sp < S_max; ++sp) {
            size_t slot = (size_t)r * S_max + sp;
            double *o = part_o + slot * p->d;
            int t0 = sp * split, t1 = t0 + split < n ? t0 + split : n;
            if (t0 >= t1) {
                part_m[slot] = -INFINITY;
                part_l[slot] = 0.0;
                for (int j = 0; j < p->d; ++j) o[j] = 0.0;
                continue;
            }
            scores(p, q, k, block_table, r, b, h, t0, t1, s);
            double m = s[0];
            for (int t = 1; t < t1 - t0; ++t) m = s[t] > m ? s[t] : m;
            part_m[slot] = m;
            part_l[slot] = weighted_v(p, v, block_table, b, h, t0, t1, s, m, o);
        }
        free(s);
    }
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* merge of partials                                                       */
/* ---------------------------------------------------------------------- */
/* max-rescale form: m = max_s m_s, w_s = l_s exp(m_s - m), l = sum w_s,
 * o = sum w_s O_s / l, lse = m + ln l.  Splits with l_s = 0 are skipped.
 * S splits per row, n_rows rows; a row with no contributing split gives
 * o = 0, lse = -inf. */
int oracle_merge(int n_rows, int S, int d, const double *part_o, const double *part_m,
                 const double *part_l, double *out, double *lse)
{
    if (n_rows < 0 || S <= 0 || d <= 0) return ORACLE_EINVAL;
    for (int r = 0; r < n_rows; ++r) {
        const double *pm = part_m + (size_t)r * S, *pl = part_l + (size_t)r * S;
        double m = -INFINITY;
        for (int s = 0; s < S; ++s)
            if (pl[s] > 0.0 && pm[s] > m) m = pm[s];
        double *o = out + (size_t)r * d;
        for (int i = 0; i < d; ++i) o[i] = 0.0;
        if (m == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double l = 0.0;
        for (int s = 0; s < S; ++s)
            if (pl[s] > 0.0) l += pl[s] * exp(pm[s] - m);
        for (int s = 0; s < S; ++s) {
            if (!(pl[s] > 0.0)) continue;
            double w = pl[s] * exp(pm[s] - m);
            const double *os = part_o + ((size_t)r * S + s) * d;
            for (int i = 0; i < d; ++i) o[i] += w * os[i];
        }
        for (int i = 0; i < d; ++i) o[i] /= l;
        lse[r] = m + log(l);
    }
    return ORACLE_OK;
}

/* log-sum-exp alpha form: L_s = m_s + ln l_s, L = ln sum exp(L_s),
 * alpha_s = exp(L_s - L), o = sum alpha_s O_s.  Same skip rule. */
int oracle_merge_lse(int n_rows, int S, int d, const double *part_o, const double *part_m,
                     const double *part_l, double *out, double *lse)
{
    if (n_rows < 0 || S <= 0 || d <= 0) return ORACLE_EINVAL;
    double *Ls = (double *)malloc((size_t)S * sizeof(double));
    if (!Ls) return ORACLE_ENOMEM;
    for (int r = 0; r < n_rows; ++r) {
        const double *pm = part_m + (size_t)r * S, *pl = part_l + (size_t)r * S;
        double *o = out + (size_t)r * d;
        for (int i = 0; i < d; ++i) o[i] = 0.0;
        double Lmax = -INFINITY;
        for (int s = 0; s < S; ++s) {
            Ls[s] = pl[s] > 0.0 ? pm[s] + log(pl[s]) : -INFINITY;
            if (Ls[s] > Lmax) Lmax = Ls[s];
        }
        if (Lmax == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        /* ln sum exp(L_s), evaluated around the largest L_s so exp stays finite */
        double acc = 0.0;
        for (int s = 0; s < S; ++s)
            if (Ls[s] > -INFINITY) acc += exp(Ls[s] - Lmax);
        double L = Lmax + log(acc);
        for (int s = 0; s < S; ++s) {
            if (Ls[s] == -INFINITY) continue;
            double alpha = exp(Ls[s] - L);
            const double *os = part_o + ((size_t)r * S + s) * d;
            for (int i = 0; i < d; ++i) o[i] += alpha * os[i];
        }
        lse[r] = L;
    }
    free(Ls);
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* FlashAttention tile recurrence over one row of scores                   */
/* ---------------------------------------------------------------------- */
/* For tiles of `tile` scores: m_j = max(m_{j-1}, rowmax(S_j)),
 * P_j = exp(S_j - m_j), l_j = exp(m_{j-1} - m_j) l_{j-1} + rowsum(P_j),
 * O_j = exp(m_{j-1} - m_j) O_{j-1} + P_j V_j; finally o = O_last / l_last.
 * The per-tile state after each tile goes to trace_m[j], trace_l[j] and
 * trace_acc[j*d + i] (O before the final divide); any trace may be NULL.
 * v is [n][d] fp64. */
int oracle_online_tiles(int n, int d, const double *s, const double *v, int tile,
                        double *trace_m, double *trace_l, double *trace_acc, double *out, double *lse)
{
    if (n <= 0 || d <= 0 || tile <= 0) return ORACLE_EINVAL;
    double *acc = (double *)calloc((size_t)d, sizeof(double));
    if (!acc) return ORACLE_ENOMEM;
    double m = -INFINITY, l = 0.0;
    for (int j = 0, t0 = 0; t0 < n; ++j, t0 += tile) {
        int t1 = t0 + tile < n ? t0 + tile : n;
        double tmax = s[t0];
        for (int t = t0 + 1; t < t1; ++t) tmax = s[t] > tmax ? s[t] : tmax;
        double m_new = m > tmax ? m : tmax;
        double corr = m == -INFINITY ? 0.0 : exp(m - m_new);
        double rowsum = 0.0;
        for (int t = t0; t < t1; ++t) rowsum += exp(s[t] - m_new);
        l = corr * l + rowsum;
        for (int i = 0; i < d; ++i) {
            double pv = 0.0;
            for (int t = t0; t < t1; ++t) pv += exp(s[t] - m_new) * v[(size_t)t * d + i];
            acc[i] = corr * acc[i] + pv;
        }
        m = m_new;
        if (trace_m) trace_m[j] = m;
        if (trace_l) trace_l[j] = l;
        if (trace_acc) memcpy(trace_acc + (size_t)j * d, acc, (size_t)d * sizeof(double));
    }
    for (int i = 0; i < d; ++i) out[i] = acc[i] / l;
    *lse = m + log(l);
    free(acc);
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* unified max value with overflow fallback                                */
/* ---------------------------------------------------------------------- */
/* Flag predicate for one score: out of the safe range [lo, hi]. */
int oracle_out_of_range(double s, double lo, double hi) { return s < lo || s > hi; }

/* Per split: if every score lies in [lo, hi], the split's partial uses the
 * unified constant phi: den = sum exp(s - phi), num = sum exp(s - phi) v,
 * m_s = phi, l_s = den, O_s = num / den.  Otherwise the split is flagged and
 * recomputed with its own maximum (the synchronized partial softmax).  The
 * partials are then merged (max-rescale form, which for all-unflagged rows is
 * the single reduction sum num / sum den).  flags [rows][S_max] (uint8),
 * partials as oracle_split_partials, out/lse as oracle_attention; *n_flagged
 * receives the number of flagged (row, split) pairs over the selected rows. */
int oracle_unified_max(const oracle_problem *p, const void *q, const void *k, const void *v,
                       const int32_t *seq_lens, const int32_t *block_table, int split, int S_max,
                       double phi, double lo, double hi,
                       const int32_t *rows, int n_rows, int n_threads,
                       double *part_o, double *part_m, double *part_l, uint8_t *flags,
                       double *out, double *lse, long long *n_flagged, int whole_row)
{
    int rc = check_problem(p, seq_lens, block_table);
    if (rc) return rc;
    if (split <= 0 || S_max <= 0 || !(lo <= hi)) return ORACLE_EINVAL;
    for (int b = 0; b < p->B; ++b) {
        int n = seq_lens ? seq_lens[b] : p->N;
        if ((n + split - 1) / split > S_max) return ORACLE_EINVAL;
    }
    int total = n_rows_total(p, rows, n_rows);
    int failed = 0;
    long long count = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1) reduction(+ : count)
    for (int i = 0; i < total; ++i) {
        int r = row_of(rows, n_rows, i);
        int b, h;
        row_coords(p, r, &b, &h);
        int n = row_tokens(p, seq_lens, r);
        double *s = (double *)malloc((size_t)split * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        /* whole_row: first the range check of every split of the row */
        int row_bad = 0;
        if (whole_row) {
            for (int sp = 0; sp < S_max; ++sp) {
                int t0 = sp * split, t1 = t0 + split < n ? t0 + split : n;
                if (t0 >= t1) continue;
                scores(p, q, k, block_table, r, b, h, t0, t1, s);
                for (int t = 0; t < t1 - t0; ++t) row_bad |= oracle_out_of_range(s[t], lo, hi);
            }
        }
        for (int sp = 0; sp < S_max; ++sp) {
            size_t slot = (size_t)r * S_max + sp;
            double *o = part_o + slot * p->d;
            int t0 = sp * split, t1 = t0 + split < n ? t0 + split : n;
            flags[slot] = 0;
            if (t0 >= t1) {
                part_m[slot] = -INFINITY;
                part_l[slot] = 0.0;
                for (int j = 0; j < p->d; ++j) o[j] = 0.0;
                continue;
            }
            scores(p, q, k, block_table, r, b, h, t0, t1, s);
            int bad = 0;
            for (int t = 0; t < t1 - t0; ++t) bad |= oracle_out_of_range(s[t], lo, hi);
            if (bad) {
                flags[slot] = 1;
                ++count;
            }
            double c = phi;
            if (whole_row ? row_bad : bad) {  /* synchronized recompute: the split's own maximum */
                c = s[0];
                for (int t = 1; t < t1 - t0; ++t) c = s[t] > c ? s[t] : c;
            }
            part_m[slot] = c;
            part_l[slot] = weighted_v(p, v, block_table, b, h, t0, t1, s, c, o);
        }
        free(s);
        oracle_merge(1, S_max, p->d, part_o + (size_t)r * S_max * p->d, part_m + (size_t)r * S_max,
                     part_l + (size_t)r * S_max, out + (size_t)r * p->d, lse + r);
    }
    if (n_flagged) *n_flagged = count;
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}
