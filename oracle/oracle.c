/*
 * oracle.c -- plain, slow, CPU reference for attention with a per-head sink term in the
 * softmax denominator.  TEST INFRASTRUCTURE ONLY: it is built and called by the tests,
 * by the smoke check and by the benchmark's CPU-baseline leg, never by the library.
 * It shares no source with the GPU path.
 *
 * What it computes (plain definition; no tiling, no online softmax, no reordering):
 *
 *   logits     a_ij = scale * sum_d q[i,d] * k[j,d]
 *              ("MiMo-V2-Flash 模型架构深度拆解", CH 3.2 and CH 10.3: scaling = head_dim^-0.5)
 *   max        m_i  = max(max_{j in J(i)} a_ij, sink_h)
 *              ("MiMo-V2-Flash 架构 QA", Q3.7; paper notes §4.3)
 *   weights    s_ij = exp(a_ij - m_i) / (exp(sink_h - m_i) + sum_{j' in J(i)} exp(a_ij' - m_i))
 *              ("MiMo-V2-Flash 架构 QA", Q3.8 formula; paper notes §4.1: the sink sits in
 *              the denominator only and has no value vector)
 *   output     o_i  = sum_{j in J(i)} s_ij * v[j,:]
 *
 *   visible set J(i):  global  -> { j : 0 <= j <= i }                 (causal lower triangle)
 *                      sliding -> { j : max(0, i-W+1) <= j <= i }     (the W most recent keys,
 *                                                                     the query's own included)
 *              (deep-dive CH 10.3 mask description; paper notes §4.3 counts 128 keys for W=128)
 *
 *   GQA: query head h reads KV head h / (Hq/Hkv) (contiguous groups).
 *   The sink is per query head, in the same units as the scaled logits (it is not
 *   multiplied by `scale`).  A NULL sink means no sink term (standard softmax).
 *   sink = +inf: every weight is 0 (the limit of the formula), so the output row is 0.
 *
 * Inputs may be float32 or bfloat16 bit patterns (dtype flag); bf16 -> double is exact.
 * All arithmetic is double precision.  OpenMP parallelises over output rows only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_FP8_E4M3 = 2 };
enum { ORACLE_GLOBAL = 0, ORACLE_SWA = 1 };
enum { ORACLE_RING = 0, ORACLE_PAGED = 1 };

/* OCP 8-bit floating point E4M3 (the "FN" variant: no infinities): sign bit 7, exponent
 * bits 6..3 with bias 7, mantissa bits 2..0; exponent 0 holds the subnormals m * 2^-9; the
 * all-ones exponent with mantissa 7 is NaN, every other code is (1 + m/8) * 2^(e - 7).
 * Largest finite value 448. */
static double e4m3_value(uint8_t code) {
    const int sgn = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double x;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) x = ldexp((double)m, -9);
    else x = ldexp(1.0 + m / 8.0, e - 7);
    return sgn ? -x : x;
}

static double load(const void *p, size_t idx, int dtype) {
    if (dtype == ORACLE_FP8_E4M3) return e4m3_value(((const uint8_t *)p)[idx]);
    if (dtype == ORACLE_BF16) {
        uint32_t u = ((uint32_t)((const uint16_t *)p)[idx]) << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return (double)((const float *)p)[idx];
}

/* The visible keys of one row: n keys of a cache (k, v in kvdtype, element = kscale or
 * vscale times the stored value), key t at kidx[t] in k and vidx[t] in v, then n2 more keys
 * held beside the cache (k2, v2 in the query's dtype, unscaled), key t at kidx2[t], vidx2[t]. */
typedef struct {
    int kvdtype;
    double kscale, vscale;
    const void *k, *v;
    const size_t *kidx, *vidx;
    int n;
    const void *k2, *v2;
    const size_t *kidx2, *vidx2;
    int n2;
} key_list;

static double key_elem(const key_list *kl, int t, int d, int dtype) {
    if (t < kl->n) return kl->kscale * load(kl->k, kl->kidx[t] + d, kl->kvdtype);
    return load(kl->k2, kl->kidx2[t - kl->n] + d, dtype);
}
static double value_elem(const key_list *kl, int t, int e, int dtype) {
    if (t < kl->n) return kl->vscale * load(kl->v, kl->vidx[t] + e, kl->kvdtype);
    return load(kl->v2, kl->vidx2[t - kl->n] + e, dtype);
}

/* One output row.  qrow: index of q[0] of the row; kl: its visible keys.  Writes dv doubles
 * to out and returns the row's log-sum-exp over the sink and the visible logits,
 * log(exp(sink) + sum_j exp(a_j)) (natural log; -inf when both are empty, +inf for a sink of
 * +inf). */
static double attend_row(int dtype, const void *q, size_t qrow, const key_list *kl, int dqk, int dv, double scale,
                         int has_sink, double sink, double *a, double *out) {
    const int n = kl->n + kl->n2;
    for (int e = 0; e < dv; ++e) out[e] = 0.0;
    if (has_sink && isinf(sink) && sink > 0) return INFINITY; /* all mass on the sink */
    double m = has_sink ? sink : -INFINITY;
    for (int t = 0; t < n; ++t) {
        double dot = 0.0;
        for (int d = 0; d < dqk; ++d) dot += load(q, qrow + d, dtype) * key_elem(kl, t, d, dtype);
        a[t] = scale * dot;
        if (a[t] > m) m = a[t];
    }
    if (n == 0 || isinf(m)) return m; /* empty visible set: the sink alone (or nothing) */
    double z = has_sink ? exp(sink - m) : 0.0;
    for (int t = 0; t < n; ++t) z += exp(a[t] - m);
    for (int t = 0; t < n; ++t) {
        double s = exp(a[t] - m) / z;
        for (int e = 0; e < dv; ++e) out[e] += s * value_elem(kl, t, e, dtype);
    }
    return m + log(z);
}

/*
 * Prefill.  q [B][Hq][L][dqk], k [B][Hkv][L][dqk], v [B][Hkv][L][dv], sink [Hq] or NULL.
 * rows == NULL: out [B][Hq][L][dv].  Otherwise rows holds nrows triplets (b, h, i) and
 * out is [nrows][dv].  Returns 0, or -1 on bad arguments.
 */
int oracle_prefill_chunk(int mode, int window, int B, int Lq, int Lk, int Hq, int Hkv, int dqk, int dv,
                         double scale, int dtype, const void *q, const void *k, const void *v,
                         const double *sink, int64_t nrows, const int64_t *rows, double *out, double *lse);

int oracle_prefill(int mode, int window, int B, int L, int Hq, int Hkv, int dqk, int dv,
                   double scale, int dtype, const void *q, const void *k, const void *v,
                   const double *sink, int64_t nrows, const int64_t *rows, double *out) {
    /* every position is a query: the chunk that is the whole sequence */
    return oracle_prefill_chunk(mode, window, B, L, L, Hq, Hkv, dqk, dv, scale, dtype, q, k, v, sink, nrows, rows,
                                out, NULL);
}

/*
 * Chunked prefill over a cached prefix: the rows of the prefill definition at positions
 * Lk - Lq .. Lk - 1 of sequences of Lk tokens (the model card's serving set-up prefills long
 * prompts in chunks).  q [B][Hq][Lq][dqk] (row r is position Lk - Lq + r), k [B][Hkv][Lk][dqk],
 * v [B][Hkv][Lk][dv].  rows == NULL: out [B][Hq][Lq][dv]; else nrows triplets (b, h, r) and
 * out [nrows][dv].  lse (optional, NULL for none): each row's log-sum-exp, [B][Hq][Lq] or
 * [nrows].  Returns 0, or -1 on bad arguments.
 */
int oracle_prefill_chunk(int mode, int window, int B, int Lq, int Lk, int Hq, int Hkv, int dqk, int dv,
                         double scale, int dtype, const void *q, const void *k, const void *v,
                         const double *sink, int64_t nrows, const int64_t *rows, double *out, double *lse) {
    if (B < 0 || Lq < 0 || Lk < Lq || Hq <= 0 || Hkv <= 0 || Hq % Hkv || dqk <= 0 || dv <= 0) return -1;
    if (mode == ORACLE_SWA && window <= 0) return -1;
    if (mode != ORACLE_SWA && mode != ORACLE_GLOBAL) return -1;
    const int G = Hq / Hkv;
    const int64_t total = rows ? nrows : (int64_t)B * Hq * Lq;
#pragma omp parallel
    {
        double *a = (double *)malloc(sizeof(double) * (size_t)(Lk > 0 ? Lk : 1));
        size_t *ki = (size_t *)malloc(sizeof(size_t) * (size_t)(Lk > 0 ? Lk : 1));
        size_t *vi = (size_t *)malloc(sizeof(size_t) * (size_t)(Lk > 0 ? Lk : 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t n = 0; n < total; ++n) {
            int64_t b, h, r;
            if (rows) {
                b = rows[3 * n];
                h = rows[3 * n + 1];
                r = rows[3 * n + 2];
            } else {
                b = n / ((int64_t)Hq * Lq);
                h = (n / Lq) % Hq;
                r = n % Lq;
            }
            const int64_t i = (int64_t)Lk - Lq + r; /* position of this query */
            const int64_t g = h / G;
            const int64_t jlo = (mode == ORACLE_SWA) ? (i - window + 1 > 0 ? i - window + 1 : 0) : 0;
            int cnt = 0;
            for (int64_t j = jlo; j <= i; ++j, ++cnt) {
                ki[cnt] = (size_t)(((b * Hkv + g) * Lk + j) * dqk);
                vi[cnt] = (size_t)(((b * Hkv + g) * Lk + j) * dv);
            }
            const key_list kl = {dtype, 1.0, 1.0, k, v, ki, vi, cnt, NULL, NULL, NULL, NULL, 0};
            const double l = attend_row(dtype, q, (size_t)(((b * Hq + h) * Lq + r) * dqk), &kl, dqk, dv, scale,
                                        sink != NULL, sink ? sink[h] : 0.0, a, out + (size_t)n * dv);
            if (lse) lse[n] = l;
        }
        free(a);
        free(ki);
        free(vi);
    }
    return 0;
}

/*
 * Decode: q_len new queries per sequence at positions n_b - q_len .. n_b - 1, where
 * n_b = seq_lens[b] counts the new tokens.  q_len = 1 is ordinary one-token decoding;
 * q_len > 1 is the parallel verification of drafted tokens ("MiMo-V2-Flash 模型架构深度拆解",
 * CH 4.4; paper notes §6.4): each new token is a causal query that sees the keys up to and
 * including its own position, so the result equals the last q_len rows of a prefill over the
 * whole sequence.  A position below 0 (n_b < q_len) has an empty visible set: its output row
 * is 0.  q [B][Hq][q_len][dqk]; sink [Hq] or NULL; out [B][Hq][q_len][dv].
 * Where the new tokens' keys and values are:
 *   k_new == NULL: already in the cache, at their positions;
 *   k_new != NULL: beside the cache, k_new [B][Hkv][q_len][dqk], v_new [B][Hkv][q_len][dv]
 *                  (token t = position n_b - q_len + t), in the query's dtype; the cache
 *                  holds the positions before n_b - q_len only (drafts whose acceptance is
 *                  not known yet must not overwrite a ring's committed keys).
 * The cache:
 * RING  (sliding mode): k [B][Hkv][window][dqk], v [B][Hkv][window][dv]; position p lives in
 *       slot p mod window.  Without k_new only q_len = 1 (the earlier queries of several
 *       would need keys the ring has already overwritten).
 * PAGED (either mode): k [num_pages][Hkv][page_size][dqk], v [num_pages][Hkv][page_size][dv];
 *       position p of sequence b lives in page block_table[b*max_pages + p/page_size] at
 *       offset p mod page_size.
 * Returns 0, or -1 on bad arguments (including a page id outside the pool).
 */
static int decode_impl(int mode, int window, int layout, int B, int Hq, int Hkv, int dqk, int dv,
                       int q_len, double scale, int dtype, const void *q, int kvdtype, double kscale,
                       double vscale, const void *k, const void *v, const int32_t *block_table,
                       int page_size, int max_pages, int num_pages, const int32_t *seq_lens,
                       const void *k_new, const void *v_new, const double *sink, double *out, double *lse) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || dqk <= 0 || dv <= 0) return -1;
    if (mode == ORACLE_SWA && window <= 0) return -1;
    if (q_len <= 0) return -1;
    if (layout == ORACLE_RING && (mode != ORACLE_SWA || (q_len != 1 && !k_new))) return -1;
    if (layout == ORACLE_PAGED && (!block_table || page_size <= 0 || max_pages < 0)) return -1;
    if (!k_new != !v_new) return -1;
    const int G = Hq / Hkv;
    int bad = 0;
    int64_t maxn = 1;
    for (int b = 0; b < B; ++b) {
        const int64_t cached = k_new ? (int64_t)seq_lens[b] - q_len : seq_lens[b];
        if (layout == ORACLE_PAGED && cached > (int64_t)max_pages * page_size) bad = 1;
        if (seq_lens[b] > maxn) maxn = seq_lens[b];
    }
    if (bad) return -1;
#pragma omp parallel
    {
        double *a = (double *)malloc(sizeof(double) * (size_t)maxn);
        size_t *ki = (size_t *)malloc(sizeof(size_t) * (size_t)maxn);
        size_t *vi = (size_t *)malloc(sizeof(size_t) * (size_t)maxn);
        size_t *ki2 = (size_t *)malloc(sizeof(size_t) * (size_t)q_len);
        size_t *vi2 = (size_t *)malloc(sizeof(size_t) * (size_t)q_len);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < (int64_t)B * Hq * q_len; ++r) {
            const int64_t b = r / ((int64_t)Hq * q_len), h = (r / q_len) % Hq, g = h / G;
            const int64_t nb = seq_lens[b];
            const int64_t i = nb - q_len + r % q_len; /* this query's position */
            const int64_t nc = k_new ? nb - q_len : nb; /* positions below nc are in the cache */
            const int64_t jlo = (mode == ORACLE_SWA) ? (i - window + 1 > 0 ? i - window + 1 : 0) : 0;
            int n = 0, n2 = 0;
            int local_bad = 0;
            for (int64_t j = jlo; j <= i; ++j) {
                if (j >= nc) { /* a new token beside the cache */
                    const int64_t t = j - nc;
                    ki2[n2] = (size_t)(((b * Hkv + g) * q_len + t) * dqk);
                    vi2[n2] = (size_t)(((b * Hkv + g) * q_len + t) * dv);
                    ++n2;
                } else if (layout == ORACLE_RING) {
                    const int64_t slot = j % window;
                    ki[n] = (size_t)(((b * Hkv + g) * window + slot) * dqk);
                    vi[n] = (size_t)(((b * Hkv + g) * window + slot) * dv);
                    ++n;
                } else {
                    const int64_t page = block_table[b * max_pages + j / page_size];
                    if (page < 0 || page >= num_pages) local_bad = 1;
                    const int64_t off = j % page_size;
                    ki[n] = (size_t)(((page * Hkv + g) * page_size + off) * dqk);
                    vi[n] = (size_t)(((page * Hkv + g) * page_size + off) * dv);
                    ++n;
                }
            }
            if (local_bad) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            const key_list kl = {kvdtype, kscale, vscale, k, v, ki, vi, n, k_new, v_new, ki2, vi2, n2};
            const double l = attend_row(dtype, q, (size_t)r * dqk, &kl, dqk, dv, scale, sink != NULL,
                                        sink ? sink[h] : 0.0, a, out + (size_t)r * dv);
            if (lse) lse[r] = l;
        }
        free(a);
        free(ki);
        free(vi);
        free(ki2);
        free(vi2);
    }
    return bad ? -1 : 0;
}

int oracle_decode(int mode, int window, int layout, int B, int Hq, int Hkv, int dqk, int dv,
                  int q_len, double scale, int dtype, const void *q, const void *k, const void *v,
                  const int32_t *block_table, int page_size, int max_pages, int num_pages,
                  const int32_t *seq_lens, const double *sink, double *out, double *lse) {
    return decode_impl(mode, window, layout, B, Hq, Hkv, dqk, dv, q_len, scale, dtype, q, dtype, 1.0, 1.0, k, v,
                       block_table, page_size, max_pages, num_pages, seq_lens, NULL, NULL, sink, out, lse);
}

/* Decode with the q_len new tokens' keys and values beside the cache (k_new, v_new, in the
 * cache's dtype; see decode_impl).  This is also chunked prefill over a cached prefix (the
 * model card's serving set-up prefills long prompts in chunks): the chunk's q_len tokens are
 * the new ones, their keys and values given contiguously, the prefix read through the page
 * table (or, in sliding mode, from a ring holding its last `window` positions). */
int oracle_decode_side(int mode, int window, int layout, int B, int Hq, int Hkv, int dqk, int dv,
                       int q_len, double scale, int dtype, const void *q, const void *k, const void *v,
                       const int32_t *block_table, int page_size, int max_pages, int num_pages,
                       const int32_t *seq_lens, const void *k_new, const void *v_new, const double *sink,
                       double *out, double *lse) {
    if (!k_new || !v_new) return -1;
    return decode_impl(mode, window, layout, B, Hq, Hkv, dqk, dv, q_len, scale, dtype, q, dtype, 1.0, 1.0, k, v,
                       block_table, page_size, max_pages, num_pages, seq_lens, k_new, v_new, sink, out, lse);
}

/*
 * Decode from a KV cache held in 8-bit floating point (the pages size the cache with one
 * byte per element: paper notes §3.2): k and v hold E4M3 codes, element values are
 * kscale * e4m3(code) and vscale * e4m3(code).  Everything else as oracle_decode (q in
 * `dtype`).  kscale, vscale > 0.
 */
int oracle_decode_fp8(int mode, int window, int layout, int B, int Hq, int Hkv, int dqk, int dv,
                      int q_len, double scale, int dtype, const void *q, const void *k, const void *v,
                      double kscale, double vscale, const int32_t *block_table, int page_size,
                      int max_pages, int num_pages, const int32_t *seq_lens, const double *sink,
                      double *out, double *lse) {
    if (!(kscale > 0) || !(vscale > 0)) return -1;
    return decode_impl(mode, window, layout, B, Hq, Hkv, dqk, dv, q_len, scale, dtype, q, ORACLE_FP8_E4M3, kscale,
                       vscale, k, v, block_table, page_size, max_pages, num_pages, seq_lens, NULL, NULL, sink, out,
                       lse);
}

/*
 * Backward of prefill attention with a sink (the sink is a learnable per-head scalar: deep-dive
 * CH 10.1 declares it a parameter; its gradient is below).  For each row i of head h, with the
 * forward weights P_ij = exp(a_ij - LSE_i) over the visible keys and P_i,sink = exp(sink_h -
 * LSE_i) (the sink has no value vector), and dO_i the gradient of the output row:
 *   dP_ij = dO_i . v_j          D_i = sum_j P_ij dP_ij          dS_ij = P_ij (dP_ij - D_i)
 *   dq_i  = scale sum_j dS_ij k_j      dk_j += scale dS_ij q_i      dv_j += P_ij dO_i
 *   dsink_h += dL/dsink through P_i,sink only = -P_i,sink D_i  (the sink enters the outputs
 *   only through the shared denominator).
 * A NULL sink has no gradient (dsink untouched).  q, k, v, dout in `dtype`; outputs doubles:
 * dq [B][Hq][L][dqk], dk [B][Hkv][L][dqk], dv [B][Hkv][L][dv] (overwritten), dsink [Hq]
 * (overwritten when sink is given).  Returns 0, or -1 on bad arguments.
 */
/* dS_ij = P_ij (dP_ij - D_i): the gradient of the loss with respect to the logit a_ij. */
static double score_grad(double p, double dp, double D) { return p * (dp - D); }

/* The quantities of one row (b, h, i) that every gradient above is built from: the visible
 * keys jlo .. jlo + n - 1, their weights pr[t] = P_i,jlo+t and dP values dp[t], D_i and the
 * sink's weight.  Returns 0 when the row has no gradient (a sink of +inf makes every weight 0). */
static int backward_row(int mode, int window, int L, int Hq, int Hkv, int dqk, int dv, double scale, int dtype,
                        const void *q, const void *k, const void *v, const double *sink, const void *dout,
                        int64_t b, int64_t h, int64_t i, double *a, double *pr, double *dp, int64_t *jlo_out,
                        int *n_out, double *D_out, double *psink_out) {
    const int64_t g = h / (Hq / Hkv);
    const size_t kvbase = (size_t)(b * Hkv + g) * L;
    const size_t qrow = (size_t)((b * Hq + h) * L + i);
    const int has_sink = sink != NULL;
    const double sk = has_sink ? sink[h] : 0.0;
    if (has_sink && isinf(sk) && sk > 0) return 0; /* every weight is 0 */
    const int64_t jlo = (mode == ORACLE_SWA) ? (i - window + 1 > 0 ? i - window + 1 : 0) : 0;
    const int n = (int)(i - jlo + 1);
    /* forward weights of this row */
    double m = has_sink ? sk : -INFINITY;
    for (int t = 0; t < n; ++t) {
        const size_t krow = (kvbase + (size_t)(jlo + t)) * dqk;
        double dot = 0.0;
        for (int d = 0; d < dqk; ++d) dot += load(q, qrow * dqk + d, dtype) * load(k, krow + d, dtype);
        a[t] = scale * dot;
        if (a[t] > m) m = a[t];
    }
    double z = has_sink ? exp(sk - m) : 0.0;
    for (int t = 0; t < n; ++t) z += exp(a[t] - m);
    for (int t = 0; t < n; ++t) pr[t] = exp(a[t] - m) / z;
    /* dP, D */
    double Dsum = 0.0;
    for (int t = 0; t < n; ++t) {
        const size_t vrow = (kvbase + (size_t)(jlo + t)) * dv;
        double dot = 0.0;
        for (int e = 0; e < dv; ++e) dot += load(dout, qrow * dv + e, dtype) * load(v, vrow + e, dtype);
        dp[t] = dot;
        Dsum += pr[t] * dot;
    }
    *jlo_out = jlo;
    *n_out = n;
    *D_out = Dsum;
    *psink_out = has_sink ? exp(sk - m) / z : 0.0;
    return 1;
}

int oracle_prefill_backward(int mode, int window, int B, int L, int Hq, int Hkv, int dqk, int dv, double scale,
                            int dtype, const void *q, const void *k, const void *v, const double *sink,
                            const void *dout, double *dq, double *dk, double *dvo, double *dsink) {
    if (B < 0 || L < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || dqk <= 0 || dv <= 0) return -1;
    if (mode == ORACLE_SWA && window <= 0) return -1;
    if (mode != ORACLE_SWA && mode != ORACLE_GLOBAL) return -1;
    const int G = Hq / Hkv;
    double *dsink_part = (double *)calloc((size_t)(B > 0 ? B : 1) * Hq, sizeof(double));
    if (!dsink_part) return -1;
    /* one (sequence, KV head) per thread: it owns the dk and dv rows of that KV head */
#pragma omp parallel
    {
        double *a = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        double *pr = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        double *dp = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t bg = 0; bg < (int64_t)B * Hkv; ++bg) {
            const int64_t b = bg / Hkv, g = bg % Hkv;
            const size_t kvbase = (size_t)(b * Hkv + g) * L;
            for (size_t e = 0; e < (size_t)L * dqk; ++e) dk[kvbase * dqk + e] = 0.0;
            for (size_t e = 0; e < (size_t)L * dv; ++e) dvo[kvbase * dv + e] = 0.0;
            for (int64_t h = g * G; h < (g + 1) * G; ++h) {
                for (int64_t i = 0; i < L; ++i) {
                    const size_t qrow = (size_t)((b * Hq + h) * L + i);
                    double *dqi = dq + qrow * dqk;
                    for (int d = 0; d < dqk; ++d) dqi[d] = 0.0;
                    int64_t jlo;
                    int n;
                    double Dsum, psink;
                    if (!backward_row(mode, window, L, Hq, Hkv, dqk, dv, scale, dtype, q, k, v, sink, dout, b, h, i, a,
                                      pr, dp, &jlo, &n, &Dsum, &psink))
                        continue;
                    if (sink) dsink_part[b * Hq + h] += -psink * Dsum;
                    for (int t = 0; t < n; ++t) {
                        const double ds = score_grad(pr[t], dp[t], Dsum);
                        const size_t j = kvbase + (size_t)(jlo + t);
                        for (int d = 0; d < dqk; ++d) {
                            dqi[d] += scale * ds * load(k, j * dqk + d, dtype);
                            dk[j * dqk + d] += scale * ds * load(q, qrow * dqk + d, dtype);
                        }
                        for (int e = 0; e < dv; ++e) dvo[j * dv + e] += pr[t] * load(dout, qrow * dv + e, dtype);
                    }
                }
            }
        }
        free(a);
        free(pr);
        free(dp);
    }
    if (sink)
        for (int h = 0; h < Hq; ++h) {
            double acc = 0.0;
            for (int b = 0; b < B; ++b) acc += dsink_part[b * Hq + h];
            dsink[h] = acc;
        }
    free(dsink_part);
    return 0;
}

/*
 * Sampled gradients, the same definitions as oracle_prefill_backward for a few entries of a
 * large problem: dq of the rows qrows[r] = (b, h, i), r < nq, into dq_out [nq][dqk]; dk and dv
 * of the keys krows[r] = (b, KV head g, j), r < nk, into dk_out [nk][dqk] and dv_out [nk][dv]
 * (the sums over every row of every head of the group that sees key j).  Returns 0, or -1 on
 * bad arguments.
 */
int oracle_prefill_backward_sampled(int mode, int window, int B, int L, int Hq, int Hkv, int dqk, int dv,
                                    double scale, int dtype, const void *q, const void *k, const void *v,
                                    const double *sink, const void *dout, int nq, const int64_t *qrows,
                                    double *dq_out, int nk, const int64_t *krows, double *dk_out, double *dv_out) {
    if (B < 0 || L < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || dqk <= 0 || dv <= 0 || nq < 0 || nk < 0) return -1;
    if (mode == ORACLE_SWA && window <= 0) return -1;
    if (mode != ORACLE_SWA && mode != ORACLE_GLOBAL) return -1;
    const int G = Hq / Hkv;
    for (int r = 0; r < nq; ++r)
        if (qrows[3 * r] < 0 || qrows[3 * r] >= B || qrows[3 * r + 1] < 0 || qrows[3 * r + 1] >= Hq ||
            qrows[3 * r + 2] < 0 || qrows[3 * r + 2] >= L)
            return -1;
    for (int r = 0; r < nk; ++r)
        if (krows[3 * r] < 0 || krows[3 * r] >= B || krows[3 * r + 1] < 0 || krows[3 * r + 1] >= Hkv ||
            krows[3 * r + 2] < 0 || krows[3 * r + 2] >= L)
            return -1;
    /* per (key, head of its group) partial sums, added in head order afterwards */
    double *part = (double *)calloc((size_t)(nk > 0 ? nk : 1) * G * (dqk + dv), sizeof(double));
    if (!part) return -1;
#pragma omp parallel
    {
        double *a = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        double *pr = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        double *dp = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < nq; ++r) {
            const int64_t b = qrows[3 * r], h = qrows[3 * r + 1], i = qrows[3 * r + 2];
            const size_t kvbase = (size_t)(b * Hkv + h / G) * L;
            double *dqi = dq_out + (size_t)r * dqk;
            for (int d = 0; d < dqk; ++d) dqi[d] = 0.0;
            int64_t jlo;
            int n;
            double Dsum, psink;
            if (!backward_row(mode, window, L, Hq, Hkv, dqk, dv, scale, dtype, q, k, v, sink, dout, b, h, i, a, pr, dp,
                              &jlo, &n, &Dsum, &psink))
                continue;
            for (int t = 0; t < n; ++t) {
                const double ds = score_grad(pr[t], dp[t], Dsum);
                const size_t j = kvbase + (size_t)(jlo + t);
                for (int d = 0; d < dqk; ++d) dqi[d] += scale * ds * load(k, j * dqk + d, dtype);
            }
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t rh = 0; rh < (int64_t)nk * G; ++rh) {
            const int r = (int)(rh / G);
            const int64_t b = krows[3 * r], g = krows[3 * r + 1], j = krows[3 * r + 2];
            const int64_t h = g * G + rh % G;
            double *pk = part + (size_t)rh * (dqk + dv), *pv = pk + dqk;
            /* the rows that see key j: i >= j, and i < j + W in sliding-window mode */
            const int64_t ihi = (mode == ORACLE_SWA && j + window - 1 < L - 1) ? j + window - 1 : L - 1;
            for (int64_t i = j; i <= ihi; ++i) {
                int64_t jlo;
                int n;
                double Dsum, psink;
                if (!backward_row(mode, window, L, Hq, Hkv, dqk, dv, scale, dtype, q, k, v, sink, dout, b, h, i, a, pr,
                                  dp, &jlo, &n, &Dsum, &psink))
                    continue;
                const int t = (int)(j - jlo);
                const double ds = score_grad(pr[t], dp[t], Dsum);
                const size_t qrow = (size_t)((b * Hq + h) * L + i);
                for (int d = 0; d < dqk; ++d) pk[d] += scale * ds * load(q, qrow * dqk + d, dtype);
                for (int e = 0; e < dv; ++e) pv[e] += pr[t] * load(dout, qrow * dv + e, dtype);
            }
        }
        free(a);
        free(pr);
        free(dp);
    }
    for (int r = 0; r < nk; ++r) {
        for (int d = 0; d < dqk; ++d) dk_out[(size_t)r * dqk + d] = 0.0;
        for (int e = 0; e < dv; ++e) dv_out[(size_t)r * dv + e] = 0.0;
        for (int hh = 0; hh < G; ++hh) {
            const double *pk = part + ((size_t)r * G + hh) * (dqk + dv);
            for (int d = 0; d < dqk; ++d) dk_out[(size_t)r * dqk + d] += pk[d];
            for (int e = 0; e < dv; ++e) dv_out[(size_t)r * dv + e] += pk[dqk + e];
        }
    }
    free(part);
    return 0;
}

/*
 * Partial rotary position embedding ("MiMo-V2-Flash 模型架构深度拆解", CH 3.5 and CH 10.5;
 * "MiMo-V2-Flash 架构 QA", Q2.7): only the first `rot` of the `dim` q/k dimensions are
 * rotated (64 of 192); pair i (i < rot/2) turns by the angle pos * theta^(-2i/rot), theta
 * 10 000 in sliding-window layers and 5 000 000 in global ones.  Pair i is made of
 * dimensions i and i + rot/2 (the rotate-half pairing).  x [rows][dim] in `dtype`, pos
 * [rows]; out [rows][dim] doubles.  Returns 0, or -1 on bad arguments.
 */
int oracle_rope(int64_t rows, int dim, int rot, double theta, int dtype, const void *x, const int64_t *pos,
                double *out) {
    if (rows < 0 || dim <= 0 || rot < 0 || rot > dim || rot % 2 || !(theta > 0)) return -1;
    const int half = rot / 2;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const size_t base = (size_t)r * dim;
        for (int d = rot; d < dim; ++d) out[base + d] = load(x, base + d, dtype);
        for (int i = 0; i < half; ++i) {
            const double ang = (double)pos[r] * pow(theta, -2.0 * i / rot);
            const double c = cos(ang), sn = sin(ang);
            const double a = load(x, base + i, dtype), b = load(x, base + i + half, dtype);
            out[base + i] = a * c - b * sn;
            out[base + i + half] = b * c + a * sn;
        }
    }
    return 0;
}

/* The value of one E4M3 code (exported for the tests). */
double oracle_e4m3_value(int code) { return e4m3_value((uint8_t)code); }

/*
 * Writing an 8-bit cache: the E4M3 code of x / scale.  The quotient is formed in float32
 * (as a float32 kernel forms it), clamped to the largest finite magnitude 448, and rounded
 * to the nearest value the format holds, ties to the even code (the one whose last mantissa
 * bit is 0).  The sign is kept, so a negative quotient that rounds to zero gives -0 (0x80).
 * NaN gives 0x7F.  The pages size the cache at one byte per element (paper notes §3.2) and
 * state no format; this is the E4M3 reading with one scale per tensor.
 */
static uint8_t e4m3_encode(double x, double scale) {
    const float y = (float)x / (float)scale;
    if (isnan(y)) return 0x7F;
    const int neg = signbit(y) ? 1 : 0;
    double a = fabs((double)y);
    if (a > 448.0) a = 448.0;
    /* spacing of the representable values around a: 2^-9 below the smallest normal 2^-6,
     * else 2^(floor(log2 a) - 3) (three mantissa bits per binade) */
    double step = ldexp(1.0, -9);
    if (a >= ldexp(1.0, -6)) {
        int e;
        frexp(a, &e); /* a = f * 2^e, f in [0.5, 1): floor(log2 a) = e - 1 */
        step = ldexp(1.0, e - 1 - 3);
    }
    const double n = a / step; /* exact: step is a power of two */
    double r = floor(n);
    const double frac = n - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    const double val = r * step;
    /* the non-negative code holding that value, found by comparing against every code */
    for (int c = 0; c < 0x7F; ++c)
        if (e4m3_value((uint8_t)c) == val) return (uint8_t)(c | (neg << 7));
    return 0x7F; /* not reached: every rounded value in [0, 448] is a code */
}

/* Codes of x[0..n) / scale (float32 inputs) into out[0..n).  Returns 0, or -1 when scale is
 * not a positive finite number. */
int oracle_e4m3_encode(int64_t n, const float *x, double scale, uint8_t *out) {
    if (n < 0 || !(scale > 0.0) || isinf(scale)) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode((double)x[i], scale);
    return 0;
}

/* Number of OpenMP threads a parallel region would use (reported next to timings). */
int oracle_threads(void) {
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
