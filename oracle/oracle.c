/*
 * CPU oracle for the context-sparse decode step.  TEST INFRASTRUCTURE ONLY:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg use it;
 * the GPU library never links, loads or calls it, and it shares no code with
 * the GPU library (it walks the page table and decodes bf16 on its own).
 *
 * What it computes, all in fp64, plainly and slowly:
 *
 *  scores   s[b,h,j] = sum_{d<128} q[b,h,d] * K[b, h/G, j, d]  for every cached
 *           token j < N_b.  The raw query-key product: the numerator of scaled
 *           dot-product attention, softmax(q K^T / sqrt(d_k)) V (sparse-attention
 *           survey page, section 1.1).  Products of two bf16 values are exact in
 *           fp64; d is summed in ascending order.  Query head h reads key/value
 *           head floor(h / G), G = Hq / Hkv (contiguous GQA groups).
 *
 *  top-k    The exact "oracle top-k" indexer of the context-sparsity paper
 *           (German summary, section 2, sparsity mechanisms: exact selection
 *           of the top-k tokens): for each (b, h), k' = min(k_b, N_b) tokens,
 *           ordered by score descending and, on equal scores, by lower token
 *           index first.  Written out ascending by token index, padded with -1.
 *
 *  attend   Softmax attention over a given index set I (the sparse decode mode
 *           of the paper's Fig. 1a reads only the selected rows): with the scale
 *           c (1/sqrt(128) by default), l_j = c * s_j, m = max_I l_j,
 *           w_j = exp(l_j - m), o = sum_I w_j V_j / sum_I w_j.  This is the
 *           attention output o = V^T a with a a distribution over the tokens
 *           (paper section 2.1, Theorem 1), restricted to I and renormalised.
 *
 *  dense    The same with I = {0, ..., N_b - 1} (the dense decode mode of
 *           Fig. 1a, which reads the whole cache).
 *
 * Layouts: q [B][Hq][128] bf16 bits; caches [pages][Hkv][16][128] bf16 bits;
 * page_table [B][max_pages] int32; seq_lens, k_per_seq [B] int32.
 * Work is spread over (b, h) with OpenMP; nothing else is reordered.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_D 128
#define ORC_PAGE 16

typedef struct {
    const uint16_t *k, *v;      /* bf16 bit patterns */
    const int32_t *page_table;
    const int32_t *seq_lens;
    int32_t batch, num_kv_heads, max_pages;
} orc_cache;

static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;  /* bf16 is the top half of an fp32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Address of token j's row for kv head g of sequence b. */
static const uint16_t *row_of(const uint16_t *cache, const orc_cache *c, int b, int g, int64_t j)
{
    int64_t page = c->page_table[(int64_t)b * c->max_pages + j / ORC_PAGE];
    int64_t slot = j % ORC_PAGE;
    return cache + ((page * c->num_kv_heads + g) * ORC_PAGE + slot) * ORC_D;
}

static double dot_q_k(const uint16_t *qrow, const uint16_t *krow)
{
    double s = 0.0;
    for (int d = 0; d < ORC_D; ++d)
        s += bf16_value(qrow[d]) * bf16_value(krow[d]);
    return s;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* scores_out: [B][Hq][n_stride] fp64; entries j >= N_b are left untouched. */
void oracle_scores(const uint16_t *k_cache, const int32_t *page_table, const int32_t *seq_lens,
                   int32_t batch, int32_t num_kv_heads, int32_t max_pages, const uint16_t *q,
                   int32_t num_q_heads, int64_t n_stride, double *scores_out)
{
    orc_cache c = {k_cache, 0, page_table, seq_lens, batch, num_kv_heads, max_pages};
    int32_t G = num_q_heads / num_kv_heads;
    int64_t pairs = (int64_t)batch * num_q_heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < pairs; ++bh) {
        int b = (int)(bh / num_q_heads), h = (int)(bh % num_q_heads), g = h / G;
        const uint16_t *qrow = q + bh * ORC_D;
        double *out = scores_out + bh * n_stride;
        for (int64_t j = 0; j < seq_lens[b]; ++j)
            out[j] = dot_q_k(qrow, row_of(k_cache, &c, b, g, j));
    }
}

/* Ordering used by the selection: higher score first, then lower index. */
typedef struct { double s; int64_t j; } scored_token;

static int by_score_then_index(const void *pa, const void *pb)
{
    const scored_token *a = (const scored_token *)pa, *b = (const scored_token *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->j > b->j) - (a->j < b->j);
}

static int by_index(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/*
 * Exact top-k from precomputed scores [B][Hq][n_stride].
 * idx_out [B][Hq][k_max]: the k' = min(k_b, N_b, k_max) selected token indices,
 * ascending, then -1.  kth_out [B][Hq] (may be NULL): the k'-th largest score
 * (the selection threshold s_(k')).
 */
void oracle_topk(const double *scores, const int32_t *seq_lens, const int32_t *k_per_seq,
                 int32_t batch, int32_t num_q_heads, int64_t n_stride, int32_t k_max,
                 int32_t *idx_out, double *kth_out)
{
    int64_t pairs = (int64_t)batch * num_q_heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < pairs; ++bh) {
        int b = (int)(bh / num_q_heads);
        int64_t n = seq_lens[b];
        int64_t kk = k_per_seq[b];
        if (kk > n) kk = n;
        if (kk > k_max) kk = k_max;
        if (kk < 0) kk = 0;
        scored_token *all = (scored_token *)malloc((size_t)(n > 0 ? n : 1) * sizeof *all);
        for (int64_t j = 0; j < n; ++j) {
            all[j].s = scores[bh * n_stride + j];
            all[j].j = j;
        }
        qsort(all, (size_t)n, sizeof *all, by_score_then_index);
        int32_t *row = idx_out + bh * k_max;
        for (int64_t i = 0; i < kk; ++i)
            row[i] = (int32_t)all[i].j;
        qsort(row, (size_t)kk, sizeof *row, by_index);
        for (int64_t i = kk; i < k_max; ++i)
            row[i] = -1;
        if (kth_out)
            kth_out[bh] = kk > 0 ? all[kk - 1].s : -INFINITY;
        free(all);
    }
}

/* Softmax attention of one (b, h) over the listed tokens; n_sel entries of sel
 * (entries < 0 are skipped).  out: 128 fp64.  With no tokens the output is 0. */
static void attend_one(const orc_cache *c, int b, int g, const uint16_t *qrow, const int32_t *sel,
                       int64_t n_sel, double scale, double *out)
{
    double m = -INFINITY;
    for (int64_t i = 0; i < n_sel; ++i) {
        if (sel[i] < 0) continue;
        double l = scale * dot_q_k(qrow, row_of(c->k, c, b, g, sel[i]));
        if (l > m) m = l;
    }
    double z = 0.0, acc[ORC_D];
    for (int d = 0; d < ORC_D; ++d) acc[d] = 0.0;
    for (int64_t i = 0; i < n_sel; ++i) {
        if (sel[i] < 0) continue;
        double w = exp(scale * dot_q_k(qrow, row_of(c->k, c, b, g, sel[i])) - m);
        const uint16_t *vrow = row_of(c->v, c, b, g, sel[i]);
        z += w;
        for (int d = 0; d < ORC_D; ++d)
            acc[d] += w * bf16_value(vrow[d]);
    }
    for (int d = 0; d < ORC_D; ++d)
        out[d] = z > 0.0 ? acc[d] / z : 0.0;
}

/* Sparse attention over idx [B][Hq][k_max] (-1 = unused); out [B][Hq][128] fp64. */
void oracle_attend(const uint16_t *k_cache, const uint16_t *v_cache, const int32_t *page_table,
                   const int32_t *seq_lens, int32_t batch, int32_t num_kv_heads, int32_t max_pages,
                   const uint16_t *q, int32_t num_q_heads, const int32_t *idx, int32_t k_max,
                   double scale, double *out)
{
    orc_cache c = {k_cache, v_cache, page_table, seq_lens, batch, num_kv_heads, max_pages};
    int32_t G = num_q_heads / num_kv_heads;
    int64_t pairs = (int64_t)batch * num_q_heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < pairs; ++bh) {
        int b = (int)(bh / num_q_heads), h = (int)(bh % num_q_heads);
        attend_one(&c, b, h / G, q + bh * ORC_D, idx + bh * k_max, k_max, scale, out + bh * ORC_D);
    }
}

/* Dense attention over every cached token; out [B][Hq][128] fp64. */
void oracle_dense(const uint16_t *k_cache, const uint16_t *v_cache, const int32_t *page_table,
                  const int32_t *seq_lens, int32_t batch, int32_t num_kv_heads, int32_t max_pages,
                  const uint16_t *q, int32_t num_q_heads, double scale, double *out)
{
    orc_cache c = {k_cache, v_cache, page_table, seq_lens, batch, num_kv_heads, max_pages};
    int32_t G = num_q_heads / num_kv_heads;
    int64_t pairs = (int64_t)batch * num_q_heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < pairs; ++bh) {
        int b = (int)(bh / num_q_heads), h = (int)(bh % num_q_heads);
        int64_t n = seq_lens[b];
        int32_t *all = (int32_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof *all);
        for (int64_t j = 0; j < n; ++j) all[j] = (int32_t)j;
        attend_one(&c, b, h / G, q + bh * ORC_D, all, n, scale, out + bh * ORC_D);
        free(all);
    }
}

/*
 * Quest-style page selection (the Sparse Frontier review: section 3.5, Table 1 --
 * Quest works at decode time on pages with a uniform budget over a full cache;
 * section 7.1 -- 16-token pages, each represented by the minimum and maximum of
 * its keys, the most relevant pages chosen at every step, the page holding the
 * current token always included; Eq. 10 -- the page representations are what the
 * selection loads).
 *
 *  quest_summaries  for every logical page p < ceil(N_b / 16) of sequence b and kv
 *                   head g: kmin_d and kmax_d over the page's cached rows (tokens
 *                   j < N_b only).  out [B][max_pages][Hkv][2][128] fp64, [0] = min,
 *                   [1] = max; pages past the sequence are left untouched.
 *  quest_bounds     U[b,h,p] = sum_d max(q_d * kmin_d, q_d * kmax_d), the largest
 *                   q.k that any key inside the page's min/max box can reach, so an
 *                   upper bound on the score of every token of the page.  (The pages
 *                   give the representation and "most relevant", not the score; this
 *                   is the score that representation plainly supports.)
 *  quest_select     per (b, h), with P = ceil(N_b / 16) pages and m' = min(m_b, P,
 *                   m_max): the last page (the current token's) plus the m' - 1 other
 *                   pages of highest bound, ties to the lower page.  pages_out
 *                   [B][Hq][m_max] ascending then -1; tok_out [B][Hq][16 m_max] the
 *                   tokens j < N_b of those pages ascending, then -1; thr_out [B][Hq]
 *                   the bound of the last page taken by rank (+inf if none was).
 */
void oracle_quest_summaries(const uint16_t *k_cache, const int32_t *page_table, const int32_t *seq_lens,
                            int32_t batch, int32_t num_kv_heads, int32_t max_pages, double *out)
{
    orc_cache c = {k_cache, 0, page_table, seq_lens, batch, num_kv_heads, max_pages};
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bg = 0; bg < (int64_t)batch * num_kv_heads; ++bg) {
        int b = (int)(bg / num_kv_heads), g = (int)(bg % num_kv_heads);
        int64_t n = seq_lens[b], pages = (n + ORC_PAGE - 1) / ORC_PAGE;
        for (int64_t p = 0; p < pages; ++p) {
            double *mn = out + (((int64_t)b * max_pages + p) * num_kv_heads + g) * 2 * ORC_D;
            double *mx = mn + ORC_D;
            for (int d = 0; d < ORC_D; ++d) { mn[d] = INFINITY; mx[d] = -INFINITY; }
            for (int64_t j = p * ORC_PAGE; j < n && j < (p + 1) * ORC_PAGE; ++j) {
                const uint16_t *row = row_of(k_cache, &c, b, g, j);
                for (int d = 0; d < ORC_D; ++d) {
                    double v = bf16_value(row[d]);
                    if (v < mn[d]) mn[d] = v;
                    if (v > mx[d]) mx[d] = v;
                }
            }
        }
    }
}

/* U [B][Hq][max_pages] fp64 from summaries [B][max_pages][Hkv][2][128]; pages past
 * the sequence are left untouched. */
void oracle_quest_bounds(const double *summ, const int32_t *seq_lens, int32_t batch, int32_t num_kv_heads,
                         int32_t max_pages, const uint16_t *q, int32_t num_q_heads, double *u_out)
{
    int32_t G = num_q_heads / num_kv_heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < (int64_t)batch * num_q_heads; ++bh) {
        int b = (int)(bh / num_q_heads), h = (int)(bh % num_q_heads), g = h / G;
        int64_t pages = ((int64_t)seq_lens[b] + ORC_PAGE - 1) / ORC_PAGE;
        const uint16_t *qrow = q + bh * ORC_D;
        for (int64_t p = 0; p < pages; ++p) {
            const double *mn = summ + (((int64_t)b * max_pages + p) * num_kv_heads + g) * 2 * ORC_D;
            const double *mx = mn + ORC_D;
            double u = 0.0;
            for (int d = 0; d < ORC_D; ++d) {
                double qd = bf16_value(qrow[d]);
                double lo = qd * mn[d], hi = qd * mx[d];
                u += lo > hi ? lo : hi;
            }
            u_out[bh * max_pages + p] = u;
        }
    }
}

void oracle_quest_select(const double *u, const int32_t *seq_lens, const int32_t *m_per_seq, int32_t batch,
                         int32_t num_q_heads, int32_t max_pages, int32_t m_max, int32_t *pages_out,
                         int32_t *tok_out, double *thr_out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < (int64_t)batch * num_q_heads; ++bh) {
        int b = (int)(bh / num_q_heads);
        int64_t n = seq_lens[b], P = (n + ORC_PAGE - 1) / ORC_PAGE;
        int64_t m = m_per_seq[b];
        if (m > P) m = P;
        if (m > m_max) m = m_max;
        if (m < 0) m = 0;
        int32_t *prow = pages_out + bh * m_max;
        int64_t taken = 0;
        double thr = INFINITY;
        if (m > 0) {
            prow[taken++] = (int32_t)(P - 1);            /* the current token's page */
            /* the other pages by bound descending, then page ascending */
            scored_token *rest = (scored_token *)malloc((size_t)(P > 1 ? P - 1 : 1) * sizeof *rest);
            for (int64_t p = 0; p < P - 1; ++p) { rest[p].s = u[bh * max_pages + p]; rest[p].j = p; }
            qsort(rest, (size_t)(P - 1), sizeof *rest, by_score_then_index);
            for (int64_t i = 0; i < m - 1; ++i) prow[taken++] = (int32_t)rest[i].j;
            if (m >= 2) thr = rest[m - 2].s;
            free(rest);
        }
        qsort(prow, (size_t)taken, sizeof *prow, by_index);
        for (int64_t i = taken; i < m_max; ++i) prow[i] = -1;
        int32_t *trow = tok_out + bh * (int64_t)m_max * ORC_PAGE;
        int64_t t = 0;
        for (int64_t i = 0; i < taken; ++i)
            for (int64_t j = (int64_t)prow[i] * ORC_PAGE; j < n && j < ((int64_t)prow[i] + 1) * ORC_PAGE; ++j)
                trow[t++] = (int32_t)j;
        for (; t < (int64_t)m_max * ORC_PAGE; ++t) trow[t] = -1;
        if (thr_out) thr_out[bh] = thr;
    }
}

/*
 * Reduced-channel ("label") scores for a lightweight indexer: the paper's Fig. 1a
 * routes the sparse mode through a lightweight indexer that picks the k rows, and
 * the German summary (section 3, indexer overhead) costs one with Double Sparsity;
 * the Sparse Frontier review (section 3.2) describes the same idea as approximate
 * attention scores from a few key dimensions.  With a fixed channel set C_g of R
 * channels per kv head (chosen offline by calibration):
 *     s~[b,h,j] = sum_{i<R} q[b,h,C_g[i]] * K[b,g,j,C_g[i]],   g = h / G,
 * summed over i in the listed order.  The selection is then the exact top-k of s~
 * (oracle_topk) and attention runs on the selected rows in full (oracle_attend).
 * channels: int32 [Hkv][R]; scores_out [B][Hq][n_stride], entries j >= N_b untouched.
 */
void oracle_label_scores(const uint16_t *k_cache, const int32_t *page_table, const int32_t *seq_lens,
                         int32_t batch, int32_t num_kv_heads, int32_t max_pages, const uint16_t *q,
                         int32_t num_q_heads, const int32_t *channels, int32_t r, int64_t n_stride,
                         double *scores_out)
{
    orc_cache c = {k_cache, 0, page_table, seq_lens, batch, num_kv_heads, max_pages};
    int32_t G = num_q_heads / num_kv_heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < (int64_t)batch * num_q_heads; ++bh) {
        int b = (int)(bh / num_q_heads), h = (int)(bh % num_q_heads), g = h / G;
        const int32_t *ch = channels + (int64_t)g * r;     /* this kv head's channel list */
        const uint16_t *qrow = q + bh * ORC_D;
        for (int64_t j = 0; j < seq_lens[b]; ++j) {
            const uint16_t *krow = row_of(k_cache, &c, b, g, j);
            double s = 0.0;
            for (int i = 0; i < r; ++i)
                s += bf16_value(qrow[ch[i]]) * bf16_value(krow[ch[i]]);
            scores_out[bh * n_stride + j] = s;
        }
    }
}

/*
 * Stochastic index selection.  The German summary of the context-sparsity paper
 * (section 2, sparsity mechanisms, and section 3A) evaluates vAttention's stochastic
 * selection, which on smaller models recovers the quality that deterministic top-k
 * loses; the pages do not give its estimator.  The reading taken here is the plain
 * Monte Carlo one: keep the deterministic set S (the valid entries of a top-k row),
 * draw s' tokens uniformly and with replacement from the residual
 * R = {0, ..., N_b - 1} \ S (M = |R| tokens), and let every drawn token stand for
 * M / s' tokens of R, so that (M / s') sum_t f(j_t) estimates sum_{j in R} f(j)
 * without bias.  The random numbers are inputs: draw t of row (b, h) is a 32-bit
 * integer x_t, mapped to the residual rank r_t = floor(x_t M / 2^32) and then to the
 * r_t-th token of R in ascending order.
 *
 * idx [B][Hq][k_max]: the first min(k_b, k_max) entries of a row are read and those
 * in [0, N_b) form S.  draws uint32 [B][Hq][s_max]; s_per_seq [B]; s'_b =
 * min(s_b, s_max), 0 when M = 0.  sample_out [B][Hq][s_max]: the drawn tokens, -1
 * from t = s'_b on.  weight_out [B][Hq]: M / s'_b (0 when nothing is drawn).
 */
void oracle_sample_residual(const int32_t *idx, const int32_t *k_per_seq, int32_t k_max, const int32_t *seq_lens,
                            int32_t batch, int32_t num_q_heads, const uint32_t *draws, const int32_t *s_per_seq,
                            int32_t s_max, int32_t *sample_out, double *weight_out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < (int64_t)batch * num_q_heads; ++bh) {
        int b = (int)(bh / num_q_heads);
        int64_t n = seq_lens[b] > 0 ? seq_lens[b] : 0;
        int64_t kk = k_per_seq[b] < k_max ? k_per_seq[b] : k_max;
        if (kk < 0) kk = 0;
        char *kept = (char *)calloc((size_t)(n > 0 ? n : 1), 1);
        for (int64_t i = 0; i < kk; ++i) {
            int32_t j = idx[bh * k_max + i];
            if (j >= 0 && j < n) kept[j] = 1;
        }
        int32_t *residual = (int32_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof *residual);
        int64_t M = 0;
        for (int64_t j = 0; j < n; ++j)
            if (!kept[j]) residual[M++] = (int32_t)j;
        int64_t s = s_per_seq[b] < s_max ? s_per_seq[b] : s_max;
        if (s < 0 || M == 0) s = 0;
        for (int64_t t = 0; t < s_max; ++t) {
            int32_t tok = -1;
            if (t < s) {
                uint64_t r = ((uint64_t)draws[bh * s_max + t] * (uint64_t)M) >> 32;
                tok = residual[r];
            }
            sample_out[bh * s_max + t] = tok;
        }
        weight_out[bh] = s > 0 ? (double)M / (double)s : 0.0;
        free(residual);
        free(kept);
    }
}

/*
 * The stochastic estimate of the attention output: the kept entries (idx, weight 1)
 * and the drawn ones (sample, weight w_bh each) enter the softmax sums as
 *     o = (sum_S e^{l_j} V_j + w sum_t e^{l_{j_t}} V_{j_t}) / (sum_S e^{l_j} + w sum_t e^{l_{j_t}}),
 * l_j = c s_j as in attend (with the same max subtraction).  Entries < 0 are skipped;
 * a token drawn twice counts twice.  out [B][Hq][128] fp64.
 */
void oracle_attend_sampled(const uint16_t *k_cache, const uint16_t *v_cache, const int32_t *page_table,
                           const int32_t *seq_lens, int32_t batch, int32_t num_kv_heads, int32_t max_pages,
                           const uint16_t *q, int32_t num_q_heads, const int32_t *idx, int32_t k_max,
                           const int32_t *sample, int32_t s_max, const double *weight, double scale, double *out)
{
    orc_cache c = {k_cache, v_cache, page_table, seq_lens, batch, num_kv_heads, max_pages};
    int32_t G = num_q_heads / num_kv_heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < (int64_t)batch * num_q_heads; ++bh) {
        int b = (int)(bh / num_q_heads), g = (int)(bh % num_q_heads) / G;
        const uint16_t *qrow = q + bh * ORC_D;
        int64_t total = (int64_t)k_max + s_max;
        double m = -INFINITY;
        for (int64_t i = 0; i < total; ++i) {
            int32_t j = i < k_max ? idx[bh * k_max + i] : sample[bh * s_max + (i - k_max)];
            if (j < 0) continue;
            double l = scale * dot_q_k(qrow, row_of(c.k, &c, b, g, j));
            if (l > m) m = l;
        }
        double z = 0.0, acc[ORC_D];
        for (int d = 0; d < ORC_D; ++d) acc[d] = 0.0;
        for (int64_t i = 0; i < total; ++i) {
            int32_t j = i < k_max ? idx[bh * k_max + i] : sample[bh * s_max + (i - k_max)];
            if (j < 0) continue;
            double wt = i < k_max ? 1.0 : weight[bh];
            double p = wt * exp(scale * dot_q_k(qrow, row_of(c.k, &c, b, g, j)) - m);
            const uint16_t *vrow = row_of(c.v, &c, b, g, j);
            z += p;
            for (int d = 0; d < ORC_D; ++d)
                acc[d] += p * bf16_value(vrow[d]);
        }
        for (int d = 0; d < ORC_D; ++d)
            out[bh * ORC_D + d] = z > 0.0 ? acc[d] / z : 0.0;
    }
}
