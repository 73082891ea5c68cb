/*
 * sparse_decode.h -- C ABI of the context-sparse decode library (gfx950 / MI355X).
 *
 * What it computes.  One decode step of attention over a paged bf16 KV cache,
 * for every query head of every sequence in a batch:
 *
 *   index   the exact top-k indexer: score every cached key with the raw product
 *           q.K^T and keep the k highest tokens (lower token index first on equal
 *           scores).  This is the "oracle top-k" selection of the context-sparsity
 *           paper (arXiv 2605.24168; German technical summary, section 2,
 *           sparsity mechanisms) and the "lightweight indexer" of its Fig. 1a.
 *   attend  softmax attention over only the selected rows, the sparse decode mode
 *           of Fig. 1a (O(k d) bytes per step instead of O(N d)), with selections
 *           that differ per token, per query and per head under GQA (paper
 *           section 1, "sparsity can serve system gains").
 *   dense   the dense decode mode of Fig. 1a: softmax attention over every cached
 *           token, the reference the sparse mode is measured against.
 * The attention form is scaled dot-product attention, softmax(q K^T / sqrt(d)) V
 * (sparse-attention survey page, section 1.1); the output is o = V^T a with a a
 * distribution over the attended tokens (paper section 2.1, Theorem 1).
 *
 * Memory.  Every pointer argument is a DEVICE pointer owned by the caller, except
 * the sdi_kv struct itself, which is a HOST struct read during the call and never
 * retained.  The library allocates nothing: each call takes a caller-provided
 * device workspace whose size the matching *_workspace() function returns.
 *
 * Streams.  `stream` is a hipStream_t (NULL = the null stream).  Calls only
 * enqueue kernels; results are valid once the stream has reached them.  The
 * library holds no state of its own between calls, so calls on different streams
 * with different workspaces may overlap; two in-flight calls must not share a
 * workspace.
 *
 * Errors.  Every check runs on the host before anything is enqueued; a call that
 * returns an error has enqueued nothing.  SDI_ERR_HIP reports a failed launch.
 * Device-side contents are the caller's contract and are not validated:
 * 1 <= seq_lens[b] <= n_max, page-table entries of the first ceil(seq_lens[b]/16)
 * pages in [0, num_pages), finite cache and query values.
 */
#ifndef SPARSE_DECODE_H
#define SPARSE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define SDI_API __attribute__((visibility("default")))
#else
#define SDI_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum {
    SDI_OK = 0,
    SDI_ERR_NULL = -1,       /* a required pointer is NULL */
    SDI_ERR_SHAPE = -2,      /* head_dim != 128, page_size != 16, heads not a multiple, sizes < 1 ... */
    SDI_ERR_K = -3,          /* k_max < 1 (pages_max < 1 for the page selection, s_max < 1 for draws) */
    SDI_ERR_WORKSPACE = -4,  /* workspace smaller than the *_workspace() size */
    SDI_ERR_HIP = -5,        /* a kernel launch failed */
    SDI_ERR_TOO_LARGE = -6   /* more than the fixed scratch of sparse_decode_attend_noalloc holds */
};

/*
 * The paged KV cache (host struct describing device memory).
 *   k_cache, v_cache  bf16 [num_pages][num_kv_heads][page_size][head_dim]: each
 *                     (page, kv head) block is 16 rows x 256 B = 4 KiB contiguous.
 *   page_table        int32 [batch][max_pages_per_seq]: token j of sequence b is
 *                     row j % 16 of page page_table[b][j / 16].
 *   seq_lens          int32 [batch]: cached tokens N_b of each sequence.
 *   n_max             host copy of max_b N_b (sizes launches and workspaces).
 * head_dim must be 128 and page_size 16.  A contiguous cache is the same layout
 * with an identity page table.
 */
typedef struct sdi_kv {
    const void *k_cache;
    const void *v_cache;
    const int32_t *page_table;
    const int32_t *seq_lens;
    int32_t batch;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t page_size;
    int32_t max_pages_per_seq;
    int32_t num_pages;
    int32_t n_max;
} sdi_kv;

/*
 * Exact top-k indexer (paper Fig. 1a "lightweight indexer"; German summary
 * section 2, exact oracle top-k; per query head, section 1).
 *   q          bf16 [batch][num_q_heads][128]; query head h reads kv head
 *              h / (num_q_heads / num_kv_heads) (contiguous GQA groups).
 *   k_per_seq  int32 [batch]: k_b.  Each (b, h) selects k' = min(k_b, N_b, k_max)
 *              tokens: the k' largest scores s_j = q . K_j (fp32 accumulation of
 *              bf16 products), ties going to the lower index.
 *   idx_out    int32 [batch][num_q_heads][k_max]: the k' indices ascending, then -1.
 *   ws         device workspace of at least sparse_decode_index_topk_workspace() bytes:
 *              per (b, h) a 32-bit key row of roundup(n_max, 128) entries (touched only
 *              by the exact re-scoring fallback and, for k a large share of N, by the
 *              all-keys mode) and a 1280-byte candidate record per 512 cached tokens --
 *              about 2.15 GB for 32 x 64 rows of up to 161 566 tokens.  Any contents on
 *              entry.
 * Reads k_cache only (v_cache may be NULL).
 */
SDI_API int sparse_decode_index_topk(const sdi_kv *kv, const void *q, int32_t num_q_heads,
                             const int32_t *k_per_seq, int32_t k_max, int32_t *idx_out,
                             void *ws, size_t ws_bytes, void *stream);

SDI_API size_t sparse_decode_index_topk_workspace(const sdi_kv *kv, int32_t num_q_heads, int32_t k_max);

/*
 * Sparse gather-attend (paper Fig. 1a sparse mode: only the selected K/V rows
 * are read; survey section 1.1 for the softmax(q K^T * scale) V form).
 *   idx        int32 [batch][num_q_heads][k_max]: token indices per (b, h); entries
 *              < 0 or >= N_b are skipped, so any list of valid indices works, not
 *              only one written by sparse_decode_index_topk.
 *   k_per_seq  int32 [batch] or NULL: only the first min(k_b, k_max) entries of each
 *              row are read (NULL reads all k_max).
 *   softmax_scale  multiplies q . K before the softmax (1/sqrt(128) is standard).
 *   out        fp32 [batch][num_q_heads][128]: sum_j e^{l_j - m} V_j / sum_j e^{l_j - m}
 *              over the listed tokens; a row with no valid index gets 0.
 */
SDI_API int sparse_decode_attend(const sdi_kv *kv, const void *q, int32_t num_q_heads, const int32_t *idx,
                         const int32_t *k_per_seq, int32_t k_max, float softmax_scale, float *out,
                         void *ws, size_t ws_bytes, void *stream);

SDI_API size_t sparse_decode_attend_workspace(const sdi_kv *kv, int32_t num_q_heads, int32_t k_max);

/*
 * sparse_decode_attend without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, checks and result as sparse_decode_attend, minus ws and
 * ws_bytes; it allocates nothing.  Rows longer than 1024 entries are split into chunks
 * whose partial results go to a fixed 32 MiB device array that the library holds on
 * each GPU it runs on until the process ends (rows up to 1024 entries need none).  A
 * call whose partials would not fit -- sparse_decode_attend_workspace() above 32 MiB,
 * i.e. 520 * batch * num_q_heads * ceil(k_max / 256) bytes -- returns SDI_ERR_TOO_LARGE
 * and launches nothing.  The GPU is the stream's (the current device for the null
 * stream); the array's address there is looked up on the first call on that GPU.
 * Every call on a GPU shares that array: calls that overlap on one GPU (on different
 * streams) race.
 */
SDI_API int sparse_decode_attend_noalloc(const sdi_kv *kv, const void *q, int32_t num_q_heads, const int32_t *idx,
                                         const int32_t *k_per_seq, int32_t k_max, float softmax_scale, float *out,
                                         void *stream);

/*
 * Dense decode (paper Fig. 1a dense mode: the whole cache is read every step).
 * Same output as sparse_decode_attend over every token j < N_b.
 */
SDI_API int dense_decode(const sdi_kv *kv, const void *q, int32_t num_q_heads, float softmax_scale,
                 float *out, void *ws, size_t ws_bytes, void *stream);

SDI_API size_t dense_decode_workspace(const sdi_kv *kv, int32_t num_q_heads);

/*
 * Lightweight top-k indexer on reduced-channel "label" rows (the paper's Fig. 1a:
 * the sparse mode routes through a lightweight indexer that picks the k rows; the
 * German summary, section 3, costs such an indexer with Double Sparsity; the Sparse
 * Frontier review, section 3.2: approximate attention scores from a few key
 * dimensions).  Each kv head g has a fixed list of 16 channels C_g (chosen offline by
 * calibration); the indexer ranks tokens by
 *     s~_j = sum_{i<16} q[C_g[i]] * K_j[C_g[i]]
 * (bf16 products, fp32 accumulation in list order) and keeps the k' = min(k_b, N_b,
 * k_max) largest, lower index first on equal scores.  Attention then runs on the
 * selected rows in full (sparse_decode_attend).
 *
 * sparse_decode_label_build gathers those channels of every cached key:
 *   channels  int32 [num_kv_heads][16] device, values in [0, 128) (not validated).
 *   labels    bf16 [num_pages][num_kv_heads][16][16] (16 rows of a page, 16 channels),
 *             sparse_decode_label_bytes() bytes, owned by the caller; pages no sequence
 *             reaches are left untouched.
 *   current_pages_only  nonzero: only each sequence's last page (the one a decode step
 *             appends to), zero: every page.
 * Reads k_cache only.
 *
 * sparse_decode_label_index_topk reads the label rows (32 B per token and kv head,
 * 1/8 of the K rows) instead of the keys:
 *   q, k_per_seq, k_max, idx_out  as for sparse_decode_index_topk.
 *   labels, channels  as written by / given to sparse_decode_label_build.
 *   ws         device workspace of sparse_decode_index_topk_workspace() bytes.
 */
SDI_API size_t sparse_decode_label_bytes(const sdi_kv *kv);

SDI_API int sparse_decode_label_build(const sdi_kv *kv, const int32_t *channels, void *labels,
                                      int32_t current_pages_only, void *stream);

SDI_API int sparse_decode_label_index_topk(const sdi_kv *kv, const void *q, int32_t num_q_heads,
                                           const void *labels, const int32_t *channels, const int32_t *k_per_seq,
                                           int32_t k_max, int32_t *idx_out, void *ws, size_t ws_bytes,
                                           void *stream);

/*
 * Quest-style page selection (the Sparse Frontier review: section 3.5, Table 1 --
 * a decode-time method selecting 16-token pages under a uniform budget over the
 * full cache; section 7.1 -- each page represented by the elementwise minimum and
 * maximum of its keys, the most relevant pages chosen every step, the page holding
 * the current token always included; Eq. 10 -- selection loads the page
 * representations).
 *
 * sparse_decode_quest_summarize writes, for every page p < ceil(N_b / 16) of every
 * sequence and every kv head, the min and the max of each of the 128 dims over the
 * page's cached rows (tokens j < N_b):
 *   summary  bf16 [num_pages][num_kv_heads][2][128] (min row, then max row), indexed
 *            by physical page, sparse_decode_quest_summary_bytes() bytes, owned by
 *            the caller; pages no sequence reaches are left untouched.
 *   current_pages_only  nonzero: only each sequence's last page ceil(N_b / 16) - 1
 *            (the page a decode step appends to), zero: every page.
 * Reads k_cache only.
 *
 * sparse_decode_quest_select scores every page of (b, q head h) with the bound
 * U = sum_d max(q_d min_d, q_d max_d) (fp32 accumulation of bf16 products; the
 * largest q.k any key inside the page's box can reach) and keeps the current page
 * plus the m' - 1 other pages of highest bound, ties to the lower page, where
 * m' = min(pages_per_seq[b], ceil(N_b / 16), pages_max):
 *   q              bf16 [batch][num_q_heads][128], as for the indexer.
 *   summary        as written by sparse_decode_quest_summarize for the same cache.
 *   pages_per_seq  int32 [batch] device: the page budget m_b.
 *   idx_out        int32 [batch][num_q_heads][16 * pages_max]: entry 16 i + r is token
 *                  16 p_i + r of the i-th selected page p_i (ascending), or -1 when
 *                  that token is past N_b or there is no i-th page.  This is an index
 *                  list for sparse_decode_attend with k_max = 16 * pages_max (and
 *                  k_per_seq NULL).
 *   ws             device workspace of sparse_decode_quest_select_workspace() bytes.
 * pages_max < 1 returns SDI_ERR_K.
 */
SDI_API size_t sparse_decode_quest_summary_bytes(const sdi_kv *kv);

SDI_API int sparse_decode_quest_summarize(const sdi_kv *kv, void *summary, int32_t current_pages_only,
                                          void *stream);

SDI_API int sparse_decode_quest_select(const sdi_kv *kv, const void *q, int32_t num_q_heads, const void *summary,
                                       const int32_t *pages_per_seq, int32_t pages_max, int32_t *idx_out,
                                       void *ws, size_t ws_bytes, void *stream);

SDI_API size_t sparse_decode_quest_select_workspace(const sdi_kv *kv, int32_t num_q_heads, int32_t pages_max);

/*
 * Stochastic index selection (the German summary of the context-sparsity paper,
 * sections 2 and 3A: vAttention's stochastic selection recovers on smaller models the
 * quality deterministic top-k loses).  The pages do not give the estimator; this is
 * the plain Monte Carlo reading.  A row keeps its top-k set S; s' tokens are drawn
 * uniformly, with replacement, from the residual R = {0, ..., N_b - 1} \ S (M tokens),
 * and each drawn token stands for w = M / s' tokens of R in the softmax sums:
 *     o = (sum_S e^{l_j} V_j + w sum_t e^{l_{j_t}} V_{j_t}) / (sum_S e^{l_j} + w sum_t e^{l_{j_t}}).
 *
 * sparse_decode_sample_residual maps caller-supplied random numbers to tokens:
 *   idx, k_per_seq, k_max  a top-k list as sparse_decode_index_topk writes it: the
 *             first min(k_b, k_max) entries of a row hold the kept tokens ascending,
 *             then -1 (other row contents are not validated: the drawn tokens then
 *             stay in [0, N_b) but do not follow the rule below).
 *   draws     uint32 [batch][num_q_heads][s_max] device, uniform 32-bit random numbers.
 *   s_per_seq int32 [batch] device: draws per row s_b; s'_b = min(s_b, s_max), and
 *             0 when the residual is empty.
 *   sample_out  int32 [batch][num_q_heads][s_max]: entry t < s'_b is the residual
 *             token of ascending rank floor(draws[t] * M / 2^32); -1 from s'_b on.
 *   weight_out  fp32 [batch][num_q_heads]: M / s'_b (0 when nothing is drawn).
 * No workspace.  k_max < 1 or s_max < 1 returns SDI_ERR_K.
 *
 * sparse_decode_attend_sampled evaluates the estimate above: of row (b, h) it reads
 * the first min(k_b, k_max) entries of idx (weight 1; k_per_seq NULL: all k_max) and
 * the first min(s_b, s_max) entries of sample (weight sample_weight[b][h] each;
 * s_per_seq NULL: all s_max), both as the calls above write them; entries outside
 * [0, N_b) are skipped and a token drawn twice counts twice.  q, softmax_scale, out
 * as for sparse_decode_attend; ws of sparse_decode_attend_sampled_workspace() bytes.
 */
SDI_API int sparse_decode_sample_residual(const sdi_kv *kv, int32_t num_q_heads, const int32_t *idx,
                                          const int32_t *k_per_seq, int32_t k_max, const uint32_t *draws,
                                          const int32_t *s_per_seq, int32_t s_max, int32_t *sample_out,
                                          float *weight_out, void *stream);

SDI_API int sparse_decode_attend_sampled(const sdi_kv *kv, const void *q, int32_t num_q_heads, const int32_t *idx,
                                         const int32_t *k_per_seq, int32_t k_max, const int32_t *sample,
                                         const float *sample_weight, const int32_t *s_per_seq, int32_t s_max,
                                         float softmax_scale, float *out, void *ws, size_t ws_bytes, void *stream);

SDI_API size_t sparse_decode_attend_sampled_workspace(const sdi_kv *kv, int32_t num_q_heads, int32_t k_max,
                                                      int32_t s_max);

/* Static description of a return code (never NULL). */
SDI_API const char *sparse_decode_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_DECODE_H */
