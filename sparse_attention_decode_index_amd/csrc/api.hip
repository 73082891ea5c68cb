// C ABI of the context-sparse decode library: argument checks, workspace sizing,
// and the launches of the gfx950 kernels.  Every check runs before anything is
// enqueued, so a call that returns an error has launched nothing.
#include <limits.h>

#include "../../include/sparse_decode.h"
#include "sdi_launch.hpp"

namespace {

int check_kv(const sdi_kv *kv, bool need_v)
{
    if (!kv || !kv->k_cache || !kv->page_table || !kv->seq_lens || (need_v && !kv->v_cache)) return SDI_ERR_NULL;
    if (kv->head_dim != 128 || kv->page_size != 16) return SDI_ERR_SHAPE;
    if (kv->batch < 1 || kv->num_kv_heads < 1 || kv->num_pages < 1 || kv->n_max < 1) return SDI_ERR_SHAPE;
    if (kv->batch > 65535) return SDI_ERR_SHAPE;            // grid z / y limits
    if (kv->max_pages_per_seq < (int32_t)(((int64_t)kv->n_max + 15) / 16)) return SDI_ERR_SHAPE;
    // cache rows are addressed with 32-bit row numbers
    if ((int64_t)kv->num_pages * kv->num_kv_heads * 16 > (int64_t)INT_MAX) return SDI_ERR_SHAPE;
    return SDI_OK;
}

int check_heads(const sdi_kv *kv, int32_t num_q_heads)
{
    if (num_q_heads < 1 || num_q_heads % kv->num_kv_heads != 0) return SDI_ERR_SHAPE;
    if (num_q_heads > 65535) return SDI_ERR_SHAPE;          // grid x / y limits
    if ((int64_t)kv->batch * num_q_heads > (int64_t)INT_MAX / 2) return SDI_ERR_SHAPE;
    return SDI_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SDI_OK : SDI_ERR_HIP; }

}  // namespace

extern "C" {

size_t sparse_decode_index_topk_workspace(const sdi_kv *kv, int32_t num_q_heads, int32_t k_max)
{
    (void)k_max;
    if (!kv || kv->batch < 1 || kv->n_max < 1 || num_q_heads < 1) return 0;
    return sdi::index_topk_workspace_bytes(kv->batch, num_q_heads, kv->n_max);
}

size_t sparse_decode_attend_workspace(const sdi_kv *kv, int32_t num_q_heads, int32_t k_max)
{
    if (!kv || kv->batch < 1 || num_q_heads < 1 || k_max < 1) return 0;
    return sdi::attend_workspace_bytes(kv->batch, num_q_heads, k_max);
}

size_t dense_decode_workspace(const sdi_kv *kv, int32_t num_q_heads)
{
    if (!kv || kv->batch < 1 || kv->n_max < 1 || num_q_heads < 1) return 0;
    return sdi::dense_workspace_bytes(kv->batch, num_q_heads, kv->n_max);
}

int sparse_decode_index_topk(const sdi_kv *kv, const void *q, int32_t num_q_heads, const int32_t *k_per_seq,
                             int32_t k_max, int32_t *idx_out, void *ws, size_t ws_bytes, void *stream)
{
    int rc = check_kv(kv, false);
    if (rc) return rc;
    if (!q || !k_per_seq || !idx_out) return SDI_ERR_NULL;
    if ((rc = check_heads(kv, num_q_heads))) return rc;
    if (k_max < 1) return SDI_ERR_K;
    const size_t need = sparse_decode_index_topk_workspace(kv, num_q_heads, k_max);
    if (need > 0 && !ws) return SDI_ERR_NULL;
    if (ws_bytes < need) return SDI_ERR_WORKSPACE;
    sdi::IndexArgs a{kv->k_cache, kv->page_table, kv->seq_lens, kv->batch, kv->num_kv_heads,
                     kv->max_pages_per_seq, kv->n_max, q, num_q_heads, k_per_seq, k_max, idx_out, ws};
    return hip_status(sdi::launch_index_topk(a, (hipStream_t)stream));
}

int sparse_decode_attend(const sdi_kv *kv, const void *q, int32_t num_q_heads, const int32_t *idx,
                         const int32_t *k_per_seq, int32_t k_max, float softmax_scale, float *out, void *ws,
                         size_t ws_bytes, void *stream)
{
    int rc = check_kv(kv, true);
    if (rc) return rc;
    if (!q || !idx || !out) return SDI_ERR_NULL;
    if ((rc = check_heads(kv, num_q_heads))) return rc;
    if (k_max < 1) return SDI_ERR_K;
    const size_t need = sparse_decode_attend_workspace(kv, num_q_heads, k_max);
    if (need > 0 && !ws) return SDI_ERR_NULL;
    if (ws_bytes < need) return SDI_ERR_WORKSPACE;
    sdi::AttendArgs a{kv->k_cache, kv->v_cache, kv->page_table, kv->seq_lens, kv->batch, kv->num_kv_heads,
                      kv->max_pages_per_seq, kv->n_max, q, num_q_heads, idx, k_per_seq, k_max, softmax_scale,
                      out, ws};
    return hip_status(sdi::launch_attend(a, (hipStream_t)stream));
}

int sparse_decode_attend_noalloc(const sdi_kv *kv, const void *q, int32_t num_q_heads, const int32_t *idx,
                                 const int32_t *k_per_seq, int32_t k_max, float softmax_scale, float *out,
                                 void *stream)
{
    int rc = check_kv(kv, true);
    if (rc) return rc;
    if (!q || !idx || !out) return SDI_ERR_NULL;
    if ((rc = check_heads(kv, num_q_heads))) return rc;
    if (k_max < 1) return SDI_ERR_K;
    sdi::AttendArgs a{kv->k_cache, kv->v_cache, kv->page_table, kv->seq_lens, kv->batch, kv->num_kv_heads,
                      kv->max_pages_per_seq, kv->n_max, q, num_q_heads, idx, k_per_seq, k_max, softmax_scale,
                      out, nullptr};
    return sdi::launch_attend_noalloc(a, (hipStream_t)stream);
}

int dense_decode(const sdi_kv *kv, const void *q, int32_t num_q_heads, float softmax_scale, float *out, void *ws,
                 size_t ws_bytes, void *stream)
{
    int rc = check_kv(kv, true);
    if (rc) return rc;
    if (!q || !out) return SDI_ERR_NULL;
    if ((rc = check_heads(kv, num_q_heads))) return rc;
    const size_t need = dense_decode_workspace(kv, num_q_heads);
    if (need > 0 && !ws) return SDI_ERR_NULL;
    if (ws_bytes < need) return SDI_ERR_WORKSPACE;
    sdi::AttendArgs a{kv->k_cache, kv->v_cache, kv->page_table, kv->seq_lens, kv->batch, kv->num_kv_heads,
                      kv->max_pages_per_seq, kv->n_max, q, num_q_heads, nullptr, nullptr, 0, softmax_scale,
                      out, ws};
    return hip_status(sdi::launch_dense(a, (hipStream_t)stream));
}

int sparse_decode_sample_residual(const sdi_kv *kv, int32_t num_q_heads, const int32_t *idx,
                                  const int32_t *k_per_seq, int32_t k_max, const uint32_t *draws,
                                  const int32_t *s_per_seq, int32_t s_max, int32_t *sample_out, float *weight_out,
                                  void *stream)
{
    int rc = check_kv(kv, false);
    if (rc) return rc;
    if (!idx || !k_per_seq || !draws || !s_per_seq || !sample_out || !weight_out) return SDI_ERR_NULL;
    if ((rc = check_heads(kv, num_q_heads))) return rc;
    if (k_max < 1 || s_max < 1) return SDI_ERR_K;
    sdi::SampleArgs a{kv->seq_lens, kv->batch, num_q_heads, idx, k_per_seq, k_max, draws, s_per_seq, s_max,
                      sample_out, weight_out};
    return hip_status(sdi::launch_sample(a, (hipStream_t)stream));
}

size_t sparse_decode_attend_sampled_workspace(const sdi_kv *kv, int32_t num_q_heads, int32_t k_max, int32_t s_max)
{
    if (!kv || kv->batch < 1 || num_q_heads < 1 || k_max < 1 || s_max < 1 || k_max > INT_MAX - s_max) return 0;
    return sdi::attend_workspace_bytes(kv->batch, num_q_heads, k_max + s_max);
}

int sparse_decode_attend_sampled(const sdi_kv *kv, const void *q, int32_t num_q_heads, const int32_t *idx,
                                 const int32_t *k_per_seq, int32_t k_max, const int32_t *sample,
                                 const float *sample_weight, const int32_t *s_per_seq, int32_t s_max,
                                 float softmax_scale, float *out, void *ws, size_t ws_bytes, void *stream)
{
    int rc = check_kv(kv, true);
    if (rc) return rc;
    if (!q || !idx || !sample || !sample_weight || !out) return SDI_ERR_NULL;
    if ((rc = check_heads(kv, num_q_heads))) return rc;
    if (k_max < 1 || s_max < 1 || k_max > INT_MAX / 2 - s_max) return SDI_ERR_K;
    const size_t need = sparse_decode_attend_sampled_workspace(kv, num_q_heads, k_max, s_max);
    if (need > 0 && !ws) return SDI_ERR_NULL;
    if (ws_bytes < need) return SDI_ERR_WORKSPACE;
    sdi::AttendArgs a{kv->k_cache, kv->v_cache, kv->page_table, kv->seq_lens, kv->batch, kv->num_kv_heads,
                      kv->max_pages_per_seq, kv->n_max, q, num_q_heads, idx, k_per_seq, k_max, softmax_scale,
                      out, ws, sample, sample_weight, s_per_seq, s_max};
    return hip_status(sdi::launch_attend(a, (hipStream_t)stream));
}

size_t sparse_decode_label_bytes(const sdi_kv *kv)
{
    if (!kv || kv->num_pages < 1 || kv->num_kv_heads < 1) return 0;
    return sdi::label_bytes(kv->num_pages, kv->num_kv_heads);
}

int sparse_decode_label_build(const sdi_kv *kv, const int32_t *channels, void *labels, int32_t current_pages_only,
                              void *stream)
{
    int rc = check_kv(kv, false);
    if (rc) return rc;
    if (!channels || !labels) return SDI_ERR_NULL;
    sdi::LabelArgs a{kv->k_cache, kv->page_table, kv->seq_lens, kv->batch, kv->num_kv_heads, kv->max_pages_per_seq,
                     kv->n_max, channels, labels, nullptr, 0, nullptr, 0, nullptr, nullptr};
    return hip_status(sdi::launch_label_build(a, current_pages_only ? 1 : 0, (hipStream_t)stream));
}

int sparse_decode_label_index_topk(const sdi_kv *kv, const void *q, int32_t num_q_heads, const void *labels,
                                   const int32_t *channels, const int32_t *k_per_seq, int32_t k_max,
                                   int32_t *idx_out, void *ws, size_t ws_bytes, void *stream)
{
    int rc = check_kv(kv, false);
    if (rc) return rc;
    if (!q || !labels || !channels || !k_per_seq || !idx_out) return SDI_ERR_NULL;
    if ((rc = check_heads(kv, num_q_heads))) return rc;
    if (k_max < 1) return SDI_ERR_K;
    const size_t need = sparse_decode_index_topk_workspace(kv, num_q_heads, k_max);
    if (need > 0 && !ws) return SDI_ERR_NULL;
    if (ws_bytes < need) return SDI_ERR_WORKSPACE;
    sdi::LabelArgs a{kv->k_cache, kv->page_table, kv->seq_lens, kv->batch, kv->num_kv_heads, kv->max_pages_per_seq,
                     kv->n_max, channels, const_cast<void *>(labels), q, num_q_heads, k_per_seq, k_max, idx_out,
                     ws};
    return hip_status(sdi::launch_label_index_topk(a, (hipStream_t)stream));
}

size_t sparse_decode_quest_summary_bytes(const sdi_kv *kv)
{
    if (!kv || kv->num_pages < 1 || kv->num_kv_heads < 1) return 0;
    return sdi::quest_summary_bytes(kv->num_pages, kv->num_kv_heads);
}

size_t sparse_decode_quest_select_workspace(const sdi_kv *kv, int32_t num_q_heads, int32_t pages_max)
{
    if (!kv || kv->batch < 1 || kv->max_pages_per_seq < 1 || num_q_heads < 1 || pages_max < 1) return 0;
    return sdi::quest_select_workspace_bytes(kv->batch, num_q_heads, kv->max_pages_per_seq, pages_max);
}

int sparse_decode_quest_summarize(const sdi_kv *kv, void *summary, int32_t current_pages_only, void *stream)
{
    int rc = check_kv(kv, false);
    if (rc) return rc;
    if (!summary) return SDI_ERR_NULL;
    sdi::QuestArgs a{kv->k_cache, kv->page_table, kv->seq_lens, kv->batch, kv->num_kv_heads,
                     kv->max_pages_per_seq, kv->n_max, summary, nullptr, 0, nullptr, 0, nullptr, nullptr};
    return hip_status(sdi::launch_quest_summary(a, current_pages_only ? 1 : 0, (hipStream_t)stream));
}

int sparse_decode_quest_select(const sdi_kv *kv, const void *q, int32_t num_q_heads, const void *summary,
                               const int32_t *pages_per_seq, int32_t pages_max, int32_t *idx_out, void *ws,
                               size_t ws_bytes, void *stream)
{
    int rc = check_kv(kv, false);
    if (rc) return rc;
    if (!q || !summary || !pages_per_seq || !idx_out) return SDI_ERR_NULL;
    if ((rc = check_heads(kv, num_q_heads))) return rc;
    if (pages_max < 1 || pages_max > INT_MAX / 16) return SDI_ERR_K;
    const size_t need = sparse_decode_quest_select_workspace(kv, num_q_heads, pages_max);
    if (!ws) return SDI_ERR_NULL;
    if (ws_bytes < need) return SDI_ERR_WORKSPACE;
    sdi::QuestArgs a{kv->k_cache, kv->page_table, kv->seq_lens, kv->batch, kv->num_kv_heads,
                     kv->max_pages_per_seq, kv->n_max, summary, q, num_q_heads, pages_per_seq, pages_max, idx_out,
                     ws};
    return hip_status(sdi::launch_quest_select(a, (hipStream_t)stream));
}

const char *sparse_decode_strerror(int code)
{
    switch (code) {
    case SDI_OK: return "ok";
    case SDI_ERR_NULL: return "a required pointer is NULL";
    case SDI_ERR_SHAPE: return "unsupported shape (head_dim must be 128, page_size 16, q heads a multiple of kv heads, sizes >= 1)";
    case SDI_ERR_K: return "k_max (or pages_max, s_max) must be at least 1";
    case SDI_ERR_WORKSPACE: return "workspace smaller than the size the *_workspace() query returns";
    case SDI_ERR_HIP: return "a HIP kernel launch failed";
    case SDI_ERR_TOO_LARGE: return "the call needs more than the fixed 32 MiB scratch of the allocation-free entry point";
    default: return "unknown sparse_decode status";
    }
}

}  // extern "C"
