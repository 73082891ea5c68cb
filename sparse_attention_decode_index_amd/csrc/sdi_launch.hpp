// Host-side launchers of the gfx950 kernels (internal to the library).
// Arguments are already validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace sdi {

struct IndexArgs {
    const void *k_cache;
    const int32_t *page_table, *seq_lens;
    int batch, num_kv_heads, max_pages, n_max;
    const void *q;
    int num_q_heads;
    const int32_t *k_per_seq;
    int k_max;
    int32_t *idx_out;
    void *ws;
};

struct AttendArgs {
    const void *k_cache, *v_cache;
    const int32_t *page_table, *seq_lens;
    int batch, num_kv_heads, max_pages, n_max;
    const void *q;
    int num_q_heads;
    const int32_t *idx;        // NULL for dense
    const int32_t *k_per_seq;  // may be NULL
    int k_max;
    float scale;
    float *out;
    void *ws;
    // two-list mode (stochastic selection): drawn tokens [B][Hq][s_max], weight [B][Hq],
    // draws per sequence [B] (NULL: s_max)
    const int32_t *sample = nullptr;
    const float *sample_weight = nullptr;
    const int32_t *s_per_seq = nullptr;
    int s_max = 0;
};

struct SampleArgs {
    const int32_t *seq_lens;
    int batch, num_q_heads;
    const int32_t *idx, *k_per_seq;   // top-k rows [B][Hq][k_max]
    int k_max;
    const uint32_t *draws;            // [B][Hq][s_max]
    const int32_t *s_per_seq;
    int s_max;
    int32_t *sample_out;              // [B][Hq][s_max]
    float *weight_out;                // [B][Hq]
};

struct QuestArgs {
    const void *k_cache;
    const int32_t *page_table, *seq_lens;
    int batch, num_kv_heads, max_pages, n_max;
    const void *summary;       // [num_pages][Hkv][2][128] bf16 (written by the summary launch)
    const void *q;             // select only
    int num_q_heads;
    const int32_t *pages_per_seq;
    int pages_max;
    int32_t *idx_out;          // [B][Hq][16 pages_max]
    void *ws;
};

struct LabelArgs {
    const void *k_cache;
    const int32_t *page_table, *seq_lens;
    int batch, num_kv_heads, max_pages, n_max;
    const int32_t *channels;   // [Hkv][16] device
    void *labels;              // [num_pages][Hkv][16][16] bf16
    const void *q;             // index only
    int num_q_heads;
    const int32_t *k_per_seq;
    int k_max;
    int32_t *idx_out;
    void *ws;
};

size_t index_topk_key_stride(int n_max);
size_t index_topk_workspace_bytes(int batch, int num_q_heads, int n_max);
hipError_t launch_index_topk(const IndexArgs &a, hipStream_t stream);

int attend_splits(int k_max);
size_t attend_workspace_bytes(int batch, int num_q_heads, int k_max);
hipError_t launch_attend(const AttendArgs &a, hipStream_t stream);
// The allocation-free form of launch_attend: the partials of split rows go to a fixed
// device array (a.ws is ignored).  Returns 0, SDI_ERR_TOO_LARGE or SDI_ERR_HIP.
int launch_attend_noalloc(AttendArgs a, hipStream_t stream);
hipError_t launch_sample(const SampleArgs &a, hipStream_t stream);

hipError_t launch_merge(const float *part_ml, const float *part_acc, int splits, int per_chunk,
                        const int32_t *counts, int count_cap, int batch, int num_q_heads, float *out,
                        hipStream_t stream, const int32_t *counts2 = nullptr, int count_cap2 = 0);

size_t label_bytes(int num_pages, int num_kv_heads);
hipError_t launch_label_build(const LabelArgs &a, int last_only, hipStream_t stream);
hipError_t launch_label_index_topk(const LabelArgs &a, hipStream_t stream);

size_t quest_summary_bytes(int num_pages, int num_kv_heads);
size_t quest_select_workspace_bytes(int batch, int num_q_heads, int max_pages, int pages_max);
hipError_t launch_quest_summary(const QuestArgs &a, int last_only, hipStream_t stream);
hipError_t launch_quest_select(const QuestArgs &a, hipStream_t stream);

int dense_splits(int n_max);
size_t dense_workspace_bytes(int batch, int num_q_heads, int n_max);
hipError_t launch_dense(const AttendArgs &a, hipStream_t stream);

}  // namespace sdi
