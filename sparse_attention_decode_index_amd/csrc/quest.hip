// Quest-style page selection for the decode step (gfx950).
//
// The Sparse Frontier review lists Quest as a decode-time method that selects
// 16-token pages under a uniform budget over the full cache (section 3.5, Table 1),
// represents each page by the elementwise minimum and maximum of its keys and,
// at every step, picks the most relevant pages, always including the page that
// holds the current token (section 7.1); what it loads to choose is the page
// representations (Eq. 10), 2 x 128 values per page and kv head instead of 16 x 128.
// The relevance score is the bound U = sum_d max(q_d min_d, q_d max_d): the largest
// q.k any key inside the page's box can reach.
//
//  1. quest_summary_kernel  per (page, kv head): min and max over the page's cached
//     rows -> summary [num_pages][Hkv][2][128] bf16 (min, then max).  One wave per
//     page: lane (r, c) takes rows r, r + 4, r + 8, r + 12 and dims 8c .. 8c + 7,
//     then the 4 row groups combine by lane shuffles.  Bounds of bf16 values are
//     bf16 values, so the summaries are exact.
//  2. quest_bound_kernel    per (b, kv head, 256 pages): U for the G query heads of
//     the group from the two summary rows (16 lanes x 16 B each), written as
//     order-preserving 32-bit keys, the current page's as the largest key.  A
//     matrix-vector product per head with a per-head choice of row, so it runs on
//     the vector ALU; the read is 512 B per page and kv head.
//  3. quest_select_kernel   per (b, q head): the m highest keys by exact radix
//     selection (lower page first on equal keys), then the selected pages'
//     tokens j < N_b ascending, -1 elsewhere, ready for the gather-attend.
#include "sdi_device.hpp"
#include "sdi_index.hpp"
#include "sdi_launch.hpp"
#include "sdi_radix.hpp"

namespace sdi {

constexpr int kQuestSumRows = 2 * kHeadDim;                   // min row + max row per (page, kv head)
constexpr int kQuestBoundPages = 256;                         // pages per bound workgroup (64 per wave)
constexpr int kQuestHeads = 8;                                // query heads per bound workgroup

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

// grid (ceil(pages / 4), Hkv, B) or (1, Hkv, B) for the current pages only; 256 threads.
__global__ __launch_bounds__(256) void quest_summary_kernel(const uint16_t *__restrict__ kc,
                                                            const int32_t *__restrict__ page_table,
                                                            const int32_t *__restrict__ seq_lens, int num_kv_heads,
                                                            int max_pages, int last_only,
                                                            uint16_t *__restrict__ summary)
{
    const int b = blockIdx.z, g = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = seq_lens[b];
    const int pages = (n + kPage - 1) / kPage;
    const int p = last_only ? (wave == 0 ? pages - 1 : -1) : (int)blockIdx.x * 4 + wave;
    if (p < 0 || p >= pages) return;                          // wave-uniform
    const int64_t phys = page_table[(int64_t)b * max_pages + p];
    const uint16_t *blk = kc + (phys * num_kv_heads + g) * kPage * kHeadDim;
    const int valid = min(kPage, n - p * kPage);
    const int rg = lane >> 4, c = lane & 15;
    float mn[8], mx[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { mn[e] = __builtin_inff(); mx[e] = -__builtin_inff(); }
    u32x4 w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (rg + 4 * i < valid) w[i] = *(const u32x4 *)(blk + (rg + 4 * i) * kHeadDim + 8 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (rg + 4 * i < valid) {
            float f[8];
            unpack8(w[i], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) { mn[e] = fminf(mn[e], f[e]); mx[e] = fmaxf(mx[e], f[e]); }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        mn[e] = fminf(mn[e], __shfl_xor(mn[e], 16, 64));
        mx[e] = fmaxf(mx[e], __shfl_xor(mx[e], 16, 64));
        mn[e] = fminf(mn[e], __shfl_xor(mn[e], 32, 64));
        mx[e] = fmaxf(mx[e], __shfl_xor(mx[e], 32, 64));
    }
    if (rg == 0) {
        uint16_t *out = summary + (phys * num_kv_heads + g) * kQuestSumRows + 8 * c;
        *(u32x4 *)out = u32x4{pack_bf16x2(mn[0], mn[1]), pack_bf16x2(mn[2], mn[3]), pack_bf16x2(mn[4], mn[5]),
                              pack_bf16x2(mn[6], mn[7])};
        *(u32x4 *)(out + kHeadDim) = u32x4{pack_bf16x2(mx[0], mx[1]), pack_bf16x2(mx[2], mx[3]),
                                           pack_bf16x2(mx[4], mx[5]), pack_bf16x2(mx[6], mx[7])};
    }
}

// grid (ceil(max_pages / 256), Hkv * head_blocks, B); 256 threads.  Each wave takes 64
// pages in 4 batches of 16 (the next batch's summary rows in flight while one is
// scored; the page-table entries of all 64 arrive first, in one load); lane group grp
// of a batch takes pages base + 4 i + grp, i = 0..3, and lane c of the group dims
// 8c .. 8c + 7.
__global__ __launch_bounds__(256) void quest_bound_kernel(const uint16_t *__restrict__ summary,
                                                          const int32_t *__restrict__ page_table,
                                                          const int32_t *__restrict__ seq_lens,
                                                          const uint16_t *__restrict__ q, int num_q_heads,
                                                          int num_kv_heads, int group, int head_blocks,
                                                          int max_pages, uint32_t *__restrict__ keys,
                                                          int64_t key_stride)
{
    const int b = blockIdx.z;
    const int g = blockIdx.y / head_blocks, hb = blockIdx.y - g * head_blocks;
    const int heads_here = min(kQuestHeads, group - hb * kQuestHeads);
    const int h0 = g * group + hb * kQuestHeads;
    const int n = seq_lens[b];
    const int pages = (n + kPage - 1) / kPage;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane >> 4, c = lane & 15;
    const int base0 = (int)blockIdx.x * kQuestBoundPages + wave * (kQuestBoundPages / 4);
    if (base0 >= pages) return;                               // wave-uniform
    const int32_t *pt = page_table + (int64_t)b * max_pages;
    // the wave's 64 page-table entries in one load (lane l: page base0 + l, clamped to
    // the row), so that the summary loads of every batch go out without another wait
    const int pt_lane = pt[min(base0 + lane, pages - 1)];

    // summary rows of batch j (pages clamped to the row; those past it are not scored)
    auto load_batch = [&](int j, u32x4 (&smin)[4], u32x4 (&smax)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = min(base0 + 16 * j + 4 * i + grp, pages - 1);
            const int64_t phys = __shfl(pt_lane, p - base0, 64);
            const uint16_t *row = summary + (phys * num_kv_heads + g) * kQuestSumRows + 8 * c;
            smin[i] = *(const u32x4 *)row;
            smax[i] = *(const u32x4 *)(row + kHeadDim);
        }
    };
    u32x4 amin[4], amax[4], bmin[4], bmax[4];
    load_batch(0, amin, amax);
    float qf[kQuestHeads][8];
#pragma unroll
    for (int h = 0; h < kQuestHeads; ++h) {
        u32x4 w = u32x4{0u, 0u, 0u, 0u};
        if (h < heads_here) w = *(const u32x4 *)(q + ((int64_t)b * num_q_heads + h0 + h) * kHeadDim + 8 * c);
        unpack8(w, qf[h]);
    }
    auto score_batch = [&](int j, const u32x4 (&smin)[4], const u32x4 (&smax)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = base0 + 16 * j + 4 * i + grp;
            float lo[8], hi[8];
            unpack8(smin[i], lo);
            unpack8(smax[i], hi);
            float mine = 0.f;                                 // head c's bound (lanes c < heads_here)
#pragma unroll
            for (int h = 0; h < kQuestHeads; ++h) {
                if (h < heads_here) {                        // uniform
                    float part = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) part = fmaf(qf[h][e], qf[h][e] >= 0.f ? hi[e] : lo[e], part);
                    part = row16_sum(part);
                    if (c == h) mine = part;
                }
            }
            if (c < heads_here && p < pages) {
                const uint32_t key = p == pages - 1 ? 0xFFFFFFFFu : score_key(mine);
                keys[((int64_t)b * num_q_heads + h0 + c) * key_stride + p] = key;
            }
        }
    };
    load_batch(1, bmin, bmax);
    score_batch(0, amin, amax);
    load_batch(2, amin, amax);
    score_batch(1, bmin, bmax);
    load_batch(3, bmin, bmax);
    score_batch(2, amin, amax);
    score_batch(3, bmin, bmax);
}

// grid (Hq, B); kThreads threads (512, or 1024 when the rows are fewer than the CUs and
// long).
template <int kThreads>
__global__ __launch_bounds__(kThreads) void quest_select_kernel(const uint32_t *__restrict__ keys,
                                                                   int64_t key_stride,
                                                                   const int32_t *__restrict__ seq_lens,
                                                                   const int32_t *__restrict__ m_per_seq,
                                                                   int num_q_heads, int m_max,
                                                                   int32_t *__restrict__ pages_tmp,
                                                                   int32_t *__restrict__ idx_out)
{
    __shared__ __attribute__((aligned(16))) uint32_t hist[kHistBins];
    __shared__ uint32_t scratch[kThreads / 64 + 2];
    __shared__ uint32_t res[8];
    const int h = blockIdx.x, b = blockIdx.y;
    const int64_t bh = (int64_t)b * num_q_heads + h;
    const int n = seq_lens[b];
    const int pages = (n + kPage - 1) / kPage;
    const int m = max(0, min(min(m_per_seq[b], pages), m_max));
    int32_t *prow = pages_tmp + bh * m_max;
    const bool all = m >= pages;
    if (!all && m > 0) {
        if (threadIdx.x < 8) res[threadIdx.x] = 0u;
        __syncthreads();
        radix_select<kThreads>(RowKeys{keys + bh * key_stride}, pages, m, m_max, 0u, 32, 0u, hist, scratch, res, prow);
        __threadfence_block();
        __syncthreads();                                      // the page list is written
    }
    int32_t *out = idx_out + bh * (int64_t)m_max * kPage;
    for (int e = threadIdx.x; e < m_max * kPage; e += kThreads) {
        const int i = e >> 4, r = e & 15;
        const int p = m == 0 ? -1 : all ? (i < pages ? i : -1) : prow[i];
        out[e] = (p >= 0 && p * kPage + r < n) ? p * kPage + r : -1;
    }
}

// ---- host side ---------------------------------------------------------------------------

size_t quest_summary_bytes(int num_pages, int num_kv_heads)
{
    return (size_t)num_pages * num_kv_heads * kQuestSumRows * sizeof(uint16_t);
}

static int64_t quest_key_stride(int max_pages) { return ((int64_t)max_pages + 63) / 64 * 64; }

size_t quest_select_workspace_bytes(int batch, int num_q_heads, int max_pages, int pages_max)
{
    const size_t rows = (size_t)batch * num_q_heads;
    return rows * ((size_t)quest_key_stride(max_pages) * sizeof(uint32_t) + (size_t)pages_max * sizeof(int32_t));
}

hipError_t launch_quest_summary(const QuestArgs &a, int last_only, hipStream_t stream)
{
    const int bx = last_only ? 1 : (a.max_pages + 3) / 4;
    hipLaunchKernelGGL(quest_summary_kernel, dim3(bx, a.num_kv_heads, a.batch), dim3(256), 0, stream,
                       (const uint16_t *)a.k_cache, a.page_table, a.seq_lens, a.num_kv_heads, a.max_pages,
                       last_only, (uint16_t *)a.summary);
    return hipGetLastError();
}

hipError_t launch_quest_select(const QuestArgs &a, hipStream_t stream)
{
    const int group = a.num_q_heads / a.num_kv_heads;
    const int head_blocks = (group + kQuestHeads - 1) / kQuestHeads;
    const int64_t stride = quest_key_stride(a.max_pages);
    uint32_t *keys = (uint32_t *)a.ws;
    int32_t *pages_tmp = (int32_t *)(keys + (size_t)a.batch * a.num_q_heads * stride);
    const int pages_used = (a.n_max + kPage - 1) / kPage;
    hipLaunchKernelGGL(quest_bound_kernel,
                       dim3((pages_used + kQuestBoundPages - 1) / kQuestBoundPages, a.num_kv_heads * head_blocks,
                            a.batch),
                       dim3(256), 0, stream, (const uint16_t *)a.summary, a.page_table, a.seq_lens,
                       (const uint16_t *)a.q, a.num_q_heads, a.num_kv_heads, group, head_blocks, a.max_pages, keys,
                       stride);
    // Fewer rows than CUs with long page lists: twice the threads per row (as for the
    // token select).
    const dim3 sgrid(a.num_q_heads, a.batch);
    if ((int64_t)a.num_q_heads * a.batch < kCUs && pages_used >= 4096)
        hipLaunchKernelGGL(quest_select_kernel<1024>, sgrid, dim3(1024), 0, stream, keys, stride, a.seq_lens,
                           a.pages_per_seq, a.num_q_heads, a.pages_max, pages_tmp, a.idx_out);
    else
        hipLaunchKernelGGL(quest_select_kernel<kSelThreads>, sgrid, dim3(kSelThreads), 0, stream, keys, stride,
                           a.seq_lens, a.pages_per_seq, a.num_q_heads, a.pages_max, pages_tmp, a.idx_out);
    return hipGetLastError();
}

}  // namespace sdi
