// Exact top-k indexer for the context-sparse decode step (gfx950).
//
// The selection is the exact "oracle top-k" of the context-sparsity paper
// (German technical summary, section 2, sparsity mechanisms): for each
// (sequence, query head) keep the k tokens with the largest raw score q . K_j,
// lower index first on equal scores, per query head (paper section 1).
//
// Three launches on the caller's stream:
//  1. zero_u32_kernel   clears the per-(b, h) first-digit histograms.
//  2. score_kernel      streams every K page once per (b, kv head) and scores it
//                       against the whole GQA group with one bf16 MFMA
//                       (16x16x32: 16 head rows x 16 tokens per page), writes
//                       order-preserving uint32 keys and counts the top 12 key
//                       bits into an LDS histogram flushed with integer atomics.
//  3. select_kernel     per (b, h): finds the threshold key from the histogram
//                       plus two 10-bit radix passes over the keys, then writes
//                       the selected indices in ascending order with one ordered
//                       compaction pass (no sort needed).
#include "sdi_device.hpp"
#include "sdi_launch.hpp"

namespace sdi {

constexpr int kScoreWaves = 4;
constexpr int kScorePagesPerWave = 16;
constexpr int kScoreUnroll = 4;
constexpr int kScoreTokensPerBlock = kScoreWaves * kScorePagesPerWave * kPage;   // 1024

constexpr int kSelThreads = 256;
constexpr int kSelPerThread = 8;
constexpr int kSelTile = kSelThreads * kSelPerThread;                           // 2048

__global__ void zero_u32_kernel(uint32_t *__restrict__ p, int64_t n)
{
    int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    int64_t step = (int64_t)gridDim.x * blockDim.x * 4;
    for (; i + 4 <= n; i += step) *(u32x4 *)(p + i) = u32x4{0u, 0u, 0u, 0u};
    for (; i < n; ++i) p[i] = 0u;
}

// grid (chunks of 1024 tokens, kv_heads * head_blocks, batch); 256 threads.
// Dynamic LDS: min(16, group) * 2048 words (two 16-bit bin counters per word).
__global__ __launch_bounds__(kScoreWaves * 64) void score_kernel(
    const uint16_t *__restrict__ kc, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const uint16_t *__restrict__ q, int num_q_heads, int num_kv_heads,
    int group, int head_blocks, int max_pages, uint32_t *__restrict__ keys, int64_t key_stride,
    uint32_t *__restrict__ ghist)
{
    extern __shared__ uint32_t hist_lds[];
    const int b = blockIdx.z;
    const int g = blockIdx.y / head_blocks, hb = blockIdx.y - g * head_blocks;
    const int n = seq_lens[b];
    const int tok0 = blockIdx.x * kScoreTokensPerBlock;
    if (tok0 >= n) return;                                   // whole block exits together
    const int heads_here = min(16, group - hb * 16);
    const int h0 = g * group + hb * 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, quad = lane >> 4;
    const int words = heads_here * (kHistBins / 2);
    for (int i = threadIdx.x; i < words; i += blockDim.x) hist_lds[i] = 0u;

    // MFMA A operand: row = head (col), k = 32 s + 8 quad .. +7.
    bf16x8 qa[4];
    {
        const bool live = col < heads_here;
        const bf16x8 *qrow =
            (const bf16x8 *)(q + ((int64_t)b * num_q_heads + h0 + (live ? col : 0)) * kHeadDim);
#pragma unroll
        for (int s = 0; s < 4; ++s)
            qa[s] = live ? qrow[4 * s + quad] : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
    __syncthreads();

    const int pages_seq = (n + kPage - 1) / kPage;
    const int p_begin = tok0 / kPage + wave * kScorePagesPerWave;
    const int p_end = min(p_begin + kScorePagesPerWave, pages_seq);
    const int32_t *pt = page_table + (int64_t)b * max_pages;
    uint32_t *keys_h = keys + ((int64_t)b * num_q_heads + h0) * key_stride;
    // MFMA B operand: column = token (row col of the page), k = 32 s + 8 quad .. +7.
    const int lane_off = col * kHeadDim + quad * 8;

    for (int p = p_begin; p < p_end; p += kScoreUnroll) {
        bf16x8 kb[kScoreUnroll][4];
#pragma unroll
        for (int u = 0; u < kScoreUnroll; ++u) {
            if (p + u < p_end) {
                const int64_t phys = pt[p + u];
                const bf16x8 *src =
                    (const bf16x8 *)(kc + (phys * num_kv_heads + g) * (kPage * kHeadDim) + lane_off);
#pragma unroll
                for (int s = 0; s < 4; ++s) kb[u][s] = src[4 * s];
            }
        }
#pragma unroll
        for (int u = 0; u < kScoreUnroll; ++u) {
            if (p + u < p_end) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], kb[u][s], acc, 0, 0, 0);
                const int t = (p + u) * kPage + col;
                if (t < n) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int hm = quad * 4 + i;
                        if (hm < heads_here) {
                            const uint32_t key = score_key(acc[i]);
                            keys_h[hm * key_stride + t] = key;
                            const uint32_t bin = key >> kHistShift;
                            atomicAdd(&hist_lds[hm * (kHistBins / 2) + (bin >> 1)], 1u << ((bin & 1u) * 16u));
                        }
                    }
                }
            }
        }
    }
    __syncthreads();
    uint32_t *gh = ghist + ((int64_t)b * num_q_heads + h0) * kHistBins;
    for (int i = threadIdx.x; i < words; i += blockDim.x) {
        const uint32_t w = hist_lds[i];
        if (w) {
            const int hm = i / (kHistBins / 2);
            const int bin = (i - hm * (kHistBins / 2)) * 2;
            uint32_t *dst = gh + hm * kHistBins + bin;
            if (w & 0xFFFFu) atomicAdd(dst, w & 0xFFFFu);
            if (w >> 16) atomicAdd(dst + 1, w >> 16);
        }
    }
}

// Keys [start, start + 8) clipped to n; returns how many are valid.
__device__ __forceinline__ int load_keys8(const uint32_t *__restrict__ src, int start, int n, uint32_t *v)
{
    if (start + 8 <= n) {
        const u32x4 a = *(const u32x4 *)(src + start);
        const u32x4 c = *(const u32x4 *)(src + start + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
        return 8;
    }
    const int cnt = n > start ? n - start : 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < cnt ? src[start + e] : 0u;
    return cnt;
}

// grid (num_q_heads, batch); 256 threads.
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const uint32_t *__restrict__ keys, int64_t key_stride, const uint32_t *__restrict__ ghist,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ k_per_seq, int num_q_heads, int k_max,
    int32_t *__restrict__ idx_out)
{
    __shared__ uint32_t hist[kHistBins];
    __shared__ uint32_t scratch[kSelThreads / 64 + 2];
    const int h = blockIdx.x, b = blockIdx.y;
    const int64_t bh = (int64_t)b * num_q_heads + h;
    const int n = seq_lens[b];
    int kk = min(min(k_per_seq[b], n), k_max);
    if (kk < 0) kk = 0;
    int32_t *out = idx_out + bh * k_max;
    if (kk == n || kk == 0) {                                // everything, or nothing
        for (int i = threadIdx.x; i < k_max; i += kSelThreads) out[i] = i < kk ? i : -1;
        return;
    }
    const uint32_t *kh = keys + bh * key_stride;

    // Digit 1 (top 12 bits) was counted by the score pass.
    for (int i = threadIdx.x; i < kHistBins; i += kSelThreads) hist[i] = ghist[bh * kHistBins + i];
    if (threadIdx.x == 0) { scratch[kSelThreads / 64] = 0u; scratch[kSelThreads / 64 + 1] = 0u; }
    __syncthreads();
    uint32_t above;
    uint32_t prefix = (uint32_t)threshold_bin<kSelThreads>(hist, kHistBins, (uint32_t)kk, scratch, above);
    uint32_t need = (uint32_t)kk - above;                    // >= 1 keys still to take inside the bin

    // Digits 2 and 3 (10 bits each) among the keys that share the prefix.
    int shift = kHistShift;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
        const int lo = shift - 10;
        for (int i = threadIdx.x; i < 1024; i += kSelThreads) hist[i] = 0u;
        __syncthreads();
        for (int base = 0; base < n; base += kSelTile) {
            uint32_t v[8];
            const int cnt = load_keys8(kh, base + threadIdx.x * kSelPerThread, n, v);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (e < cnt && (v[e] >> shift) == prefix) atomicAdd(&hist[(v[e] >> lo) & 1023u], 1u);
        }
        __syncthreads();
        const uint32_t d = (uint32_t)threshold_bin<kSelThreads>(hist, 1024, need, scratch, above);
        need -= above;
        prefix = (prefix << 10) | d;
        shift = lo;
    }

    // Threshold key T and r = how many keys equal to T to take (lowest indices first).
    const uint32_t T = prefix, r = need;
    uint32_t run_sel = 0, run_eq = 0;
    for (int base = 0; base < n; base += kSelTile) {
        uint32_t v[8];
        const int start = base + threadIdx.x * kSelPerThread;
        const int cnt = load_keys8(kh, start, n, v);
        uint32_t gt = 0, eq = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            gt += (e < cnt && v[e] > T) ? 1u : 0u;
            eq += (e < cnt && v[e] == T) ? 1u : 0u;
        }
        uint32_t tot;
        const uint32_t pre = block_exclusive_scan<kSelThreads>((eq << 16) | gt, scratch, tot);
        const uint32_t eq_left = r > run_eq ? r - run_eq : 0u;
        uint32_t pos = run_sel + (pre & 0xFFFFu) + min(pre >> 16, eq_left);
        uint32_t eq_rank = run_eq + (pre >> 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (e < cnt) {
                bool take = v[e] > T;
                if (v[e] == T) take = (eq_rank++ < r);
                if (take) {
                    if (pos < (uint32_t)kk) out[pos] = start + e;   // never past this row
                    ++pos;
                }
            }
        }
        run_sel += (tot & 0xFFFFu) + min(tot >> 16, eq_left);
        run_eq += tot >> 16;
    }
    for (int i = (int)run_sel + threadIdx.x; i < k_max; i += kSelThreads) out[i] = -1;
}

size_t index_topk_key_stride(int n_max) { return (size_t)((n_max + 63) / 64) * 64; }

size_t index_topk_workspace_bytes(int batch, int num_q_heads, int n_max)
{
    const size_t bh = (size_t)batch * num_q_heads;
    return bh * (index_topk_key_stride(n_max) + kHistBins) * sizeof(uint32_t);
}

hipError_t launch_index_topk(const IndexArgs &a, hipStream_t stream)
{
    const int group = a.num_q_heads / a.num_kv_heads;
    const int head_blocks = (group + 15) / 16;
    const int64_t key_stride = (int64_t)index_topk_key_stride(a.n_max);
    const int64_t bh = (int64_t)a.batch * a.num_q_heads;
    uint32_t *keys = (uint32_t *)a.ws;
    uint32_t *ghist = keys + bh * key_stride;

    const int64_t hist_words = bh * kHistBins;
    const int zblocks = (int)std::min<int64_t>(2048, (hist_words / 4 + 255) / 256 + 1);
    hipLaunchKernelGGL(zero_u32_kernel, dim3(zblocks), dim3(256), 0, stream, ghist, hist_words);

    const int heads_max = std::min(16, group);
    const size_t lds = (size_t)heads_max * (kHistBins / 2) * sizeof(uint32_t);
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)score_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    dim3 sgrid((a.n_max + kScoreTokensPerBlock - 1) / kScoreTokensPerBlock, a.num_kv_heads * head_blocks, a.batch);
    hipLaunchKernelGGL(score_kernel, sgrid, dim3(kScoreWaves * 64), lds, stream, (const uint16_t *)a.k_cache,
                       a.page_table, a.seq_lens, (const uint16_t *)a.q, a.num_q_heads, a.num_kv_heads, group,
                       head_blocks, a.max_pages, keys, key_stride, ghist);

    hipLaunchKernelGGL(select_kernel, dim3(a.num_q_heads, a.batch), dim3(kSelThreads), 0, stream, keys, key_stride,
                       ghist, a.seq_lens, a.k_per_seq, a.num_q_heads, a.k_max, a.idx_out);
    return hipGetLastError();
}

}  // namespace sdi
