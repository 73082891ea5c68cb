// Exact top-k indexer for the context-sparse decode step (gfx950).
//
// The selection is the exact "oracle top-k" of the context-sparsity paper
// (German technical summary, section 2, sparsity mechanisms): for each
// (sequence, query head) keep the k tokens with the largest raw score q . K_j,
// lower index first on equal scores, per query head (paper section 1).
//
// Scores are fp32 sums of bf16 products from one MFMA instruction sequence; a
// score's order-preserving uint32 key is its rank key.  Three launches:
//
//  1. zero_hist_kernel  clears the per-(b, h) 4096-bin histograms.
//  2. score_kernel   streams every K page once per (b, kv head) with contiguous
//                    non-temporal 1 KiB loads, transposes each page through LDS
//                    into the MFMA operand layout, scores 16 tokens x up to 8
//                    heads of the GQA group per 4 MFMAs (16x16x32 bf16), and
//                    writes only the top 16 bits of each key ("code").  Codes are
//                    staged in LDS and written as whole lines: interleaving key
//                    writes with the K stream is what costs bandwidth, and 16-bit
//                    codes halve it.  The top 12 code bits are counted into an LDS
//                    histogram per head, flushed with integer atomics.
//  3. select_kernel  per (b, h): the 12-bit histogram gives the bin b* holding the
//                    k-th key; ONE ordered-compaction pass over the codes lists
//                    the tokens above b* (all selected) and the tokens inside b*
//                    with their codes, in LDS.  A 4-bit histogram of the latter
//                    gives the code c* of the k-th key; the exact keys of the
//                    tokens with code c* are recomputed with the same MFMA sequence
//                    (bit-identical); an 8+8-bit radix on their low halves gives
//                    the exact threshold; the selected part of the bin list is
//                    compacted and merged with the above list into the output.  If
//                    a list outgrows LDS, the head is re-scored to full 32-bit keys
//                    in the workspace and a generic radix select runs over them.
#include "sdi_device.hpp"
#include "sdi_launch.hpp"

namespace sdi {

// ---- score pass --------------------------------------------------------------------------
constexpr int kScoreWaves = 8;
constexpr int kScorePagesPerWave = 32;
constexpr int kScoreUnroll = 2;                               // pages per register buffer
constexpr int kHeadBlock = 8;                                 // query heads scored per workgroup
constexpr int kScoreTokensPerBlock = kScoreWaves * kScorePagesPerWave * kPage;   // 4096
constexpr int kStageRow = kRowBytes + 16;                     // padded LDS row: conflict-free both ways
constexpr int kStagePage = kPage * kStageRow;                 // 4352 B
constexpr int kCodeBlockPages = 8;                            // codes leave LDS every 8 pages (128 tokens)
constexpr int kCodeBlock = kCodeBlockPages * kPage;
static_assert(kScorePagesPerWave % kCodeBlockPages == 0, "code blocks tile a wave's pages");
constexpr int kHistWordsPerHead = kHistBins / 2;              // two 16-bit counters per word

__global__ void zero_hist_kernel(uint32_t *__restrict__ p, int64_t n)
{
    int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    const int64_t step = (int64_t)gridDim.x * blockDim.x * 4;
    for (; i + 4 <= n; i += step) *(u32x4 *)(p + i) = u32x4{0u, 0u, 0u, 0u};
    for (; i < n; ++i) p[i] = 0u;
}

// ---- select ------------------------------------------------------------------------------
constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelCodesPerThread = 32;                        // 64 B of codes per thread per round
constexpr int kSelRound = kSelThreads * kSelCodesPerThread;   // 32768 tokens
constexpr int kSelACap = 8192;                                // tokens above the threshold bin
constexpr int kSelCCap = 4096;                                // tokens in the threshold's 12-bit bin
constexpr int kSelECap = 2048;                                // of those, tokens with the threshold code
constexpr int kSelPerThread = 8;                              // generic path
constexpr int kSelTile = kSelThreads * kSelPerThread;

__device__ __forceinline__ uint32_t code_at(const u32x4 (&w)[4], int e)
{
    const uint32_t word = w[e >> 3][(e >> 1) & 3];
    return (e & 1) ? (word >> 16) : (word & 0xFFFFu);
}

// MFMA B operand for the q rows of a head block: lane (col, quad) holds head col's
// dims 32 s + 8 quad .. +7 (zeros for heads past the block).
__device__ __forceinline__ void load_q_operand(bf16x8 (&qb)[4], const uint16_t *__restrict__ q, int64_t row0,
                                               int heads_here, int col, int quad)
{
    const bool live = col < heads_here;
    const bf16x8 *qrow = (const bf16x8 *)(q + (row0 + (live ? col : 0)) * kHeadDim);
#pragma unroll
    for (int s = 0; s < 4; ++s)
        qb[s] = live ? qrow[4 * s + quad] : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// The score MFMA sequence: D[token 4 quad + i][head col] for 16 tokens (A: row col,
// dims 32 s + 8 quad) and up to 16 heads (B).  Every recomputation uses this same
// function so that keys agree bit for bit.
__device__ __forceinline__ f32x4 score_mfma(const bf16x8 (&ka)[4], const bf16x8 (&qb)[4])
{
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], qb[s], acc, 0, 0, 0);
    return acc;
}

// grid (ceil(n_max / 4096), kv_heads * head_blocks, batch); 512 threads.
__global__ __launch_bounds__(kScoreWaves * 64) void score_kernel(
    const uint16_t *__restrict__ kc, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const uint16_t *__restrict__ q, int num_q_heads, int num_kv_heads,
    int group, int head_blocks, int max_pages, uint16_t *__restrict__ codes, int64_t code_stride,
    uint32_t *__restrict__ ghist)
{
    __shared__ int32_t pt_lds[kScoreWaves * kScorePagesPerWave];
    __shared__ __attribute__((aligned(16))) unsigned char stage_all[kScoreWaves * kScoreUnroll * kStagePage];
    __shared__ __attribute__((aligned(16))) uint16_t code_all[kScoreWaves * kHeadBlock * kCodeBlock];
    __shared__ uint32_t hist_lds[kHeadBlock * kHistWordsPerHead];
    const int b = blockIdx.z;
    const int g = blockIdx.y / head_blocks, hb = blockIdx.y - g * head_blocks;
    const int n = seq_lens[b];
    const int tok0 = blockIdx.x * kScoreTokensPerBlock;
    if (tok0 >= n) return;                                    // whole block exits together
    const int heads_here = min(kHeadBlock, group - hb * kHeadBlock);
    const int h0 = g * group + hb * kHeadBlock;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, quad = lane >> 4;
    unsigned char *stage = stage_all + wave * kScoreUnroll * kStagePage;
    uint16_t *cstage = code_all + wave * kHeadBlock * kCodeBlock;
    for (int i = threadIdx.x; i < heads_here * kHistWordsPerHead; i += blockDim.x) hist_lds[i] = 0u;

    bf16x8 qb[4];
    load_q_operand(qb, q, (int64_t)b * num_q_heads + h0, heads_here, col, quad);

    const int pages_seq = (n + kPage - 1) / kPage;
    const int p_base = tok0 / kPage;                          // first page of this workgroup
    const int p_begin = p_base + wave * kScorePagesPerWave;
    const int p_end = min(p_begin + kScorePagesPerWave, pages_seq);
    {
        const int32_t *pt = page_table + (int64_t)b * max_pages;
        const int i = threadIdx.x;
        if (i < kScoreWaves * kScorePagesPerWave && p_base + i < pages_seq) pt_lds[i] = pt[p_base + i];
    }
    __syncthreads();                                          // page slice staged, histogram cleared

    const uint16_t *k_head = kc + (int64_t)g * kPage * kHeadDim;                 // + phys * Hkv * 4 KiB
    const int64_t page_elems = (int64_t)num_kv_heads * kPage * kHeadDim;
    uint16_t *code_h = codes + ((int64_t)b * num_q_heads + h0) * code_stride;
    // contiguous loads: chunk s (1 KiB) of a page, lane -> row 4 s + lane / 16, dims 8 (lane % 16)
    const int wr_off = (lane >> 4) * kStageRow + (lane & 15) * 16;
    // MFMA A operand: row col, dims 32 s + 8 quad -> bytes 64 s + 16 quad
    const int rd_off = col * kStageRow + quad * 16;

    auto load_group = [&](u32x4 (&kr)[kScoreUnroll][4], int p) {
        int64_t phys[kScoreUnroll];
#pragma unroll
        for (int u = 0; u < kScoreUnroll; ++u) phys[u] = pt_lds[min(p + u, p_end - 1) - p_base];
#pragma unroll
        for (int u = 0; u < kScoreUnroll; ++u) {
            const u32x4 *src = (const u32x4 *)(k_head + phys[u] * page_elems) + lane;
#pragma unroll
            for (int s = 0; s < 4; ++s) kr[u][s] = __builtin_nontemporal_load(src + 64 * s);
        }
    };
    auto score_group = [&](const u32x4 (&kr)[kScoreUnroll][4], int p) {
#pragma unroll
        for (int u = 0; u < kScoreUnroll; ++u)
#pragma unroll
            for (int s = 0; s < 4; ++s) *(u32x4 *)(stage + u * kStagePage + s * 4 * kStageRow + wr_off) = kr[u][s];
#pragma unroll
        for (int u = 0; u < kScoreUnroll; ++u) {
            const int pp = p + u;
            if (pp < p_end) {                                 // wave-uniform
                bf16x8 ka[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) ka[s] = *(const bf16x8 *)(stage + u * kStagePage + s * 64 + rd_off);
                const f32x4 acc = score_mfma(ka, qb);
                // lane holds tokens 4 quad .. +3 of head col: stage their codes
                const uint32_t c0 = score_key(acc[0]) >> 16, c1 = score_key(acc[1]) >> 16;
                const uint32_t c2 = score_key(acc[2]) >> 16, c3 = score_key(acc[3]) >> 16;
                const int slot = (pp - p_begin) & (kCodeBlockPages - 1);
                if (col < heads_here) {
                    *(uint2 *)(cstage + col * kCodeBlock + slot * kPage + 4 * quad) =
                        uint2{c0 | (c1 << 16), c2 | (c3 << 16)};
                    const int t0 = pp * kPage + 4 * quad;
                    uint32_t *hrow = hist_lds + col * kHistWordsPerHead;
                    const uint32_t cs[4] = {c0, c1, c2, c3};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t bin = cs[i] >> 4;             // top 12 key bits
                        if (t0 + i < n) atomicAdd(&hrow[bin >> 1], 1u << ((bin & 1u) * 16u));
                    }
                }
                if (slot == kCodeBlockPages - 1 || pp == p_end - 1) {
                    // flush: lane -> head (lane / 16) + 4 j, 8 tokens (16 B) at 8 (lane % 16)
                    const int tb = (pp - slot) * kPage;
                    const int tt = 8 * (lane & 15);
                    for (int hh = lane >> 4; hh < heads_here; hh += 4) {
                        const u32x4 v = *(const u32x4 *)(cstage + hh * kCodeBlock + tt);
                        uint16_t *dst = code_h + hh * code_stride + tb + tt;
                        if (tb + tt + 8 <= n) {
                            *(u32x4 *)dst = v;
                        } else {
                            for (int e = 0; e < 8; ++e)
                                if (tb + tt + e < n) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
                        }
                    }
                }
            }
        }
    };

    if (p_begin < p_end) {                                    // wave-uniform
        u32x4 ka[kScoreUnroll][4], kb[kScoreUnroll][4];
        load_group(ka, p_begin);
        for (int p = p_begin; p < p_end; p += 2 * kScoreUnroll) {
            load_group(kb, p + kScoreUnroll);
            score_group(ka, p);
            load_group(ka, p + 2 * kScoreUnroll);
            score_group(kb, p + kScoreUnroll);
        }
    }
    __syncthreads();
    uint32_t *gh = ghist + ((int64_t)b * num_q_heads + h0) * kHistBins;
    for (int i = threadIdx.x; i < heads_here * kHistWordsPerHead; i += blockDim.x) {
        const uint32_t wv = hist_lds[i];
        if (wv) {
            const int hm = i / kHistWordsPerHead;
            uint32_t *dst = gh + hm * kHistBins + (i - hm * kHistWordsPerHead) * 2;
            if (wv & 0xFFFFu) atomicAdd(dst, wv & 0xFFFFu);
            if (wv >> 16) atomicAdd(dst + 1, wv >> 16);
        }
    }
}

// ---- select helpers ----------------------------------------------------------------------

// Largest bin B of hist[0..nbins) (nbins = 64 * per, per <= 64) with
// sum_{bins >= B} >= need, found by one wave in two parallel levels: lane l sums
// bins top - l*per ... (from the highest bins down), a wave scan locates the lane
// group holding the crossing, and a second scan over that group's `per` bins
// locates the bin.  Every lane of the calling wave gets bin and above (the count
// over bins > B).  Returns false (outputs untouched) if the total is below need.
__device__ __forceinline__ bool wave_threshold(const uint32_t *hist, int nbins, uint32_t need, uint32_t &bin,
                                               uint32_t &above)
{
    const int lane = threadIdx.x & 63, per = nbins / 64;
    const int top = nbins - 1 - lane * per;
    uint32_t mine = 0;
    for (int i = 0; i < per; ++i) mine += hist[top - i];
    const uint32_t x = wave_inclusive_scan(mine);
    const uint64_t cross = __ballot(x >= need);
    if (cross == 0) return false;
    const int L = __ffsll((unsigned long long)cross) - 1;
    const uint32_t before = __shfl(x - mine, L, 64);
    const int top_l = nbins - 1 - L * per;
    const uint32_t c = lane < per ? hist[top_l - lane] : 0u;
    const uint32_t y = before + wave_inclusive_scan(c);
    const uint64_t cross2 = __ballot(lane < per && y >= need);
    const int I = __ffsll((unsigned long long)cross2) - 1;
    bin = (uint32_t)(top_l - I);
    above = __shfl(y - c, I, 64);
    return true;
}

// Workgroup form: wave 0 searches, res[0] = bin, res[1] = above; ends with a barrier.
__device__ __forceinline__ void threshold_bin_wave(const uint32_t *hist, int nbins, uint32_t need, uint32_t *res)
{
    if (threadIdx.x < 64) {
        uint32_t bin, above;
        if (wave_threshold(hist, nbins, need, bin, above) && threadIdx.x == 0) { res[0] = bin; res[1] = above; }
    }
    __syncthreads();
}

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Number of entries of the ascending list a[0..len) that are < x.
__device__ __forceinline__ int count_below(const uint32_t *a, int len, uint32_t x)
{
    int lo = 0, hi = len;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// Codes [start, start + 32) of a row into four 16-byte words (zeros past n).
__device__ __forceinline__ int load_codes(const uint16_t *__restrict__ row, int start, int n, u32x4 (&w)[4])
{
    if (start + kSelCodesPerThread <= n) {
        const u32x4 *src = (const u32x4 *)(row + start);
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = src[i];
        return kSelCodesPerThread;
    }
    const int cnt = n > start ? n - start : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e0 = 8 * i + 2 * j;
            const uint32_t lo = e0 < cnt ? row[start + e0] : 0u;
            const uint32_t hi = e0 + 1 < cnt ? row[start + e0 + 1] : 0u;
            x[j] = lo | (hi << 16);
        }
        w[i] = u32x4{x[0], x[1], x[2], x[3]};
    }
    return cnt;
}

// Keys [start, start + 8) of a 32-bit key row, clipped to n.
__device__ __forceinline__ int load_keys8(const uint32_t *__restrict__ src, int start, int n, uint32_t (&v)[8])
{
    if (start + 8 <= n) {
        const u32x4 a = *(const u32x4 *)(src + start), c = *(const u32x4 *)(src + start + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
        return 8;
    }
    const int cnt = n > start ? n - start : 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < cnt ? src[start + e] : 0u;
    return cnt;
}

// Exact 32-bit keys of up to 16 tokens of one head block: the 16 K rows (cache row
// number per lane `col`, or -1) as the MFMA A operand, the block's q as B.  Lanes
// with col == head-in-block return the scores of tokens 4 quad .. +3.
__device__ __forceinline__ f32x4 rescore16(const uint16_t *__restrict__ kc, int row, const bf16x8 (&qb)[4],
                                          int quad)
{
    bf16x8 ka[4];
    const bf16x8 *src = (const bf16x8 *)(kc + (int64_t)(row < 0 ? 0 : row) * kHeadDim);
#pragma unroll
    for (int s = 0; s < 4; ++s)
        ka[s] = row >= 0 ? src[4 * s + quad] : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    return score_mfma(ka, qb);
}

// Generic select over full 32-bit keys in memory: 12 + 10 + 10-bit radix passes,
// then one ordered-compaction pass writes the selection.
__device__ __forceinline__ void select_generic(const uint32_t *__restrict__ kh, int n, int kk, int k_max, uint32_t *hist,
                               uint32_t *scratch, uint32_t *res, int32_t *__restrict__ out)
{
    uint32_t prefix = 0, need = (uint32_t)kk;
    int shift = 32;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int w = pass == 0 ? 12 : 10, lo = shift - w, nb = 1 << w;
        for (int i = threadIdx.x; i < nb; i += kSelThreads) hist[i] = 0u;
        if (threadIdx.x == 0) { res[0] = 0u; res[1] = 0u; }
        __syncthreads();
        for (int base = 0; base < n; base += kSelTile) {
            uint32_t v[8];
            const int cnt = load_keys8(kh, base + threadIdx.x * kSelPerThread, n, v);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (e < cnt && (shift == 32 || (v[e] >> shift) == prefix))
                    atomicAdd(&hist[(v[e] >> lo) & (uint32_t)(nb - 1)], 1u);
        }
        __syncthreads();
        threshold_bin_wave(hist, nb, need, res);
        need -= res[1];
        prefix = (shift == 32 ? 0u : (prefix << w)) | res[0];
        shift = lo;
        __syncthreads();                                     // res consumed before its next write
    }
    const uint32_t T = prefix, r = need;                     // take keys > T and the first r keys == T
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
                    if (pos < (uint32_t)kk) out[pos] = start + e;
                    ++pos;
                }
            }
        }
        run_sel += (tot & 0xFFFFu) + min(tot >> 16, eq_left);
        run_eq += tot >> 16;
    }
    for (int i = (int)run_sel + threadIdx.x; i < k_max; i += kSelThreads) out[i] = -1;
}

struct SelectArgs {
    const uint16_t *kc;
    const int32_t *page_table, *seq_lens, *k_per_seq;
    const uint16_t *q;
    const uint16_t *codes;
    const uint32_t *ghist;                                    // 4096-bin histogram of the top 12 code bits
    uint32_t *keys32;                                         // generic-path scratch, one row per (b, h)
    int64_t stride;
    int num_q_heads, num_kv_heads, group, max_pages, k_max;
    int32_t *idx_out;
};

// Generic path for one head: re-score every token to its full 32-bit key in the
// workspace row, then radix-select over the keys.  Called by the whole workgroup.
__device__ __forceinline__ void select_rescore_generic(const SelectArgs &a, int64_t bh, int b, int g, int hb, int hn,
                                       int heads_here, int n, int kk, uint32_t *hist, uint32_t *scratch,
                                       uint32_t *res, int32_t *__restrict__ out)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, quad = lane >> 4;
    uint32_t *krow = a.keys32 + bh * a.stride;
    const int32_t *pt = a.page_table + (int64_t)b * a.max_pages;
    bf16x8 qb[4];
    load_q_operand(qb, a.q, (int64_t)b * a.num_q_heads + g * a.group + hb * kHeadBlock, heads_here, col, quad);
    for (int t0 = wave * 16; t0 < n; t0 += kSelWaves * 16) {
        const int tok = t0 + col;
        const int row = tok < n ? (pt[tok >> 4] * a.num_kv_heads + g) * kPage + (tok & 15) : -1;
        const f32x4 acc = rescore16(a.kc, row, qb, quad);
        if (col == hn) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (t0 + 4 * quad + i < n) krow[t0 + 4 * quad + i] = score_key(acc[i]);
        }
    }
    __threadfence_block();
    __syncthreads();
    select_generic(krow, n, kk, a.k_max, hist, scratch, res, out);
}

// grid (num_q_heads, batch); kSelThreads threads.
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a)
{
    __shared__ uint32_t whist[kHistBins];                     // digit-1 histogram, then scratch lists
    __shared__ uint32_t A[kSelACap];                          // tokens above the threshold bin
    __shared__ uint32_t Ci[kSelCCap];                         // tokens inside the bin (compacted in place later)
    __shared__ uint16_t Cc[kSelCCap];                         // their codes
    __shared__ uint32_t hist16[16];
    __shared__ uint32_t scratch[kSelWaves + 2];
    __shared__ uint32_t res[8];
    uint32_t *Ek = whist;                                     // exact keys of the tokens with code c* (kSelECap)
    uint16_t *Ep = (uint16_t *)(whist + kSelECap);            // their positions in C (kSelECap)
    uint32_t *hist3 = whist + kSelECap + kSelECap / 2;        // 256
    uint32_t *hist4 = hist3 + 256;                            // 256

    const int h = blockIdx.x, b = blockIdx.y;
    const int64_t bh = (int64_t)b * a.num_q_heads + h;
    const int n = a.seq_lens[b];
    int kk = min(min(a.k_per_seq[b], n), a.k_max);
    if (kk < 0) kk = 0;
    int32_t *out = a.idx_out + bh * a.k_max;
    if (kk == n || kk == 0) {                                 // everything, or nothing
        for (int i = threadIdx.x; i < a.k_max; i += kSelThreads) out[i] = i < kk ? i : -1;
        return;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, quad = lane >> 4;
    const int g = h / a.group, hl = h - g * a.group, hb = hl / kHeadBlock, hn = hl - hb * kHeadBlock;
    const int heads_here = min(kHeadBlock, a.group - hb * kHeadBlock);
    const int32_t *pt = a.page_table + (int64_t)b * a.max_pages;
    const uint16_t *crow = a.codes + bh * a.stride;
    const int rounds = (n + kSelRound - 1) / kSelRound;

    u32x4 w[4];
    int cnt = load_codes(crow, threadIdx.x * kSelCodesPerThread, n, w);
    for (int i = threadIdx.x; i < kHistBins; i += kSelThreads) whist[i] = a.ghist[bh * kHistBins + i];
    if (threadIdx.x < 16) hist16[threadIdx.x] = 0u;
    if (threadIdx.x < 8) res[threadIdx.x] = 0u;
    __syncthreads();
    // 1. the 12-bit bin b* holding the k-th key (histogram from the score pass)
    threshold_bin_wave(whist, kHistBins, (uint32_t)kk, res);
    const uint32_t bstar = res[0], above = res[1];
    const uint32_t in_bin = whist[bstar];
    if (above > (uint32_t)kSelACap || in_bin > (uint32_t)kSelCCap) {
        __syncthreads();                                      // everyone has read res and whist[b*]
        select_rescore_generic(a, bh, b, g, hb, hn, heads_here, n, kk, whist, scratch, res, out);
        return;
    }

    // 2. one pass: A = tokens above b*, C = tokens inside b* (+ their codes and a 4-bit histogram)
    uint32_t run_a = 0, run_c = 0;
    for (int r = 0; r < rounds; ++r) {
        const int start = r * kSelRound + threadIdx.x * kSelCodesPerThread;
        u32x4 wn[4];
        int cnt_n = 0;
        if (r + 1 < rounds) cnt_n = load_codes(crow, start + kSelRound, n, wn);   // next round in flight
        uint32_t ma = 0, mc = 0;
        uint32_t nib[4] = {0u, 0u, 0u, 0u};                   // low 4 code bits, 8 tokens per word
#pragma unroll
        for (int e = 0; e < kSelCodesPerThread; ++e) {
            const uint32_t c = code_at(w, e), d = c >> 4;
            ma |= (e < cnt && d > bstar) ? (1u << e) : 0u;
            mc |= (e < cnt && d == bstar) ? (1u << e) : 0u;
            nib[e >> 3] |= (c & 15u) << (4 * (e & 7));
        }
        const uint32_t n0 = nib[0], n1 = nib[1], n2 = nib[2], n3 = nib[3];
        uint32_t tot;
        const uint32_t pre = block_exclusive_scan<kSelThreads>(((uint32_t)__popc(mc) << 16) | (uint32_t)__popc(ma),
                                                               scratch, tot);
        uint32_t pa = run_a + (pre & 0xFFFFu), pc = run_c + (pre >> 16);
        while (ma) {
            const int e = __builtin_ctz(ma);
            ma &= ma - 1u;
            if (pa < (uint32_t)kSelACap) A[pa] = (uint32_t)(start + e);
            ++pa;
        }
        while (mc) {
            const int e = __builtin_ctz(mc);
            mc &= mc - 1u;
            const int q8 = e >> 3;                              // scalars, not an indexed array
            const uint32_t nw = q8 == 0 ? n0 : q8 == 1 ? n1 : q8 == 2 ? n2 : n3;
            const uint32_t c = (bstar << 4) | ((nw >> (4 * (e & 7))) & 15u);
            if (pc < (uint32_t)kSelCCap) { Ci[pc] = (uint32_t)(start + e); Cc[pc] = (uint16_t)c; }
            ++pc;
            atomicAdd(&hist16[c & 15u], 1u);
        }
        run_a += tot & 0xFFFFu;
        run_c += tot >> 16;
        if (r + 1 < rounds) {
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = wn[i];
            cnt = cnt_n;
        }
    }
    __syncthreads();
    const int na_tot = (int)min(run_a, (uint32_t)kSelACap);
    const int m = (int)min(run_c, (uint32_t)kSelCCap);

    // 3. wave 0: the code c* of the k-th key (4-bit digit), then the list E of bin
    //    entries with code c*, in order.
    if (threadIdx.x < 64) {
        const uint32_t need1 = (uint32_t)kk - above;
        uint32_t d2 = 0, ab2 = 0;
        // 16 bins, highest first: lane l < 16 looks at bin 15 - l
        const uint32_t cnt2 = lane < 16 ? hist16[15 - lane] : 0u;
        const uint32_t x = wave_inclusive_scan(cnt2);
        const uint64_t cross = __ballot(lane < 16 && x >= need1);
        if (cross) {
            const int L = __ffsll((unsigned long long)cross) - 1;
            d2 = (uint32_t)(15 - L);
            ab2 = __shfl(x - cnt2, L, 64);
        }
        const uint32_t cstar = (bstar << 4) | d2;
        uint32_t me = 0;
        for (int i0 = 0; i0 < m; i0 += 64) {
            const int i = i0 + lane;
            const bool eq = i < m && Cc[i] == cstar;
            const uint64_t bal = __ballot(eq);
            const uint32_t before = (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
            if (eq && me + before < (uint32_t)kSelECap) Ep[me + before] = (uint16_t)i;
            me += (uint32_t)__popcll(bal);
        }
        if (lane == 0) { res[2] = cstar; res[3] = need1 - ab2; res[4] = me; }
    }
    __syncthreads();
    const uint32_t cstar = res[2];
    uint32_t need = res[3];                                   // >= 1 of the tokens with code c*
    const int me = (int)res[4];
    if (me > kSelECap) {
        __syncthreads();
        select_rescore_generic(a, bh, b, g, hb, hn, heads_here, n, kk, whist, scratch, res, out);
        return;
    }

    // 4. exact keys of E (16 per MFMA group, all waves)
    {
        bf16x8 qb[4];
        load_q_operand(qb, a.q, (int64_t)b * a.num_q_heads + g * a.group + hb * kHeadBlock, heads_here, col, quad);
        for (int c0 = wave * 16; c0 < me; c0 += kSelWaves * 16) {
            int row = -1;
            if (c0 + col < me) {
                const int tok = (int)Ci[Ep[c0 + col]];
                row = (pt[tok >> 4] * a.num_kv_heads + g) * kPage + (tok & 15);
            }
            const f32x4 acc = rescore16(a.kc, row, qb, quad);
            if (col == hn) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (c0 + 4 * quad + i < me) Ek[c0 + 4 * quad + i] = score_key(acc[i]);
            }
        }
    }
    if (threadIdx.x < 512) hist3[threadIdx.x] = 0u;           // hist3 and hist4
    __syncthreads();

    // 5. wave 0: exact threshold among E (key bits 15..8, then 7..0), flags of the
    //    selected E entries, then the selected bin entries compacted in place, in order.
    if (threadIdx.x < 64) {
        for (int i = lane; i < me; i += 64) atomicAdd(&hist3[(Ek[i] >> 8) & 255u], 1u);
        wave_lds_sync();
        uint32_t d3 = 0, ab3 = 0;
        wave_threshold(hist3, 256, need, d3, ab3);
        need -= ab3;
        const uint32_t pref3 = (cstar << 8) | d3;
        for (int i = lane; i < me; i += 64)
            if ((Ek[i] >> 8) == pref3) atomicAdd(&hist4[Ek[i] & 255u], 1u);
        wave_lds_sync();
        uint32_t d4 = 0, ab4 = 0;
        wave_threshold(hist4, 256, need, d4, ab4);
        need -= ab4;
        const uint32_t T = (pref3 << 8) | d4, r = need;
        // flags in E order: key > T, or key == T among the first r
        uint32_t eq_run = 0;
        for (int i0 = 0; i0 < me; i0 += 64) {
            const int i = i0 + lane;
            const uint32_t k = i < me ? Ek[i] : 0u;
            const bool is_eq = i < me && k == T;
            const uint64_t bal = __ballot(is_eq);
            const uint32_t rank = eq_run + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
            if (i < me) Ek[i] = (k > T || (is_eq && rank < r)) ? 1u : 0u;
            eq_run += (uint32_t)__popcll(bal);
        }
        wave_lds_sync();
        // compact C in place: keep code > c*, or code == c* with its E flag set
        uint32_t kept = 0, e_run = 0;
        for (int i0 = 0; i0 < m; i0 += 64) {
            const int i = i0 + lane;
            const uint32_t c = i < m ? Cc[i] : 0u;
            const bool is_eq = i < m && c == cstar;
            const uint64_t beq = __ballot(is_eq);
            const uint32_t eidx = e_run + (uint32_t)__popcll(beq & ((1ull << lane) - 1ull));
            const bool keep = i < m && (c > cstar || (is_eq && Ek[eidx] != 0u));
            const uint64_t bk = __ballot(keep);
            const uint32_t tok = i < m ? Ci[i] : 0u;                 // read before this row is written
            if (keep) Ci[kept + (uint32_t)__popcll(bk & ((1ull << lane) - 1ull))] = tok;
            kept += (uint32_t)__popcll(bk);
            e_run += (uint32_t)__popcll(beq);
        }
        if (lane == 0) res[5] = kept;
    }
    __syncthreads();
    const int ns = (int)res[5];                               // selected bin entries, ascending in Ci

    // 6. merge the two ascending lists into the output row
    for (int i = threadIdx.x; i < na_tot; i += kSelThreads) {
        const uint32_t x = A[i];
        out[i + count_below(Ci, ns, x)] = (int32_t)x;
    }
    for (int j = threadIdx.x; j < ns; j += kSelThreads) {
        const uint32_t x = Ci[j];
        out[j + count_below(A, na_tot, x)] = (int32_t)x;
    }
    for (int i = na_tot + ns + threadIdx.x; i < a.k_max; i += kSelThreads) out[i] = -1;
}

// ---- host side ---------------------------------------------------------------------------

size_t index_topk_key_stride(int n_max) { return (size_t)((n_max + 127) / 128) * 128; }

size_t index_topk_workspace_bytes(int batch, int num_q_heads, int n_max)
{
    // per (b, h): a 32-bit key row for the generic path, the 16-bit codes, the 4096-bin histogram
    return (size_t)batch * num_q_heads *
           (index_topk_key_stride(n_max) * (sizeof(uint32_t) + sizeof(uint16_t)) + kHistBins * sizeof(uint32_t));
}

hipError_t launch_index_topk(const IndexArgs &a, hipStream_t stream)
{
    const int group = a.num_q_heads / a.num_kv_heads;
    const int head_blocks = (group + kHeadBlock - 1) / kHeadBlock;
    const int64_t stride = (int64_t)index_topk_key_stride(a.n_max);
    const size_t rows = (size_t)a.batch * a.num_q_heads;
    uint32_t *keys32 = (uint32_t *)a.ws;
    uint32_t *ghist = keys32 + rows * stride;
    uint16_t *codes = (uint16_t *)(ghist + rows * kHistBins);

    const int64_t hist_words = (int64_t)rows * kHistBins;
    const int zblocks = (int)std::min<int64_t>(1024, (hist_words / 4 + 255) / 256);
    hipLaunchKernelGGL(zero_hist_kernel, dim3(std::max(zblocks, 1)), dim3(256), 0, stream, ghist, hist_words);

    dim3 sgrid((a.n_max + kScoreTokensPerBlock - 1) / kScoreTokensPerBlock, a.num_kv_heads * head_blocks, a.batch);
    hipLaunchKernelGGL(score_kernel, sgrid, dim3(kScoreWaves * 64), 0, stream, (const uint16_t *)a.k_cache,
                       a.page_table, a.seq_lens, (const uint16_t *)a.q, a.num_q_heads, a.num_kv_heads, group,
                       head_blocks, a.max_pages, codes, stride, ghist);

    SelectArgs s{(const uint16_t *)a.k_cache, a.page_table, a.seq_lens, a.k_per_seq, (const uint16_t *)a.q,
                 codes, ghist, keys32, stride, a.num_q_heads, a.num_kv_heads, group, a.max_pages, a.k_max,
                 a.idx_out};
    hipLaunchKernelGGL(select_kernel, dim3(a.num_q_heads, a.batch), dim3(kSelThreads), 0, stream, s);
    return hipGetLastError();
}

}  // namespace sdi
